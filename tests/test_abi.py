"""C-ABI checks that need no GPU: the library loads, exports every function
that include/gr.h declares, and rejects bad arguments on the host before any
HIP call (so none of these tests launches a kernel)."""
import ctypes
import os
import re

import pytest
import torch

import write_gr_read_amd as gr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gr.h")

INVALID, NOT_SUPPORTED, LAUNCH, WORKSPACE = 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gr.library_path()):
        pytest.skip("libgr.so not built")
    return gr.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("gr_read", "gr_write", "gr_fused_write_read", "residual_add_rmsnorm",
              "gr_workspace_size", "gr_status_string", "gr_last_error"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    for f in declared_functions():
        assert hasattr(L, f), f"libgr.so does not export {f}"


def test_status_strings(L):
    assert L.gr_status_string(0) == b"success"
    assert L.gr_status_string(WORKSPACE) == b"workspace too small"
    assert L.gr_status_string(99) == b"unknown status"


FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced here
MISALIGNED = FAKE + 2


def layer(n=4, d=64, r=8, eps=1e-6, gamma=FAKE, wd=FAKE, wu=FAKE, ww=FAKE):
    return gr._Layer(n, d, r, eps, gamma, wd, wu, ww)


def call_read(L, N=4, lay=None, state=FAKE, u=FAKE, s=FAKE, dt=1, ws=None, ws_bytes=0):
    lay = layer() if lay is None else lay
    return L.gr_read(state, dt, N, ctypes.byref(lay), u, s, ws, ws_bytes, None)


def test_zero_tokens_is_a_noop(L):
    assert call_read(L, N=0, state=None, u=None, s=None) == 0
    assert L.gr_write(None, None, None, 1, 0, 4, 64, None) == 0
    assert L.residual_add_rmsnorm(None, None, None, 1e-6, None, 1, 0, 64, None) == 0
    assert L.gr_fused_write_read(None, None, None, 1, 0, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), INVALID),
    (dict(dt=7), INVALID),
    (dict(state=None), INVALID),
    (dict(state=MISALIGNED), INVALID),
    (dict(u=None), INVALID),
    (dict(s=MISALIGNED), INVALID),
    (dict(lay=layer(n=0)), INVALID),
    (dict(lay=layer(n=9)), INVALID),
    (dict(lay=layer(d=0)), INVALID),
    (dict(lay=layer(d=12)), NOT_SUPPORTED),      # bf16 needs d % 8 == 0
    (dict(lay=layer(r=-1)), INVALID),
    (dict(lay=layer(r=513)), INVALID),
    (dict(lay=layer(eps=-1.0)), INVALID),
    (dict(lay=layer(eps=float("nan"))), INVALID),
    (dict(lay=layer(gamma=None)), INVALID),
    (dict(lay=layer(wd=None)), INVALID),
    (dict(lay=layer(wu=MISALIGNED)), INVALID),
    (dict(lay=layer(r=0)), INVALID),             # r == 0 requires no gate weights
    (dict(lay=layer(ww=MISALIGNED)), INVALID),
    (dict(N=1 << 31), NOT_SUPPORTED),
])
def test_read_rejects_bad_arguments(L, kw, code):
    assert call_read(L, **kw) == code
    assert L.gr_last_error() != b""


def test_fp32_width_rule(L):
    assert call_read(L, dt=0, lay=layer(d=6)) == NOT_SUPPORTED


def test_fp8_state_rules(L):
    """fp8 (e4m3) is a state dtype: d must be a multiple of 16; the n = 1
    add+RMSNorm and the tanh stand-in (one dtype for all tensors) refuse it."""
    assert call_read(L, dt=2, lay=layer(d=24)) == NOT_SUPPORTED
    assert L.gr_write(FAKE, FAKE, FAKE, 2, 4, 4, 40, None) == NOT_SUPPORTED
    assert L.residual_add_rmsnorm(FAKE, FAKE, FAKE, 1e-6, FAKE + 16, 2, 4, 64, None) == NOT_SUPPORTED
    assert L.gr_bench_tanh_standin(FAKE, FAKE, 2, 16, None) == NOT_SUPPORTED
    assert L.gr_last_error() != b""
    nbytes = ctypes.c_size_t(1)
    assert L.gr_workspace_size(1, 2, 256, ctypes.byref(layer(d=64)), ctypes.byref(nbytes)) == 0


def test_write_and_addnorm_reject_bad_arguments(L):
    assert L.gr_write(FAKE, FAKE, FAKE, 1, 4, 0, 64, None) == INVALID
    assert L.gr_write(FAKE, FAKE, FAKE, 1, 4, 4, 60, None) == NOT_SUPPORTED
    assert L.gr_write(FAKE, None, FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.residual_add_rmsnorm(FAKE, FAKE, FAKE, -1.0, FAKE, 1, 4, 64, None) == INVALID
    assert L.residual_add_rmsnorm(FAKE, FAKE, FAKE, 1e-6, FAKE, 1, 4, 64, None) == INVALID  # out == x
    assert L.residual_add_rmsnorm(FAKE, FAKE, None, 1e-6, FAKE + 16, 1, 4, 64, None) == INVALID
    assert L.gr_bench_copy(FAKE, FAKE, 17, None) == INVALID


def test_workspace_query_and_check(L):
    lay = layer(n=4, d=4096, r=64)
    nbytes = ctypes.c_size_t(123)
    assert L.gr_workspace_size(0, 1, 16384, ctypes.byref(lay), ctypes.byref(nbytes)) == 0
    assert L.gr_workspace_size(5, 1, 16384, ctypes.byref(lay), ctypes.byref(nbytes)) == INVALID
    assert L.gr_workspace_size(0, 1, 0, ctypes.byref(lay), ctypes.byref(nbytes)) == 0
    assert nbytes.value == 0
    need = ctypes.c_size_t(0)
    L.gr_workspace_size(1, 1, 16384, ctypes.byref(lay), ctypes.byref(need))
    if need.value > 0:
        assert call_read(L, N=16384, lay=lay, ws=FAKE, ws_bytes=need.value - 16) == WORKSPACE


def test_workspace_size_follows_the_write_projection(L):
    """r = 128 with W_write is a wide gate (132 projection rows, no W' planes);
    without W_write it is narrow (128 rows), and with 8 token tiles or more
    (1024 tokens here) its W' hi / lo planes (n x 2 x 128 x d bf16) are part of
    the workspace: the query sizes the call as it will be made."""
    d = 4096
    sizes = {}
    for ww in (FAKE, None):
        nbytes = ctypes.c_size_t(0)
        assert L.gr_workspace_size(1, 1, 1024, ctypes.byref(layer(d=d, r=128, ww=ww)),
                                   ctypes.byref(nbytes)) == 0
        sizes[ww] = nbytes.value
    assert sizes[None] >= 4 * 2 * 128 * d * 2
    assert sizes[FAKE] > 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_launch_failure_is_reported_without_a_gpu(L):
    """With valid arguments but no GPU, the launch itself fails and is mapped
    to GR_ERROR_LAUNCH with the runtime's message (host-forced error path)."""
    st = L.gr_write(FAKE, FAKE + 4096, FAKE + 8192, 1, 4, 4, 64, None)
    assert st == LAUNCH
    assert b"launch failed" in L.gr_last_error()


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gr.residual_add_rmsnorm(x, x.clone(), torch.ones(64, dtype=torch.bfloat16))


def test_variant_calls_reject_bad_arguments(L):
    """expand / static read / round-robin write / per-channel write / collapse:
    host-side checks only (no launch)."""
    for dt in (0, 1, 2):
        assert L.gr_expand(None, None, dt, 0, 4, 64, None) == 0          # N = 0
    assert L.gr_expand(FAKE, FAKE, 1, 4, 0, 64, None) == INVALID          # n < 1
    assert L.gr_expand(FAKE, FAKE, 1, 4, 9, 64, None) == INVALID          # n > 8
    assert L.gr_expand(FAKE, FAKE, 1, 4, 4, 60, None) == NOT_SUPPORTED    # d % 8
    assert L.gr_expand(FAKE, FAKE, 2, 4, 4, 40, None) == NOT_SUPPORTED    # fp8: d % 16
    assert L.gr_expand(FAKE, FAKE, 7, 4, 4, 64, None) == INVALID          # dtype
    assert L.gr_expand(None, FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.gr_static_read(FAKE, MISALIGNED, FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.gr_static_read(FAKE, FAKE, None, 1, 4, 4, 64, None) == INVALID
    assert L.gr_round_robin_write(FAKE, FAKE, -1, 1, 4, 4, 64, None) == INVALID
    assert L.gr_round_robin_write(FAKE, None, 3, 1, 4, 4, 64, None) == INVALID
    assert L.gr_write_per_channel(FAKE, FAKE, None, 1, 4, 4, 64, None) == INVALID
    assert L.gr_write_per_channel(FAKE, FAKE, FAKE, 0, 4, 4, 62, None) == NOT_SUPPORTED
    assert L.gr_collapse(FAKE, FAKE, -1.0, FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.gr_collapse(FAKE, FAKE, float("nan"), FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.gr_collapse(FAKE, None, 1e-6, FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.gr_last_error() != b""


def hc_layer(n=4, d=64, mode=1, iters=20, eps=1e-6, lam=(1.0, 1.0, 1.0), gamma=FAKE, wn=FAKE, wp=FAKE,
             hs=FAKE):
    return gr._HcLayer(n, d, mode, iters, eps, *lam, gamma, wn, wp, hs)


def test_hc_calls_reject_bad_arguments(L):
    """Hyper-Connections / mHC calls: host-side checks only (no launch)."""
    rd = lambda lay, dt=1, N=4, state=FAKE, u=FAKE, c=FAKE: L.gr_hc_read(state, dt, N, ctypes.byref(lay), u, c, None)
    assert L.gr_hc_read(None, 1, 0, None, None, None, None) == 0                     # N = 0
    assert L.gr_hc_write(None, None, None, 1, 0, 4, 64, None) == 0
    assert L.gr_hc_fused_write_read(None, None, None, 1, 0, None, None, None, None) == 0
    assert rd(hc_layer(n=0)) == INVALID
    assert rd(hc_layer(n=9)) == INVALID
    assert rd(hc_layer(mode=2)) == INVALID
    assert rd(hc_layer(iters=-1)) == INVALID
    assert rd(hc_layer(iters=1001)) == INVALID
    assert rd(hc_layer(eps=-1.0)) == INVALID
    assert rd(hc_layer(lam=(1.0, float("inf"), 1.0))) == INVALID
    assert rd(hc_layer(d=60)) == NOT_SUPPORTED                                         # bf16: d % 8
    assert rd(hc_layer(), dt=2) == NOT_SUPPORTED                                       # no fp8 state
    assert rd(hc_layer(), dt=7) == INVALID
    assert rd(hc_layer(wp=None)) == INVALID
    assert rd(hc_layer(hs=MISALIGNED)) == INVALID
    assert rd(hc_layer(), c=None) == INVALID
    assert rd(hc_layer(), N=-1) == INVALID
    assert L.gr_hc_write(FAKE, FAKE, FAKE, 1, 4, 0, 64, None) == INVALID               # n < 1
    assert L.gr_hc_write(FAKE, None, FAKE, 1, 4, 4, 64, None) == INVALID
    assert L.gr_hc_write(FAKE, FAKE, FAKE, 0, 4, 4, 62, None) == NOT_SUPPORTED         # fp32: d % 4
    lay = hc_layer()
    assert L.gr_hc_fused_write_read(FAKE, FAKE, None, 1, 4, ctypes.byref(lay), FAKE, FAKE, None) == INVALID
    assert L.gr_hc_fused_write_read(FAKE, FAKE, FAKE, 1, 4, None, FAKE, FAKE, None) == INVALID
    assert b"gr_hc_fused_write_read" in L.gr_last_error()
