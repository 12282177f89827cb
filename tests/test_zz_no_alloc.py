"""gr_fused_write_read_noalloc (the entry point for callers that cannot
allocate) against gr_fused_write_read with a caller workspace: called through
the C ABI twice in a row on one GPU, the second call with fewer tokens, each
result equal to the workspace call's bit for bit (same kernels, same inputs).
A call whose scratch would exceed the library's static array is refused
before any launch."""
import ctypes

import pytest
import torch

import write_gr_read_amd as gr
from write_gr_read_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WORKSPACE = 4


def noalloc(L, R, y, s_in, p, u, s):
    N, n, d = R.shape
    lay = gr._layer(p, n, d, torch.bfloat16, R.device, 1e-6)
    L.gr_fused_write_read_noalloc.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int64,
                                                                      ctypes.POINTER(gr._Layer)] + [ctypes.c_void_p] * 3
    L.gr_fused_write_read_noalloc.restype = ctypes.c_int
    return L.gr_fused_write_read_noalloc(R.data_ptr(), y.data_ptr(), s_in.data_ptr(), 1, N, ctypes.byref(lay),
                                         u.data_ptr(), s.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("d,r", [(4096, 64), (1024, 32)])
def test_noalloc_matches_workspace_call_twice(d, r):
    L = gr.lib()
    for N, seed in ((5000, 81), (700, 82)):      # the second call smaller than the first
        X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=seed + d, branch_scale=(1.0, 0.5, 2.0, 1.0))
        p = X.params[1].to(DEV)
        y = X.y.to(DEV)
        s_in = torch.rand(N, 4, device=DEV) * 2
        Rw = X.X.to(DEV)
        uw, sw = gr.fused_write_read(Rw, y, s_in, p)              # workspace from the binding
        Rn = X.X.to(DEV)
        un = torch.full((N, d), 7.0, dtype=torch.bfloat16, device=DEV)
        sn = torch.full((N, 4), 7.0, device=DEV)
        assert noalloc(L, Rn, y, s_in, p, un, sn) == 0, L.gr_last_error()
        torch.cuda.synchronize()
        assert torch.equal(Rn, Rw), f"N={N}: state differs"
        assert torch.equal(un, uw), f"N={N}: u differs"
        assert torch.equal(sn, sw), f"N={N}: s differs"


def test_noalloc_refuses_more_than_its_scratch():
    L = gr.lib()
    N, d, r = 1 << 20, 4096, 64                   # ~2 GB of records: far beyond 48 MiB
    p = inputs.make_gr_inputs(1, 4, d, r, "bf16", seed=83).params[1].to(DEV)
    tiny = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    lay = gr._layer(p, 4, d, torch.bfloat16, p.gamma.device, 1e-6)
    L.gr_fused_write_read_noalloc.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int64,
                                                                      ctypes.POINTER(gr._Layer)] + [ctypes.c_void_p] * 3
    st = L.gr_fused_write_read_noalloc(tiny.data_ptr(), tiny.data_ptr(), tiny.data_ptr(), 1, N, ctypes.byref(lay),
                                       tiny.data_ptr(), tiny.data_ptr(), None)
    assert st == WORKSPACE
    assert b"static array" in L.gr_last_error()
