"""GPU parity of the variants on the widened state against the fp64 oracle:
expand ("Paper reading: Qwen3.8 Flash Next", part 2, sec. 6, eq:rcv), the
AltUp-style static read and round-robin write (sec. 1, eq:input, eq:output),
the per-channel write ("Qwen3.8-Flash-Next architecture notes, 06 Residual",
sec. 3) and the collapse (RMSNorm of the branch sum).

Stored states (expand, both writes) are compared bit for bit: each side forms
the value in fp32 (one fp32 add / FMA, or a copy) and rounds it once to the
state dtype.  u and the collapse output use the bf16 / fp32 tolerance rule of
tests/parity.py, with the static read's condition scale sum_i |h_i R_i|.
"""
import numpy as np
import pytest
import torch

import oracle
import write_gr_read_amd as gr
from write_gr_read_amd import inputs
from parity import check, check_exact, sample_tokens, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gr.lib()  # raises if the HIP library is missing: no silent fallback


# (d = 12288: the collapse forms the branch sum twice instead of staging it in LDS)
SHAPES = [(37, 4, 64), (1, 4, 4096), (300, 1, 256), (129, 3, 512), (64, 8, 128), (1000, 4, 2048),
          (5, 2, 12288)]


def tol_dtype(dt):
    return "f32" if dt == "f32" else "bf16"


@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("N,n,d", SHAPES)
def test_variants_shapes(N, n, d, dt):
    V = inputs.make_variant_inputs(N, n, d, dt, seed=N * 7 + n * 3 + d, branch_scale=None)
    X = V.X.to(DEV)
    label = f"{dt}-N{N}-n{n}-d{d}"
    # expand
    R0 = gr.expand(V.e.to(DEV), n, dtype=V.X.dtype)
    check_exact(f"{label} expand", R0, oracle.expand(V.e, n, dt))
    # static read
    u = gr.static_read(X, V.h.to(DEV))
    ou = oracle.static_read(V.X, V.h, dt)
    A = np.abs(to64(V.h)[None, :, None] * to64(V.X)).sum(axis=1)
    check(f"{label} static read", u, ou, tol_dtype(dt))
    # round-robin write, two depths
    for layer in (0, 2 * n + 1):
        Xr = X.clone()
        gr.round_robin_write(Xr, V.y.to(DEV), layer)
        check_exact(f"{label} round-robin write l={layer}", Xr,
                    oracle.round_robin_write(V.X, V.y, layer, dt))
    # per-channel write
    Xp = X.clone()
    gr.write_per_channel(Xp, V.y.to(DEV), V.s.to(DEV))
    check_exact(f"{label} per-channel write", Xp, oracle.write_per_channel(V.X, V.y, V.s, dt))
    # collapse
    out = gr.collapse(X, V.w.to(DEV))
    check(f"{label} collapse", out, oracle.collapse(V.X, V.w, 1e-6, dt), tol_dtype(dt))
    torch.cuda.synchronize()


def test_per_channel_write_with_constant_strengths_is_gr_write():
    """Strengths constant along channels: the per-channel write equals the
    per-branch write (gr_write) bit for bit."""
    V = inputs.make_variant_inputs(200, 4, 512, "bf16", seed=3)
    X = V.X.to(DEV)
    sb = torch.tensor([0.5, 1.25, 2.0, 0.0], device=DEV)
    a = gr.write_per_channel(X.clone(), V.y.to(DEV), sb[:, None].expand(4, 512).contiguous())
    b = gr.write(X.clone(), V.y.to(DEV), sb[None].expand(200, 4).contiguous())
    assert torch.equal(a, b)


def test_round_robin_leaves_other_branches_untouched():
    V = inputs.make_variant_inputs(50, 4, 256, "bf16", seed=5)
    X = V.X.to(DEV)
    Xr = gr.round_robin_write(X.clone(), V.y.to(DEV), 6)
    for i in (0, 1, 3):
        assert torch.equal(Xr[:, i], X[:, i])
    assert not torch.equal(Xr[:, 2], X[:, 2])


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_variants_prefill_size_sampled(dt):
    """The prefill shape (N = 16384, d = 4096, n = 4): whole GPU calls, sampled
    tokens compared with the oracle run on just those tokens."""
    V = inputs.make_variant_inputs(16384, 4, 4096, dt, seed=9, branch_scale=(1.0, 0.5, 2.0, 1.0))
    idx = sample_tokens(16384, 48, seed=9)
    X = V.X.to(DEV)
    R0 = gr.expand(V.e.to(DEV), 4, dtype=V.X.dtype)
    check_exact("expand (sampled)", R0.cpu()[idx], oracle.expand(V.e[idx], 4, dt))
    u = gr.static_read(X, V.h.to(DEV)).cpu()
    A = np.abs(to64(V.h)[None, :, None] * to64(V.X[idx])).sum(axis=1)
    check("static read (sampled)", u[idx], oracle.static_read(V.X[idx], V.h, dt), "bf16")
    Xr = gr.round_robin_write(X.clone(), V.y.to(DEV), 7).cpu()
    check_exact("round-robin write (sampled)", Xr[idx], oracle.round_robin_write(V.X[idx], V.y[idx], 7, dt))
    Xp = gr.write_per_channel(X.clone(), V.y.to(DEV), V.s.to(DEV)).cpu()
    check_exact("per-channel write (sampled)", Xp[idx], oracle.write_per_channel(V.X[idx], V.y[idx], V.s, dt))
    out = gr.collapse(X, V.w.to(DEV)).cpu()
    check("collapse (sampled)", out[idx], oracle.collapse(V.X[idx], V.w, 1e-6, dt), "bf16")
