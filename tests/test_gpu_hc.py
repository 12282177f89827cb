"""GPU parity of the Hyper-Connections (HC) and mHC calls against the fp64 oracle
("Paper reading: Qwen3.8 Flash Next", part 2 (Residual), sec. 2, eq:block,
eq:mix, eq:combine; "DepthBench", sec. 2.5, mHC).

Bars (tests/parity.py): u and the coefficient record at the dtype's tolerance
(bf16: 2e-2 * max(|o|, RMS/16) per element and relative L2 <= 4e-3; fp32:
1e-5 * RMS); the written state within one rounding of the exact sum
(check_sum_store).  The read half of a fused call is compared with the
oracle's read of the state the GPU stored, so a one-ulp difference in a
written element is not counted twice.
"""
import numpy as np
import pytest
import torch

import oracle
import write_gr_read_amd as gr
from write_gr_read_amd import inputs
from parity import check, check_sum_store, sample_tokens, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gr.lib()


def orc_read(R, p, dtype):
    return oracle.hc_read(R, p.gamma, p.w_norm, p.w_proj, p.h_static, p.lam, p.mode, p.iters, p.eps, dtype)


def write_terms(R, y, coeff):
    """T = sum_j |H_res_ij R_j| + |H_comb_i y| per written element."""
    R, y, c = to64(R), to64(y), to64(coeff)
    N, n, d = R.shape
    Hc, Hr = c[:, :n], c[:, n:].reshape(N, n, n)
    return np.einsum("tij,tjc->tic", np.abs(Hr), np.abs(R)) + np.abs(Hc)[:, :, None] * np.abs(y)[:, None, :]


def run_case(Xin, label, dt):
    """read (set 0) -> coefficients; write; fused write + read (set 1)."""
    p0, p1 = Xin.params
    n = Xin.n
    X, y = Xin.X.to(DEV), Xin.y.to(DEV)
    # read
    u0, c0 = gr.hc_read(X, p0.to(DEV))
    ou0, oc0 = orc_read(Xin.X, p0, dt)
    check(f"{label} read u", u0, ou0, dt)
    check(f"{label} read coeff", c0, oc0, dt)
    # write with the oracle's coefficients (fp32 values)
    cin = torch.from_numpy(oc0).float()
    Xw = X.clone()
    gr.hc_write(Xw, y, cin.to(DEV))
    oRw = oracle.hc_write(Xin.X, Xin.y, cin, dt)
    check_sum_store(f"{label} write state", Xw, oRw, write_terms(Xin.X, Xin.y, cin), n, dt)
    # fused: the same write, then the next block's read on the stored state
    Xf = X.clone()
    u1, c1 = gr.hc_fused_write_read(Xf, y, cin.to(DEV), p1.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(Xf, Xw), f"{label}: fused state differs from hc_write's"
    ou1, oc1 = orc_read(Xf.cpu(), p1, dt)
    check(f"{label} fused u", u1, ou1, dt)
    check(f"{label} fused coeff", c1, oc1, dt)
    return Xf, u1, c1


FAST = [  # (N, n, d, mode): bf16, n in {1, 2, 4}, d <= 4096 -> the one-pass kernel
    (1, 4, 4096, "mhc"), (37, 4, 4096, "mhc"), (600, 4, 4096, "hc"), (257, 4, 2048, "mhc"),
    (130, 4, 2560, "hc"), (65, 4, 256, "mhc"), (300, 4, 1032, "hc"), (200, 2, 4096, "mhc"),
    (99, 2, 1024, "hc"), (150, 1, 4096, "mhc"), (40, 1, 520, "hc"),
]


@pytest.mark.parametrize("N,n,d,mode", FAST)
def test_hc_fast_shapes(N, n, d, mode):
    """Several tokens per workgroup, ragged chunk counts (d = 2560, 1032, 520:
    threads with one chunk or none past d/8), every branch count of the kernel,
    both operator families, random static terms and lambdas of order 1."""
    Xin = inputs.make_hc_inputs(N, n, d, mode, "bf16", seed=N + 7 * d + n, lam=(0.8, 1.3, 1.1),
                                static="random", w_std=0.05, branch_scale=(1.0, 0.5, 2.0, 1.0)[:n])
    run_case(Xin, f"hc-{mode}-N{N}-n{n}-d{d}", "bf16")


GENERIC = [  # fp32, n outside {1, 2, 4}, d > 4096 -> the generic kernel
    (64, 4, 256, "mhc", "f32"), (64, 4, 256, "hc", "f32"), (50, 3, 512, "mhc", "bf16"),
    (40, 8, 256, "hc", "bf16"), (33, 4, 8192, "mhc", "bf16"), (20, 5, 96, "mhc", "f32"),
]


@pytest.mark.parametrize("N,n,d,mode,dt", GENERIC)
def test_hc_generic_shapes(N, n, d, mode, dt):
    Xin = inputs.make_hc_inputs(N, n, d, mode, dt, seed=3 * N + d + n, lam=(0.9, 1.2, 0.7),
                                static="random", w_std=0.05)
    run_case(Xin, f"hc-generic-{mode}-N{N}-n{n}-d{d}-{dt}", dt)


@pytest.mark.parametrize("mode", ["hc", "mhc"])
def test_hc_fast_equals_generic(mode, monkeypatch):
    """The one-pass kernel and the generic kernel on the same inputs: the written
    state bit for bit (both sum H_comb y then H_res_i0 R_0 .. in fp32 FMAs), u
    and the coefficients within the bf16 tolerance of each other."""
    Xin = inputs.make_hc_inputs(500, 4, 4096, mode, "bf16", seed=41, lam=(0.8, 1.3, 1.1),
                                static="random", w_std=0.05)
    X, y = Xin.X.to(DEV), Xin.y.to(DEV)
    cin = torch.rand(500, 20, device=DEV) + 0.25
    p = Xin.params[1].to(DEV)
    Xa = X.clone()
    ua, ca = gr.hc_fused_write_read(Xa, y, cin, p)
    monkeypatch.setenv("GR_KERNEL_VARIANT", "generic")
    Xb = X.clone()
    ub, cb = gr.hc_fused_write_read(Xb, y, cin, p)
    torch.cuda.synchronize()
    assert torch.equal(Xa, Xb)
    check(f"hc-{mode} fast vs generic u", ua, to64(ub), "bf16")
    check(f"hc-{mode} fast vs generic coeff", ca, to64(cb), "bf16")


@pytest.mark.parametrize("mode", ["hc", "mhc"])
def test_hc_prefill_full_sampled(mode):
    """The prefill shape (N = 16384, d = 4096, n = 4) at full size in the
    launch configuration the benchmark times; 96 sampled tokens compared."""
    Xin = inputs.make_hc_inputs(16384, 4, 4096, mode, "bf16", seed=9000 + (mode == "mhc"),
                                branch_scale=(1.0, 0.5, 2.0, 1.0))
    p0, p1 = Xin.params
    idx = sample_tokens(Xin.N, 96, seed=5)
    X, y = Xin.X.to(DEV), Xin.y.to(DEV)
    _, c0 = gr.hc_read(X, p0.to(DEV))
    c0h = c0.cpu()
    _, oc0 = orc_read(Xin.X[idx], p0, "bf16")
    check(f"hc-{mode}-prefill read coeff (sampled)", c0h[idx], oc0, "bf16")
    u1, c1 = gr.hc_fused_write_read(X, y, c0, p1.to(DEV))
    Xh = X.cpu()
    oRw = oracle.hc_write(Xin.X[idx], Xin.y[idx], c0h[idx], "bf16")
    check_sum_store(f"hc-{mode}-prefill state (sampled)", Xh[idx], oRw,
                    write_terms(Xin.X[idx], Xin.y[idx], c0h[idx]), 4, "bf16")
    ou1, oc1 = orc_read(Xh[idx], p1, "bf16")
    check(f"hc-{mode}-prefill fused u (sampled)", u1.cpu()[idx], ou1, "bf16")
    check(f"hc-{mode}-prefill fused coeff (sampled)", c1.cpu()[idx], oc1, "bf16")


def test_hc_static_identity_is_pre_norm_on_gpu():
    """Static terms e_k, 1, I with W = 0 on equal branches (the Pre-Norm start of
    the paper reading, sec. 2): the written branches equal the library's own
    n = 1 residual add and u equals its RMSNorm output, element for element."""
    N, n, d = 300, 4, 4096
    Xin = inputs.make_hc_inputs(N, n, d, "hc", "bf16", seed=77)
    r = Xin.X[:, 0].contiguous()
    R = r[:, None, :].repeat(1, n, 1).to(DEV)
    p = Xin.params[0]
    p = inputs.HCLayer("hc", p.gamma, p.w_norm, torch.zeros_like(p.w_proj),
                       inputs.hc_static_terms("hc", n, 2), (0.5, 0.5, 0.5)).to(DEV)
    y = Xin.y.to(DEV)
    coeff = torch.cat([torch.ones(n), torch.eye(n).reshape(-1)]).repeat(N, 1).to(DEV)
    u, c = gr.hc_fused_write_read(R, y, coeff, p)
    x = r.to(DEV).clone()
    out = gr.residual_add_rmsnorm(x, y, p.w_norm)
    torch.cuda.synchronize()
    for i in range(n):
        assert torch.equal(R[:, i], x)
    assert torch.equal(c, coeff)
    check("hc pre-norm u vs residual_add_rmsnorm", u, to64(out), "bf16")


def test_hc_deterministic_and_graph_replay():
    """Two calls give identical bytes; a captured call replayed three times (with
    eager work in between) equals the eager call each time."""
    Xin = inputs.make_hc_inputs(900, 4, 4096, "mhc", "bf16", seed=55, lam=(0.8, 1.3, 1.1),
                                static="random", w_std=0.05)
    X0, y = Xin.X.to(DEV), Xin.y.to(DEV)
    cin = torch.rand(900, 20, device=DEV) + 0.25
    p = Xin.params[1].to(DEV)
    outs = []
    for _ in range(2):
        R = X0.clone()
        u, c = gr.hc_fused_write_read(R, y, cin, p)
        torch.cuda.synchronize()
        outs.append((R, u, c))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    Rg, ug, cg = X0.clone(), torch.empty_like(outs[0][1]), torch.empty_like(outs[0][2])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gr.hc_fused_write_read(Rg, y, cin, p, u=ug, coeff=cg)
    for k in range(3):
        Rg.copy_(X0)
        ug.zero_(); cg.zero_()
        gr.hc_fused_write_read(X0.clone(), y, cin, p)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        R1, u1, c1 = outs[0]
        assert torch.equal(Rg, R1) and torch.equal(ug, u1) and torch.equal(cg, c1), f"replay {k}"


def test_hc_empty_and_argument_errors():
    Xin = inputs.make_hc_inputs(4, 4, 256, "mhc", "bf16", seed=1)
    p = Xin.params[0].to(DEV)
    empty = torch.empty((0, 4, 256), dtype=torch.bfloat16, device=DEV)
    u, c = gr.hc_read(empty, p)
    assert u.shape == (0, 256) and c.shape == (0, 20)
    with pytest.raises(gr.GRError):
        bad = inputs.HCLayer("mhc", p.gamma, p.w_norm, p.w_proj, p.h_static, p.lam, iters=-1)
        gr.hc_read(Xin.X.to(DEV), bad)
    with pytest.raises(TypeError):
        gr.hc_read(Xin.X.to(DEV).to(torch.float8_e4m3fn), p)


def test_hc_past_2_to_31_elements():
    """N x n x d above 2^31 elements (131372 x 4 x 4096 bf16, a 4.3 GB state):
    the one-pass kernel's token offsets pass 32 bits.  Tokens on both sides of
    the boundary (token 131072 starts at element 2^31) are compared with the
    oracle, which gets those rows of the same device tensors."""
    N, n, d = 131372, 4, 4096
    P = inputs.make_hc_inputs(1, n, d, "mhc", "bf16", seed=94, lam=(0.8, 1.3, 1.1), static="random",
                              w_std=0.05).params
    X, y = inputs.make_device_state(N, n, d, "bf16", seed=95, device=DEV)
    idx = np.unique(np.concatenate([[0, 1, 65535, 131070, 131071, 131072, 131073, N - 2, N - 1],
                                    sample_tokens(N, 24, seed=96)]))
    ti = torch.from_numpy(idx).to(DEV)
    Xs = X[ti].cpu()
    _, c0 = gr.hc_read(X, P[0].to(DEV))
    _, oc0 = orc_read(Xs, P[0], "bf16")
    check("hc 2^31 read coeff (sampled)", c0[ti].cpu(), oc0, "bf16")
    cs = c0[ti].cpu()
    u1, c1 = gr.hc_fused_write_read(X, y, c0, P[1].to(DEV))
    Xw = X[ti].cpu()
    oRw = oracle.hc_write(Xs, y[ti].cpu(), cs, "bf16")
    check_sum_store("hc 2^31 fused state (sampled)", Xw, oRw, write_terms(Xs, y[ti].cpu(), cs), n, "bf16")
    ou1, oc1 = orc_read(Xw, P[1], "bf16")
    check("hc 2^31 fused u (sampled)", u1[ti].cpu(), ou1, "bf16")
    check("hc 2^31 fused coeff (sampled)", c1[ti].cpu(), oc1, "bf16")
    del X, y, u1, c0, c1
    torch.cuda.empty_cache()


def test_hc_two_streams():
    """Calls queued on two streams at once (the HC kernels share no library
    memory): every result equals the same call made alone."""
    A = inputs.make_hc_inputs(700, 4, 4096, "mhc", "bf16", seed=81, static="random", w_std=0.05)
    B = inputs.make_hc_inputs(300, 2, 2048, "hc", "bf16", seed=82, static="random", w_std=0.05)
    cins = [torch.rand(700, 20) + 0.25, torch.rand(300, 6) + 0.25]
    alone = []
    for Xin, cin in zip((A, B), cins):
        R = Xin.X.to(DEV)
        u, c = gr.hc_fused_write_read(R, Xin.y.to(DEV), cin.to(DEV), Xin.params[1].to(DEV))
        torch.cuda.synchronize()
        alone.append((R, u, c))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for Xin, cin, st in zip((A, B), cins, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            p, y, ci = Xin.params[1].to(DEV), Xin.y.to(DEV), cin.to(DEV)
            for _ in range(3):
                R = Xin.X.to(DEV)
                u, c = gr.hc_fused_write_read(R, y, ci, p)
            outs.append((R, u, c))
    torch.cuda.synchronize()
    for (R1, u1, c1), (R2, u2, c2) in zip(alone, outs):
        assert torch.equal(R1, R2) and torch.equal(u1, u2) and torch.equal(c1, c2)
