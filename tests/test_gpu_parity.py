"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Same seeded inputs on both sides; sizes the oracle finishes in seconds that
span several tiles plus ragged tails, and the full workload sizes on sampled
tokens.  Tolerances are in tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import write_gr_read_amd as gr
from write_gr_read_amd import inputs
from parity import check, check_chain, check_exact, combine_scale, sample_tokens, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu_and_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gr.lib()  # raises if the HIP library is missing: no silent fallback


def dev_params(p):
    return p.to(DEV)


def orc_read(X, p, dtype, eps=1e-6):
    """Oracle read; returns (u, s, A) with A the combine's condition scale."""
    u, s, rho, G = oracle.read(X, p.gamma, p.w_down, p.w_up, p.w_write, eps, dtype, detail=True)
    return u, s, combine_scale(X, p.gamma, rho, G)


def orc_fused(X, y, s, p, dtype, eps=1e-6):
    """Oracle fused write+read; returns (R', u, s, A)."""
    R, u, s_out = oracle.fused(X, y, s, p.gamma, p.w_down, p.w_up, p.w_write, eps, dtype)
    u2, s2, A = orc_read(R, p, dtype, eps)
    assert np.array_equal(u, u2) and np.array_equal(s_out, s2)
    return R, u, s_out, A


def run_read_write_fused(Xin: inputs.GRInputs, label: str):
    """read(P0), write, fused(P1) on the GPU vs the oracle, whole tensors."""
    dt = Xin.dtype
    p0, p1 = Xin.params[0], Xin.params[1]
    X = Xin.X.to(DEV)
    y = Xin.y.to(DEV)
    # read
    u0, s0 = gr.read(X, dev_params(p0))
    ou0, os0, A0 = orc_read(Xin.X, p0, dt)
    check(f"{label} read u", u0, ou0, dt)
    check(f"{label} read s", s0, os0, dt)
    # write with the oracle's strengths (same input on both sides)
    s_in = torch.from_numpy(os0).float()
    Xw = X.clone()
    gr.write(Xw, y, s_in.to(DEV))
    oRw = oracle.write(Xin.X, Xin.y, s_in.double().numpy(), dt)
    check_exact(f"{label} write state", Xw, oRw)
    # fused write + read of the next sublayer
    Xf = X.clone()
    u1, s1 = gr.fused_write_read(Xf, y, s_in.to(DEV), dev_params(p1))
    oR, ou1, os1, A1 = orc_fused(Xin.X, Xin.y, s_in.double().numpy(), p1, dt)
    check_exact(f"{label} fused state", Xf, oR)
    check(f"{label} fused u", u1, ou1, dt)
    check(f"{label} fused s", s1, os1, dt)
    # the fused state is exactly the standalone write's
    assert torch.equal(Xf, Xw), f"{label}: fused state differs from gr_write's"
    torch.cuda.synchronize()


def test_tiny_fp32_workload():
    """Workload 1: N=64, d=256, n=4, r=16, fp32: read, write and fused."""
    run_read_write_fused(inputs.workload(1), "tiny-f32")


@pytest.mark.parametrize("N,n,d,r", [
    (37, 4, 256, 16), (1, 4, 4096, 64), (5, 1, 64, 0), (9, 2, 128, 1), (17, 3, 64, 5),
    (3, 8, 32, 2), (70, 4, 512, 32), (130, 4, 1024, 48), (33, 4, 2048, 32), (64, 4, 256, 0),
    (200, 4, 4096, 64), (264, 4, 4096, 64),
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shapes(N, n, d, r, dtype):
    """Off-workload shapes: several tiles, ragged token tails, n in 1..8,
    r in {0, 1, 2, 5, ...}; both storage dtypes.  With a bf16 state the few-token
    kernel 1 takes its one-batch forms at 1 (N <= 64 at d = 4096), 2 (N = 200,
    264) and 4 k-steps (the decode workload); at N = 264 (two 16-token groups per
    wave) the last workgroup's second group is empty."""
    X = inputs.make_gr_inputs(N, n, d, r, dtype, seed=N * 131 + n * 17 + d + r, w_std=0.05,
                              branch_scale=None)
    run_read_write_fused(X, f"N{N}-n{n}-d{d}-r{r}-{dtype}")


@pytest.mark.parametrize("N,n,d,r", [
    (37, 4, 256, 16), (1, 4, 4096, 64), (5, 1, 64, 0), (17, 3, 64, 5), (70, 4, 512, 32),
    (130, 4, 1024, 48), (300, 4, 192, 32), (129, 4, 384, 96), (257, 4, 320, 128), (64, 4, 256, 0),
    (256, 4, 4096, 64), (1024, 4, 4096, 64),
])
@pytest.mark.parametrize("path", ["default", "generic"])
def test_fp8_state_shapes(N, n, d, r, path, monkeypatch):
    """fp8 (e4m3) branch state, bf16 everything else: read, write and fused
    against the oracle on the same stored e4m3 values (state bit for bit,
    u at the bf16 tolerance).  "default" takes the MFMA kernels wherever the
    shape allows (n = 4, r a multiple of 16, d a multiple of 64), including a
    last channel range of one 64-channel unit (d = 192, 320), every k-step
    count of the up projection and the few-token kernel 1 (at N = 1024, its
    largest size, ahead of the resident kernel 2);
    "generic" forces the shape-generic kernels on the same shapes."""
    if path == "generic":
        monkeypatch.setenv("GR_KERNEL_VARIANT", "generic")
    X = inputs.make_gr_inputs(N, n, d, r, "fp8", seed=3 * N + 5 * n + d + r, w_std=0.05,
                              branch_scale=(1.0, 0.5, 2.0, 1.0)[:n] if n == 4 else None)
    run_read_write_fused(X, f"fp8-{path}-N{N}-n{n}-d{d}-r{r}")


@pytest.mark.parametrize("N,d,r,w_std", [(2500, 4096, 64, 0.05), (1200, 8192, 32, 0.5),
                                         (3000, 192, 16, 0.3), (700, 2560, 96, 0.2)])
def test_fp8_state_many_tiles(N, d, r, w_std):
    """fp8 state with more token tiles than kernel-2 workgroups, so each
    workgroup walks several tiles (and, at d = 192, a range of one unit)."""
    X = inputs.make_gr_inputs(N, 4, d, r, "fp8", seed=11 * N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"fp8-tiles-N{N}-d{d}-r{r}")


def test_fp8_state_saturates():
    """Writes that overflow e4m3 store +-448 (the saturation reading)."""
    X = inputs.make_gr_inputs(20, 4, 64, 8, "fp8", seed=77, x_std=100.0, y_std=200.0)
    R = X.X.to(DEV)
    s = torch.full((20, 4), 2.0, device=DEV)
    gr.write(R, X.y.to(DEV), s)
    oR = oracle.write(X.X, X.y, s.cpu().double().numpy(), "fp8")
    check_exact("fp8 saturating write", R, oR)
    assert np.abs(oR).max() == 448.0 and torch.isfinite(R.float()).all()


@pytest.mark.parametrize("N,d,r,w_std", [
    (37, 256, 16, 0.05), (1, 4096, 64, 0.05), (130, 1024, 48, 0.3), (300, 192, 32, 0.05),
    (129, 384, 96, 0.2), (257, 320, 128, 0.05), (2500, 4096, 64, 0.05), (1200, 8192, 32, 0.5),
])
@pytest.mark.parametrize("form", ["staged", "resident"])
def test_kernel2_forms(N, d, r, w_std, form, monkeypatch):
    """Both forms of the fast path's gate/combine kernel on every shape class
    (the library picks one by token count): a ragged last channel range
    (d = 192, 320), every k-step count of the up projection (r = 16 .. 128),
    ragged token tiles, and more token tiles than workgroups (N = 2500 at
    d = 4096, N = 1200 at d = 8192), so a workgroup walks several tiles."""
    monkeypatch.setenv("GR_KERNEL_VARIANT", form)
    X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=7 * N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"{form}-N{N}-d{d}-r{r}")


@pytest.mark.parametrize("N,d,r,dtype", [(4133, 4096, 64, "bf16"), (8250, 2048, 32, "fp8")])
def test_resident_walk_order(N, d, r, dtype):
    """Many tokens, every token compared: kernel 1 rotates its walk per token
    tile (with channel splits at N = 4133), and each resident kernel-2
    workgroup visits its tiles in two passes (recently written ones first);
    with several tiles per workgroup from both passes and a ragged last tile,
    a tile visited twice or not at all would show here."""
    X = inputs.make_gr_inputs(N, 4, d, r, dtype, seed=11 * N + d + r, w_std=0.2,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"walk-N{N}-d{d}-r{r}-{dtype}")


@pytest.mark.parametrize("N,d,r,w_std", [(37, 256, 16, 0.05), (300, 192, 32, 0.05), (257, 320, 128, 0.2),
                                         (2500, 4096, 64, 0.05)])
@pytest.mark.parametrize("form", ["staged", "resident"])
def test_kernel2_forms_fp8(N, d, r, w_std, form, monkeypatch):
    """Both kernel-2 forms on an e4m3 state (staged: 8 bytes per lane widened
    to bf16 words; resident: 64-channel units), a ragged last range (d = 192,
    320) and several tiles per workgroup (N = 2500)."""
    monkeypatch.setenv("GR_KERNEL_VARIANT", form)
    X = inputs.make_gr_inputs(N, 4, d, r, "fp8", seed=5 * N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"fp8-{form}-N{N}-d{d}-r{r}")


@pytest.mark.parametrize("N,d,r,w_std", [(64, 512, 32, 0.5), (130, 1024, 48, 0.3),
                                         (48, 4096, 64, 0.2)])
def test_saturating_gate(N, d, r, w_std):
    """Large gate weights drive G over the whole (0, 1) range and s far from 1,
    so a gate value landing on the wrong channel or branch cannot hide inside
    the tolerance (with N(0, 0.02) weights G stays near 1/2)."""
    X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=N + d + r, w_std=w_std)
    _, _, _, G = oracle.read(X.X, X.params[0].gamma, X.params[0].w_down, X.params[0].w_up,
                             X.params[0].w_write, detail=True)
    assert G.min() < 0.05 and G.max() > 0.95
    run_read_write_fused(X, f"saturating-N{N}-d{d}-r{r}")


@pytest.mark.parametrize("N,d,r", [(100, 4096, 64), (511, 1024, 48), (512, 4096, 64), (600, 8192, 64),
                                   (512, 4096, 96), (896, 1024, 32), (897, 1024, 32), (1025, 1024, 32),
                                   (1000, 1024, 32), (1024, 2048, 64), (2065, 1024, 16), (3000, 4096, 64)])
def test_kernel1_forms_by_token_count(N, d, r):
    """Kernel 1 takes its few-token form with fewer than 8 tiles of 128 tokens
    (N <= 1024, n = 4) and the tile walk with channel splits from there, until
    the grid is full; both sides of each switch, ragged tails, every token
    compared.  The few-token form takes one 16-token group per wave below 256
    tokens (N = 100) or with more than 5 row blocks (r = 96), two from there
    (sharing each W fragment), with its batch loop at N = 600, d = 8192 (two
    groups) and N = 512, r = 96 (one group)."""
    X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=7 * N + d + r, w_std=0.2,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"k1-forms-N{N}-d{d}-r{r}")


def test_workspace_needs_no_initialisation():
    """Every workspace byte a call reads is written earlier in the same call:
    a workspace full of 0xFF (NaN floats, huge counts) changes nothing."""
    X = inputs.make_gr_inputs(300, 4, 1024, 32, "bf16", seed=45)
    p0, p1 = dev_params(X.params[0]), dev_params(X.params[1])
    R = X.X.to(DEV)
    y = X.y.to(DEV)
    s_in = torch.full((300, 4), 0.75, device=DEV)
    runs = []
    for fill in (0xFF, 0x00):
        gr.read(R, p0)  # make sure this stream's workspace exists
        dev = torch.device(DEV)
        gr._workspaces[(dev, gr._stream(dev))].fill_(fill)
        Rc = R.clone()
        u, s = gr.fused_write_read(Rc, y, s_in, p1)
        torch.cuda.synchronize()
        runs.append((Rc.cpu(), u.cpu(), s.cpu()))
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b)
    assert torch.isfinite(runs[0][1].float()).all()


@pytest.mark.parametrize("N,d,r,w_std", [
    (1, 2560, 320, 0.05), (64, 2560, 320, 0.05), (37, 512, 144, 0.05), (130, 1024, 256, 0.2),
    (300, 640, 320, 0.05), (129, 2560, 160, 0.3), (200, 448, 224, 0.5), (2500, 256, 320, 0.2),
])
def test_wide_gate_shapes(N, d, r, w_std):
    """Gate ranks beyond 124 (r + n > 128 projection rows): kernel 1's wide
    form (raw weights in LDS, gamma . R' split into hi / lo on the state side)
    and kernel 2's 32-channel resident form.  Ragged token tiles, channel
    splits at few tokens (N = 1, 64) and in the tile walk (N = 2500: four
    splits, whose record reduction gathers a lane's outputs in rounds), r from
    144 to 320, and large weights (w_std = 0.5) so the gate spans (0, 1)."""
    X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=13 * N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"wide-N{N}-d{d}-r{r}")


@pytest.mark.parametrize("N,d,r,w_std", [(4300, 256, 320, 0.2), (4200, 384, 192, 0.05)])
@pytest.mark.parametrize("form", ["default", "resident"])
def test_wide_gate_many_tokens(N, d, r, w_std, form, monkeypatch):
    """Wide gates at 4096 tokens and more, every token compared: by default
    kernel 2 walks XCD by XCD (token tiles T = x, x + 8, ... on XCD x, each
    workgroup taking its share of (channel range, tile) units and restaging
    W_up per range); "resident" forces the plain range-per-workgroup walk."""
    if form == "resident":
        monkeypatch.setenv("GR_KERNEL_VARIANT", "resident")
    X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=17 * N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"wide-{form}-N{N}-d{d}-r{r}")


@pytest.mark.parametrize("N,d,r,w_std", [
    (1, 2560, 320, 0.05), (64, 2560, 320, 0.05), (37, 512, 144, 0.05), (130, 1024, 256, 0.2),
    (300, 640, 320, 0.05), (129, 2560, 160, 0.3), (200, 384, 224, 0.5), (4300, 256, 320, 0.2),
    (4200, 384, 192, 0.05), (50, 448, 224, 0.05),
])
def test_fp8_state_wide_gate(N, d, r, w_std):
    """e4m3 state with a gate rank beyond 124: kernel 1's wide form on e4m3
    rows and kernel 2's XCD walk with four 32-channel ranges (one 128-byte
    line of e4m3) in lockstep, at few and many tokens; d = 448 is not a
    multiple of 128 and takes the shape-generic kernels."""
    X = inputs.make_gr_inputs(N, 4, d, r, "fp8", seed=19 * N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0))
    run_read_write_fused(X, f"fp8-wide-N{N}-d{d}-r{r}")


def test_wide_gate_without_write_projection():
    """r = 320 with no W_write: 320 projection rows (20 blocks), s == 1."""
    X = inputs.make_gr_inputs(100, 4, 1280, 320, "bf16", seed=43, with_write=False)
    u, s = gr.read(X.X.to(DEV), dev_params(X.params[0]))
    assert torch.all(s == 1.0)
    ou, _, A = orc_read(X.X, X.params[0], "bf16")
    check("wide no-write u", u, ou, "bf16")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_no_write_projection_gives_unit_strength(dt):
    """No W_write: s == 1 (the fp32 case takes the small-row kernel, whose
    one-batch form loads W_down rows in place of the missing write rows)."""
    X = inputs.make_gr_inputs(40, 4, 256, 16, dt, seed=41, with_write=False)
    u, s = gr.read(X.X.to(DEV), dev_params(X.params[0]))
    assert torch.all(s == 1.0)
    ou, _, A = orc_read(X.X, X.params[0], dt)
    check("no-write u", u, ou, dt)
    if dt == "f32":
        S = X.X.to(DEV)
        u2, s2 = gr.fused_write_read(S, X.y.to(DEV), s.clone(), dev_params(X.params[0]))
        assert torch.all(s2 == 1.0)


def test_zero_write_projection_gives_exactly_one():
    X = inputs.make_gr_inputs(40, 4, 512, 16, "bf16", seed=42)
    p = X.params[0]
    p.w_write = torch.zeros_like(p.w_write)
    _, s = gr.read(X.X.to(DEV), dev_params(p))
    assert torch.all(s == 1.0)


@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
def test_empty_inputs(dt):
    """N = 0 on every GR call through the binding: no error, empty outputs."""
    X = inputs.make_gr_inputs(1, 4, 256, 16, "f32" if dt == "f32" else "bf16", seed=3)
    p = X.params[0].to(DEV)
    sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dt]
    pdt = torch.float32 if dt == "f32" else torch.bfloat16
    S = torch.empty((0, 4, 256), dtype=sdt, device=DEV)
    y = torch.empty((0, 256), dtype=pdt, device=DEV)
    s = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    u, s1 = gr.read(S, p)
    assert u.shape == (0, 256) and s1.shape == (0, 4)
    assert gr.write(S, y, s).shape == (0, 4, 256)
    u, s1 = gr.fused_write_read(S, y, s, p)
    assert u.shape == (0, 256) and s1.shape == (0, 4)
    if dt != "fp8":
        x = torch.empty((0, 256), dtype=pdt, device=DEV)
        w = torch.ones(256, dtype=pdt, device=DEV)
        assert gr.residual_add_rmsnorm(x, x.clone(), w).shape == (0, 256)
    torch.cuda.synchronize()


def test_zero_strength_and_zero_output_are_identities():
    X = inputs.make_gr_inputs(50, 4, 512, 16, "bf16", seed=43)
    R = X.X.to(DEV)
    y = X.y.to(DEV)
    R1 = R.clone()
    gr.write(R1, y, torch.zeros(50, 4, device=DEV))
    assert torch.equal(R1, R)
    R2 = R.clone()
    gr.write(R2, torch.zeros_like(y), torch.rand(50, 4, device=DEV) * 2)
    assert torch.equal(R2, R)
    R3 = R.clone()
    gr.fused_write_read(R3, y, torch.zeros(50, 4, device=DEV), dev_params(X.params[1]))
    assert torch.equal(R3, R)


def test_bf16_store_rounding_is_round_to_nearest_even():
    """With s = 1, wherever the sum is exact in fp32 the stored state is exactly
    torch's round-to-nearest-even bf16 of the sum (ties included)."""
    X = inputs.make_gr_inputs(64, 4, 1024, 0, "bf16", seed=44, n_param_sets=0)
    Rf, yf = X.X.float(), X.y.float()
    f32_sum = Rf + yf[:, None, :]
    exact = f32_sum.double() == X.X.double() + X.y.double()[:, None, :]
    assert exact.float().mean().item() > 0.99
    R = X.X.to(DEV)
    gr.write(R, X.y.to(DEV), torch.ones(64, 4, device=DEV))
    got = R.cpu()
    want = f32_sum.to(torch.bfloat16)
    assert bool((got.view(torch.int16) == want.view(torch.int16))[exact].all())


def test_n1_gr_equals_add_rmsnorm():
    """n = 1, unit gate, no write projection, s = 1: the fused GR call is the
    fused residual add + RMSNorm."""
    X = inputs.make_gr_inputs(300, 1, 4096, 0, "bf16", seed=45, with_write=False)
    p = X.params[0]
    R = X.X.to(DEV)
    u, s = gr.fused_write_read(R, X.y.to(DEV), torch.ones(300, 1, device=DEV), dev_params(p))
    x = X.X[:, 0].contiguous().to(DEV)
    out = gr.residual_add_rmsnorm(x, X.y.to(DEV), p.gamma[0].contiguous().to(DEV))
    assert torch.equal(R[:, 0], x)
    check("n1 u vs addnorm", u, out, "bf16")
    assert torch.all(s == 1.0)


def test_deterministic():
    X = inputs.make_gr_inputs(200, 4, 2048, 32, "bf16", seed=46)
    outs = []
    for _ in range(2):
        R = X.X.to(DEV)
        _, s0 = gr.read(R, dev_params(X.params[0]))
        u, s = gr.fused_write_read(R, X.y.to(DEV), s0, dev_params(X.params[1]))
        outs.append((R.cpu(), u.cpu(), s.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_outputs_stay_in_bounds():
    """Outputs carved out of larger canary-filled buffers: nothing outside the
    result regions changes."""
    N, n, d, r = 45, 4, 512, 16
    X = inputs.make_gr_inputs(N, n, d, r, "bf16", seed=47)
    pad = 4096
    canary = -1234.5
    Rbuf = torch.full((pad + N * n * d + pad,), canary, dtype=torch.bfloat16, device=DEV)
    ubuf = torch.full((pad + N * d + pad,), canary, dtype=torch.bfloat16, device=DEV)
    sbuf = torch.full((pad + N * n + pad,), canary, dtype=torch.float32, device=DEV)
    R = Rbuf[pad:pad + N * n * d].view(N, n, d)
    R.copy_(X.X.to(DEV))
    u = ubuf[pad:pad + N * d].view(N, d)
    s = sbuf[pad:pad + N * n].view(N, n)
    s_in = torch.ones(N, n, device=DEV)
    gr.fused_write_read(R, X.y.to(DEV), s_in, dev_params(X.params[1]), u=u, s=s)
    for buf, lo, hi in ((Rbuf, pad, pad + N * n * d), (ubuf, pad, pad + N * d),
                        (sbuf, pad, pad + N * n)):
        assert torch.all(buf[:lo] == canary) and torch.all(buf[hi:] == canary)


# ---------------------------------------------------------------- the workloads

def sampled_read_parity(Xin, idx, label, fused=True):
    """Run the whole workload on the GPU; compare sampled tokens with the
    oracle evaluated on just those tokens (GR is per token)."""
    dt = Xin.dtype
    p0, p1 = Xin.params[0], Xin.params[1]
    X = Xin.X.to(DEV)
    _, s0 = gr.read(X, dev_params(p0))
    _, os0, _ = orc_read(Xin.X[idx], p0, dt)
    check(f"{label} read s (sampled)", s0.cpu()[idx], os0, dt)
    # the fused call's strengths: the oracle's at the sampled tokens (same
    # input on both sides), the GPU's elsewhere
    s_in = s0.clone()
    s_in[torch.from_numpy(idx).to(DEV)] = torch.from_numpy(os0).float().to(DEV)
    u1, s1 = gr.fused_write_read(X, Xin.y.to(DEV), s_in, dev_params(p1))
    oR, ou1, os1, A1 = orc_fused(Xin.X[idx], Xin.y[idx], os0, p1, dt)
    Xc = X.cpu()
    u1c = u1.cpu()
    check_exact(f"{label} fused state (sampled)", Xc[idx], oR)
    check(f"{label} fused u (sampled)", u1c[idx], ou1, dt)
    check(f"{label} fused s (sampled)", s1.cpu()[idx], os1, dt)
    assert torch.isfinite(u1c.float()).all() and torch.isfinite(Xc.float()).all()


def test_prefill_workload_subset():
    """Workload 3 (d=4096, n=4, r=64, per-branch scales 1, 0.5, 2, 1), first
    1024 tokens, every token compared."""
    run_read_write_fused(inputs.workload(3, N=1024), "prefill-1024")


def test_prefill_workload_full_sampled():
    """Workload 3 at its full size (N=16384), 96 sampled tokens."""
    Xin = inputs.workload(3)
    sampled_read_parity(Xin, sample_tokens(Xin.N, 96, seed=3), "prefill-16384")


def test_prefill_fp8_workload_subset():
    """Workload 6 (the prefill shape with an e4m3 state), first 1024 tokens,
    every token compared."""
    run_read_write_fused(inputs.workload(6, N=1024), "prefill-fp8-1024")


def test_prefill_fp8_workload_full_sampled():
    """Workload 6 at its full size (N=16384), 96 sampled tokens."""
    Xin = inputs.workload(6)
    sampled_read_parity(Xin, sample_tokens(Xin.N, 96, seed=6), "prefill-fp8-16384")


def test_real_shape_r320_subset():
    """Workload 7 (the pages' model shape: d = 2560, r = d/8 = 320), first
    256 tokens, every token compared."""
    run_read_write_fused(inputs.workload(7, N=256), "d2560-r320-256")


def test_real_shape_r320_full_sampled():
    """Workload 7 at its full size (N=16384), 64 sampled tokens."""
    Xin = inputs.workload(7)
    sampled_read_parity(Xin, sample_tokens(Xin.N, 64, seed=7), "d2560-r320-16384")


def test_real_shape_fp8_subset():
    """Workload 8 (d = 2560, r = 320, e4m3 state), first 256 tokens, every
    token compared."""
    run_read_write_fused(inputs.workload(8, N=256), "fp8-d2560-r320-256")


def test_real_shape_fp8_full_sampled():
    """Workload 8 at its full size (N=16384), 64 sampled tokens."""
    Xin = inputs.workload(8)
    sampled_read_parity(Xin, sample_tokens(Xin.N, 64, seed=8), "fp8-d2560-r320-16384")


def test_state_beyond_2_31_elements():
    """N x n x d above 2^31 elements (131372 x 4 x 4096 bf16, a 4.3 GB state):
    kernel 1's tile walk, kernel 2's resident walk and the record reduction
    address past 32-bit element offsets.  Tokens sampled on both sides of the
    boundary (token 131072 starts at element 2^31) are compared with the
    oracle, which gets those rows of the same device tensors."""
    N, n, d, r = 131372, 4, 4096, 64
    P = inputs.make_gr_inputs(1, n, d, r, "bf16", seed=91, n_param_sets=2).params
    X, y = inputs.make_device_state(N, n, d, "bf16", seed=92, device=DEV)
    idx = np.unique(np.concatenate([[0, 1, 65535, 131070, 131071, 131072, 131073, N - 2, N - 1],
                                    sample_tokens(N, 24, seed=93)]))
    ti = torch.from_numpy(idx).to(DEV)
    Xs, ys = X[ti].cpu(), y[ti].cpu()
    u0, s0 = gr.read(X, dev_params(P[0]))
    ou0, os0, A0 = orc_read(Xs, P[0], "bf16")
    check("2^31 read u (sampled)", u0[ti].cpu(), ou0, "bf16")
    check("2^31 read s (sampled)", s0[ti].cpu(), os0, "bf16")
    s_in = s0.clone()
    s_in[ti] = torch.from_numpy(os0).float().to(DEV)
    u1, s1 = gr.fused_write_read(X, y, s_in, dev_params(P[1]))
    oR, ou1, os1, A1 = orc_fused(Xs, ys, os0, P[1], "bf16")
    check_exact("2^31 fused state (sampled)", X[ti].cpu(), oR)
    check("2^31 fused u (sampled)", u1[ti].cpu(), ou1, "bf16")
    check("2^31 fused s (sampled)", s1[ti].cpu(), os1, "bf16")
    del X, y, u0, u1
    torch.cuda.empty_cache()


def test_decode_workload():
    """Workload 4 (N=256), every token."""
    run_read_write_fused(inputs.workload(4), "decode-256")


def test_add_rmsnorm_workload():
    """Workload 2 (n=1, N=8192, d=4096): full size, 128 sampled tokens, plus
    a ragged small case compared whole."""
    A = inputs.workload(2)
    x = A.x.to(DEV)
    out = gr.residual_add_rmsnorm(x, A.y.to(DEV), A.w.to(DEV))
    idx = sample_tokens(A.N, 128, seed=2)
    h, o = oracle.add_rmsnorm(A.x[idx], A.y[idx], A.w, A.eps, "bf16")
    check("addnorm h", x.cpu()[idx], h, "bf16")
    check("addnorm out", out.cpu()[idx], o, "bf16")
    for N, d, dt in ((7, 24, "bf16"), (13, 4100, "f32"), (3, 40000, "bf16"), (5, 8, "bf16")):
        B = inputs.make_addnorm_inputs(N, d, dt, seed=N + d)
        x = B.x.to(DEV)
        out = gr.residual_add_rmsnorm(x, B.y.to(DEV), B.w.to(DEV))
        h, o = oracle.add_rmsnorm(B.x, B.y, B.w, B.eps, dt)
        check(f"addnorm h {N}x{d}", x, h, dt)
        check(f"addnorm out {N}x{d}", out, o, dt)


@pytest.mark.parametrize("N,d,dt,alias", [(1500, 4096, "bf16", False), (2049, 2048, "f32", False),
                                         (3001, 8192, "bf16", True), (1100, 16384, "bf16", False)])
def test_add_rmsnorm_walk(N, d, dt, alias):
    """The persistent add + RMSNorm (above 1024 tokens): every token compared,
    token counts that are not multiples of the grid, every rows-per-thread
    count, and out written over y (the one aliasing the call allows)."""
    B = inputs.make_addnorm_inputs(N, d, dt, seed=3 * N + d)
    x, y = B.x.to(DEV), B.y.to(DEV)
    out = gr.residual_add_rmsnorm(x, y, B.w.to(DEV), out=y if alias else None)
    h, o = oracle.add_rmsnorm(B.x, B.y, B.w, B.eps, dt)
    check(f"addnorm-walk h {N}x{d}", x, h, dt)
    check(f"addnorm-walk out {N}x{d}", out, o, dt)


def gpu_chain(Xin):
    X = Xin.X.to(DEV)
    ps = [dev_params(p) for p in Xin.params]
    u, s = gr.read(X, ps[0])
    y = gr.tanh_standin(u)
    for p in ps[1:]:
        u, s = gr.fused_write_read(X, y, s, p)
        y = gr.tanh_standin(u)
    gr.write(X, y, s)
    return X


def test_tanh_standin():
    """16-byte vectors and a count with a ragged tail (the element-wise form)."""
    u = torch.randn(5003, dtype=torch.float32) * 3
    for dt in (torch.float32, torch.bfloat16):
        uu = u.to(dt)
        ref = oracle.tanh_standin(uu, "f32" if dt == torch.float32 else "bf16")
        check(f"tanh {dt}", gr.tanh_standin(uu.to(DEV)), ref, "bf16")


def chain_scale(X0, ss, ys):
    """A for a chained state: |R^(0)| + sum_u |s^(u) y^(u)| (oracle values)."""
    A = np.abs(to64(X0))
    for s, y in zip(ss, ys):
        A = A + np.abs(s[:, :, None] * y[:, None, :])
    return A


def test_chain_workload_subset():
    """Workload 5's 32-sublayer chain (d=2048, n=4, r=32) on its first 256
    tokens: final state vs the oracle's own chain (its own s, y and F)."""
    Xin = inputs.workload(5, N=256)
    R = gpu_chain(Xin)
    oR, ss, ys = oracle.chain(Xin.X, Xin.params, Xin.eps, "bf16", record=True)
    check_chain("chain final state", R, oR, chain_scale(Xin.X, ss, ys))
    # The GPU trajectory is as close to the exact chain (fp64 storage, no
    # rounding) as the oracle's own bf16 trajectory is.
    exact = oracle.chain(Xin.X, Xin.params, Xin.eps, "f64")
    dev_gpu = np.sqrt(np.mean((to64(R) - exact) ** 2))
    dev_orc = np.sqrt(np.mean((oR - exact) ** 2))
    assert dev_gpu <= 1.1 * dev_orc, (dev_gpu, dev_orc)


def test_chain_closed_form_with_gpu_strengths():
    """P8, eq:rcv: after the 32-sublayer chain the state is R^(0) + sum_l s^(l) y^(l),
    formed here in fp64 from the GPU's own strengths and sublayer outputs, up to
    the 32 stores.  Each write rounds R + s y once to fp32 (one FMA) and once to
    bf16 (at most half an ulp, 2^-8 of the value), so element by element
    |g - closed| <= 1.01 (2^-8 + 2^-23) sum_l |R^(l)| with R^(l) the partial sums
    (the 1 % covers the earlier errors carried into each rounded value)."""
    Xin = inputs.workload(5, N=256)
    X = Xin.X.to(DEV)
    ps = [dev_params(p) for p in Xin.params]
    writes = []
    u, s = gr.read(X, ps[0])
    y = gr.tanh_standin(u)
    for p in ps[1:]:
        writes.append((s.clone(), y.clone()))
        u, s = gr.fused_write_read(X, y, s, p)
        y = gr.tanh_standin(u)
    writes.append((s.clone(), y.clone()))
    gr.write(X, y, s)
    torch.cuda.synchronize()
    assert len(writes) == 32
    part = to64(Xin.X)
    total = np.zeros_like(part)
    for sl, yl in writes:
        part = part + to64(sl)[:, :, None] * to64(yl)[:, None, :]
        total += np.abs(part)
    err = np.abs(to64(X) - part)
    bound = 1.01 * (2.0 ** -8 + 2.0 ** -23) * total
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} elements past the rounding bound; worst ratio "
                           f"{float((err / np.maximum(bound, 1e-300)).max()):.3f}")
    # the bound is not vacuous: the rounding errors are there, and well inside it
    assert 0 < float(err.max()) and float((err / np.maximum(bound, 1e-300)).max()) < 1


def test_chain_workload_full_sampled():
    """Workload 5 at full size (N=32768): the oracle runs the chain on 32
    sampled tokens."""
    Xin = inputs.workload(5)
    R = gpu_chain(Xin).cpu()
    idx = sample_tokens(Xin.N, 32, seed=5)
    oR, ss, ys = oracle.chain(Xin.X[idx], Xin.params, Xin.eps, "bf16", record=True)
    check_chain("chain-full final state (sampled)", R[idx], oR, chain_scale(Xin.X[idx], ss, ys))


def test_concurrent_streams_keep_separate_workspaces():
    """Two fused calls in flight at once on two streams (default priority),
    each with its own inputs and, through the binding, its own workspace:
    every result equals the same call made alone, bit for bit.  A shared
    workspace would mix the two calls' records."""
    A = inputs.make_gr_inputs(4500, 4, 2048, 64, "bf16", seed=31, branch_scale=(1.0, 0.5, 2.0, 1.0))
    B = inputs.make_gr_inputs(700, 4, 2048, 64, "bf16", seed=32, branch_scale=(1.0, 0.5, 2.0, 1.0))
    runs = []
    for Xin in (A, B):
        p = dev_params(Xin.params[1])
        R = Xin.X.to(DEV)
        s_in = torch.full((Xin.N, 4), 0.9, device=DEV)
        u, s = gr.fused_write_read(R, Xin.y.to(DEV), s_in, p)        # alone, current stream
        torch.cuda.synchronize()
        runs.append((Xin, p, s_in, R, u, s))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (Xin, p, s_in, _, _, _), st in zip(runs, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            R = Xin.X.to(DEV, non_blocking=False)
            y = Xin.y.to(DEV)
            for _ in range(3):                                        # several calls queued per stream
                Rc = R.clone()
                u, s = gr.fused_write_read(Rc, y, s_in, p)
            outs.append((Rc, u, s))
    torch.cuda.synchronize()
    for (_, _, _, R1, u1, s1), (R2, u2, s2) in zip(runs, outs):
        assert torch.equal(R1, R2) and torch.equal(u1, u2) and torch.equal(s1, s2)


def test_graph_replay_matches_eager():
    """The fused call captured in a HIP graph (torch.cuda.CUDAGraph) and
    replayed three times, with eager work and synchronisations in between:
    every replay gives the eager result bit for bit (state, u, s).  The
    kernels record no memset, so the graph holds kernel nodes only."""
    X = inputs.make_gr_inputs(300, 4, 1024, 64, "bf16", seed=21, branch_scale=(1.0, 0.5, 2.0, 1.0))
    p = dev_params(X.params[1])
    R0, y = X.X.to(DEV), X.y.to(DEV)
    s_in = torch.rand(300, 4, device=DEV) * 2
    # eager reference
    Re = R0.clone()
    ue, se = gr.fused_write_read(Re, y, s_in, p)
    # static buffers for the graph; one eager call first (no allocation inside the capture)
    Rg = R0.clone()
    ug = torch.empty_like(ue)
    sg = torch.empty_like(se)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gr.fused_write_read(Rg, y, s_in, p, u=ug, s=sg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):     # the warmed-up stream: same workspace
        gr.fused_write_read(Rg, y, s_in, p, u=ug, s=sg)
    for k in range(3):
        Rg.copy_(R0)                                # eager work between replays
        ug.zero_(); sg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Rg, Re), f"replay {k}: state differs"
        assert torch.equal(ug, ue), f"replay {k}: u differs"
        assert torch.equal(sg, se), f"replay {k}: s differs"
