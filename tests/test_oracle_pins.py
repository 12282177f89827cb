"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

None of these re-types the oracle's loops.  Each checks a closed form, a
special case that reduces to a textbook or library routine (torch's own
rms_norm / sigmoid / silu / tanh in float64), an invariant, or the pages'
worked example.  Sources:
  * "Paper reading: Qwen3.8 Flash Next", part 2 (Residual): sec. 4 (Gated
    Residual: eq:rms, eq:gate, eq:use_gate, eq:s, eq:write; GatedNorm),
    sec. 6 (eq:rcv branch accumulator, eq:auv contribution decomposition),
    sec. 7 (read and write fused).
  * "Qwen3.8-Flash-Next architecture notes, 06 Residual": the two-branch
    example, sections 2 and 3.
  * "Residual" (LLM inference): sec. 2.2 (Pre-Norm), 2.3 (residual stream
    unrolling), 3.3 (fused add + RMSNorm).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from write_gr_read_amd import inputs


def rmsnorm_lib(x, g, eps):
    """torch's RMSNorm (library routine) in float64 over the last axis."""
    x = torch.as_tensor(np.asarray(x, dtype=np.float64))
    g = torch.as_tensor(np.asarray(g, dtype=np.float64))
    return F.rms_norm(x, (x.shape[-1],), weight=g, eps=eps).numpy()


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


# ---------------------------------------------------------------- rounding

def test_round_bf16_matches_torch_on_fp32_values(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half = 0x8000), near-ties and subnormals
    ties = (rng.integers(0, 2**16, size=4000, dtype=np.uint32) << 16) | 0x8000
    near = ties ^ 1
    sub = rng.integers(0, 0x00800000, size=2000, dtype=np.uint32)
    bits = np.concatenate([bits, ties, near, sub, sub | 0x80000000])
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).double().numpy()
    got = np.array([orc.round_bf16(float(v)) for v in vals])
    both_inf = np.isinf(ref) & np.isinf(got) & (np.sign(ref) == np.sign(got))
    assert np.all((got == ref) | both_inf)


# ---------------------------------------------------------------- P1: n=1, unit gate

@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_n1_unit_gate_is_prenorm(orc, eps):
    """n=1, r=0, no write projection: read == RMSNorm(R; gamma), s == 1, and the
    write is the plain residual add, i.e. x + F(Norm(x)) exactly."""
    rng = np.random.default_rng(2)
    N, d = 7, 24
    R = rng.standard_normal((N, 1, d))
    g = 1 + 0.1 * rng.standard_normal((1, d))
    y = 0.1 * rng.standard_normal((N, d))
    u, s = orc.read(R, g, None, None, None, eps=eps, dtype="f64")
    np.testing.assert_allclose(u, rmsnorm_lib(R[:, 0], g[0], eps), rtol=1e-13, atol=1e-15)
    assert np.all(s == 1.0)
    Rw = orc.write(R, y, s, dtype="f64")
    np.testing.assert_array_equal(Rw[:, 0], R[:, 0] + y)


def test_n1_fused_equals_add_rmsnorm(orc):
    """The fused GR write+read at n=1 with unit gate and unit write strength is
    the fused residual add + RMSNorm (same stored h, same normalised output)."""
    X = inputs.make_gr_inputs(33, 1, 64, 0, "bf16", seed=3, n_param_sets=1, with_write=False)
    p = X.params[0]
    s1 = np.ones((33, 1))
    Rf, uf, sf = orc.fused(X.X, X.y, s1, p.gamma, None, None, None, dtype="bf16")
    h, out = orc.add_rmsnorm(X.X[:, 0], X.y, p.gamma[0], dtype="bf16")
    np.testing.assert_array_equal(Rf[:, 0], h)
    np.testing.assert_array_equal(uf, out)


def test_add_rmsnorm_vs_library(orc):
    A = inputs.make_addnorm_inputs(40, 128, "bf16", seed=4)
    xs, ys = A.x.float(), A.y.float()
    assert torch.equal(xs.double() + ys.double(), (xs + ys).double())  # fp32 sum exact here
    h_ref = (xs + ys).to(torch.bfloat16).double().numpy()
    h, out = orc.add_rmsnorm(A.x, A.y, A.w, dtype="bf16")
    np.testing.assert_array_equal(h, h_ref)
    o_ref = torch.from_numpy(rmsnorm_lib(h_ref, A.w.double().numpy(), 1e-6)).float() \
        .to(torch.bfloat16).double().numpy()
    # the oracle rounds fp64 -> bf16 once, torch fp64 -> fp32 -> bf16; allow one ulp
    assert np.max(np.abs(out - o_ref) / np.maximum(np.abs(o_ref), 1e-30)) <= 2 ** -7
    h64, out64 = orc.add_rmsnorm(A.x, A.y, A.w, dtype="f64")
    np.testing.assert_allclose(out64, rmsnorm_lib(h64, A.w.double().numpy(), 1e-6), rtol=1e-13)


# ---------------------------------------------------------------- P2: n=1 is GatedNorm

def test_n1_gated_read_is_gatednorm(orc):
    """GatedNorm(u) = RMSNorm(u) * sigmoid(W2 SiLU(W1 RMSNorm(u))); the GR read
    with one branch is exactly that with W1 = W_down, W2 = W_up."""
    rng = np.random.default_rng(5)
    N, d, r = 9, 16, 5
    R = rng.standard_normal((N, 1, d))
    g = 1 + 0.05 * rng.standard_normal((1, d))
    W1 = 0.3 * rng.standard_normal((r, d))
    W2 = 0.3 * rng.standard_normal((d, r))
    u, s = orc.read(R, g, W1, W2, None, eps=1e-6, dtype="f64")
    xn = torch.from_numpy(rmsnorm_lib(R[:, 0], g[0], 1e-6))
    gate = torch.sigmoid(F.silu(xn @ torch.from_numpy(W1).T) @ torch.from_numpy(W2).T)
    np.testing.assert_allclose(u, (xn * gate).numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P3 / P4: identities

def test_zero_write_projection_gives_unit_strength_exactly(orc):
    X = inputs.make_gr_inputs(12, 4, 32, 8, "bf16", seed=6, n_param_sets=1)
    p = X.params[0]
    u, s = orc.read(X.X, p.gamma, p.w_down, p.w_up, torch.zeros_like(p.w_write), dtype="bf16")
    assert np.all(s == 1.0)  # 2 * sigmoid(0) == 1
    Rw = orc.write(X.X, X.y, s, dtype="bf16")
    ref = (X.X.double() + X.y.double()[:, None, :]).float().to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(Rw, ref)


def test_write_rounds_through_fp32(orc):
    """eq:write is stored as the fp32 value of R + s y rounded to the storage
    dtype (the pages fix no precision; the kernels' fp32 is the reading).
    Worked cases, exact by hand: R = 1, y = 3/256, s = 1 - 2^-24 (an fp32).
    Exact sum 1 + 3/256 - 3*2^-32: its fp32 is the bf16 midpoint 1 + 3/256,
    which rounds to even, 1 + 2^-6; a single rounding of the exact sum would
    give 1 + 2^-7.  With s = 1 + 2^-23 the fp32 sum is again the midpoint and
    goes up to 1 + 2^-6, as the exact sum does."""
    R = np.array([[[1.0]]])
    y = np.array([[3.0 / 256]])
    s_dn = np.array([[1.0 - 2.0 ** -24]])
    s_up = np.array([[1.0 + 2.0 ** -23]])
    assert float(np.float32(s_dn[0, 0])) == s_dn[0, 0] and float(np.float32(s_up[0, 0])) == s_up[0, 0]
    assert orc.write(R, y, s_dn, dtype="bf16")[0, 0, 0] == 1.0 + 2.0 ** -6
    assert orc.write(R, y, s_up, dtype="bf16")[0, 0, 0] == 1.0 + 2.0 ** -6
    # fp32 storage: the single fp32 rounding of the exact sum
    assert orc.write(R, y, s_dn, dtype="f32")[0, 0, 0] == 1.0 + 3.0 / 256
    # f64: the exact sum
    assert orc.write(R, y, s_dn, dtype="f64")[0, 0, 0] == 1.0 + 3.0 / 256 - 3.0 * 2.0 ** -32
    # random cases, characterised without the oracle's own formula: against one
    # round-to-nearest-even of the exact sum to 8 significant bits (Python's
    # round() is ties-to-even), the oracle may differ only where the fp32 value
    # of the sum is exactly a midpoint between two bf16 values, and then by one
    # bf16 unit in the last place -- and such midpoints do occur in the sample
    rng = np.random.default_rng(3)
    Rr = torch.from_numpy(rng.standard_normal((64, 4, 64))).to(torch.bfloat16)
    yr = torch.from_numpy(2.0 ** -7 * rng.integers(-64, 64, (64, 64))).to(torch.bfloat16)
    sr = torch.from_numpy(rng.uniform(0, 2, (64, 4))).float()
    sr[:, 0] = 1.0 - 2.0 ** -24
    exact = (Rr.double() + sr.double()[:, :, None] * yr.double()[:, None, :]).numpy()  # exact in fp64
    got = orc.write(Rr, yr, sr.double().numpy(), dtype="bf16")

    def rne8(x):
        if x == 0.0:
            return 0.0
        _, e = math.frexp(x)
        return math.ldexp(round(math.ldexp(x, 8 - e)), e - 8)

    def is_bf16_midpoint(f):
        _, e = math.frexp(f)
        return math.ldexp(f, 9 - e) % 2 == 1        # odd in the 9th significant bit, nothing below
    one = np.vectorize(rne8)(exact)
    f32 = exact.astype(np.float32).astype(np.float64)
    diff = got != one
    assert diff.any(), "the sample should contain double-rounding cases"
    for g_, o_, f_ in zip(got[diff], one[diff], f32[diff]):
        _, e = math.frexp(o_)
        assert abs(g_ - o_) == math.ldexp(1.0, e - 8) or abs(g_ - o_) == math.ldexp(1.0, e - 9)
        assert is_bf16_midpoint(f_)


def test_round_e4m3_matches_torch_and_saturates(orc):
    """OCP e4m3 rounding (fp8 branch state) equals torch's float8_e4m3fn cast
    -- round to nearest, ties to even, subnormal step 2^-9 -- wherever that
    cast is finite; beyond the largest finite value 448 the state saturates
    (reading: e4m3fn has no infinity)."""
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(20000) * 4, rng.standard_normal(20000) * 0.01,
                           rng.standard_normal(2000) * 200,
                           # ties: midpoints between neighbours at several scales, subnormals
                           [1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 5 * 2.0 ** -10, 0.0, -1.0625,
                            440.0, 447.0, 456.0, 463.0]])
    vals = vals.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(vals).float().to(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.round_e4m3(v) for v in vals])
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(got[finite], ref[finite])
    big = ~finite
    assert big.sum() > 0
    np.testing.assert_array_equal(got[big], np.copysign(448.0, vals[big]))
    for v, want in ((464.0, 448.0), (1e6, 448.0), (-1e6, -448.0), (448.0, 448.0)):
        assert orc.round_e4m3(v) == want


def test_fp8_state_write_and_read(orc):
    """fp8 storage: the write stores e4m3(fp32(R + s y)); the read's u is bf16.
    Worked write cases (R = 1, y = 1/16): s = 1 gives 1.0625, an e4m3
    midpoint, stored as 1 (ties to even); s = 1 + 2^-23 gives an exact sum
    just above the midpoint whose fp32 value IS the midpoint, so it is also
    stored as 1 (one rounding of the exact sum would give 1.125)."""
    R = np.array([[[1.0]]])
    y = np.array([[1.0 / 16]])
    assert orc.write(R, y, np.array([[1.0]]), dtype="fp8")[0, 0, 0] == 1.0
    assert orc.write(R, y, np.array([[1.0 + 2.0 ** -23]]), dtype="fp8")[0, 0, 0] == 1.0
    assert orc.write(R, y, np.array([[1.0 + 2.0 ** -19]]), dtype="fp8")[0, 0, 0] == 1.125  # fp32 sum one ulp above
    # random state: every stored value is an e4m3 number (fixed point of the rounding)
    X = inputs.make_gr_inputs(6, 4, 64, 8, "bf16", seed=31, n_param_sets=1)
    R8 = X.X.float().to(torch.float8_e4m3fn).double().numpy()
    s = np.random.default_rng(2).uniform(0, 2, (6, 4)).astype(np.float32).astype(np.float64)
    Rw = orc.write(R8, X.y, s, dtype="fp8")
    np.testing.assert_array_equal(Rw, torch.from_numpy(Rw).float().to(torch.float8_e4m3fn).double().numpy())
    exact = (R8 + s[:, :, None] * X.y.double().numpy()[:, None, :]).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(Rw, np.array([orc.round_e4m3(v) for v in exact.ravel()]).reshape(exact.shape))
    # the read of an fp8 state stores u in bf16: the exact read rounded once
    p = X.params[0]
    u8, s8 = orc.read(R8, p.gamma, p.w_down, p.w_up, p.w_write, dtype="fp8")
    u64, s64 = orc.read(R8, p.gamma, p.w_down, p.w_up, p.w_write, dtype="f64")
    np.testing.assert_array_equal(u8, np.array([orc.round_bf16(v) for v in u64.ravel()]).reshape(u64.shape))
    np.testing.assert_array_equal(s8, s64.astype(np.float32).astype(np.float64))


def test_zero_strength_or_zero_output_is_identity(orc):
    X = inputs.make_gr_inputs(10, 4, 48, 4, "bf16", seed=7, n_param_sets=1)
    R0 = X.X.double().numpy()
    s = np.random.default_rng(0).uniform(0, 2, size=(10, 4))
    np.testing.assert_array_equal(orc.write(X.X, X.y, np.zeros((10, 4))), R0)
    np.testing.assert_array_equal(orc.write(X.X, np.zeros((10, 48)), s), R0)


# ---------------------------------------------------------------- P5: the two-branch example

@pytest.mark.parametrize("k,alpha,omega", [(1.5, 2.0, 3.0), (-0.7, 5.0, -1.0), (3.0, -4.0, 0.25)])
def test_two_branch_example_closed_form(orc, k, alpha, omega):
    """Normalised branches (1,0) and (0,1); the first branch's gate favours
    dimension 1 and the second's dimension 2.  With a rank-1 gate
    W_down = [k,0,0,k], W_up = [a,-a,-a,a]^T:  z = k, t = a SiLU(k),
    G_1 = (s(t), s(-t)), G_2 = (s(-t), s(t)), u = (s(t)/2, s(t)/2);
    W_write = [[w,0,0,0],[0,0,0,-w]] gives s = (2 s(w/2), 2 s(-w/2))."""
    R = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    g = np.full((2, 2), 1 / math.sqrt(2))
    wd = np.array([[k, 0, 0, k]], dtype=float)
    wu = np.array([[alpha], [-alpha], [-alpha], [alpha]])
    ww = np.array([[omega, 0, 0, 0], [0, 0, 0, -omega]], dtype=float)
    u, s, rho, G = orc.read(R, g, wd, wu, ww, eps=0.0, dtype="f64", detail=True)
    t = alpha * k * sig(k)
    np.testing.assert_allclose(G[0], [[sig(t), sig(-t)], [sig(-t), sig(t)]], rtol=1e-14)
    np.testing.assert_allclose(u[0], [sig(t) / 2, sig(t) / 2], rtol=1e-14)
    np.testing.assert_allclose(s[0], [2 * sig(omega / 2), 2 * sig(-omega / 2)], rtol=1e-14)
    assert abs(s[0].sum() - 2.0) < 1e-14


# ---------------------------------------------------------------- one-hot weights pin layouts

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_hot_weights_pin_vec_order_and_layouts(orc, seed):
    """W_down [r][n*d], W_up [n*d][r], W_write [n][n*d] with one non-zero each:
    only that entry's path is active, so u and s have simple closed forms.
    A transposed operand or a wrong vec index moves the active entry."""
    rng = np.random.default_rng(10 + seed)
    N, n, d, r = 4, 3, 5, 4
    R = rng.standard_normal((N, n, d)) * np.array([1.0, 0.5, 2.0])[None, :, None]
    g = 1 + 0.1 * rng.standard_normal((n, d))
    k0, j0, j1, j2, i0 = rng.integers(r), rng.integers(n * d), rng.integers(n * d), \
        rng.integers(n * d), rng.integers(n)
    beta, alpha, omega = 2.5, -3.0, 1.7
    wd = np.zeros((r, n * d)); wd[k0, j1] = beta
    wu = np.zeros((n * d, r)); wu[j0, k0] = alpha
    ww = np.zeros((n, n * d)); ww[i0, j2] = omega
    u, s = orc.read(R, g, wd, wu, ww, eps=1e-6, dtype="f64")
    for t in range(N):
        rh = np.stack([rmsnorm_lib(R[t, i], g[i], 1e-6) for i in range(n)])  # [n, d]
        v = rh.reshape(-1)
        zk = beta * v[j1] / n
        ell = alpha * zk * sig(zk)
        # G == 1/2 everywhere except entry j0, where it is sigmoid(ell)
        u_ref = rh.sum(0) / (2 * n)
        u_ref[j0 % d] += (sig(ell) - 0.5) * rh[j0 // d, j0 % d] / n
        s_ref = np.ones(n); s_ref[i0] = 2 * sig(omega * v[j2] / n)
        np.testing.assert_allclose(u[t], u_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(s[t], s_ref, rtol=1e-14)


def test_unit_gate_is_branch_mean(orc):
    rng = np.random.default_rng(20)
    R = rng.standard_normal((3, 4, 8))
    g = 1 + 0.1 * rng.standard_normal((4, 8))
    u, _ = orc.read(R, g, None, None, None, dtype="f64")
    for t in range(3):
        ref = np.mean([rmsnorm_lib(R[t, i], g[i], 1e-6) for i in range(4)], axis=0)
        np.testing.assert_allclose(u[t], ref, rtol=1e-13)


def test_mean_state_write_is_special_case(orc):
    """Write rows tiled [w, w, ..., w] give s_i = 2 sigmoid(w_i . mean_j R-hat_j)."""
    rng = np.random.default_rng(21)
    n, d = 4, 6
    R = rng.standard_normal((2, n, d))
    g = np.ones((n, d))
    w = 0.5 * rng.standard_normal((n, d))
    ww = np.tile(w, (1, n))
    _, s = orc.read(R, g, None, None, ww, dtype="f64")
    for t in range(2):
        mean = np.mean([rmsnorm_lib(R[t, i], g[i], 1e-6) for i in range(n)], axis=0)
        np.testing.assert_allclose(s[t], [2 * sig(w[i] @ mean) for i in range(n)], rtol=1e-13)


# ---------------------------------------------------------------- P6 / P7: invariants

def test_branch_permutation_equivariance(orc):
    """Branches are exchangeable: permuting them (state rows, gains, the column
    blocks of W_down and W_write, the row blocks of W_up and the rows of W_write)
    leaves u unchanged and permutes s and the written state."""
    X = inputs.make_gr_inputs(6, 4, 16, 6, "f32", seed=22, n_param_sets=1, w_std=0.3)
    p = X.params[0]
    perm = [2, 0, 3, 1]
    n, d = 4, 16
    cols = np.concatenate([np.arange(i * d, (i + 1) * d) for i in perm])
    Rp = X.X[:, perm]
    gp = p.gamma[perm]
    wdp = p.w_down[:, cols]
    wup = p.w_up[cols]
    wwp = p.w_write[perm][:, cols]
    u, s = orc.read(X.X, p.gamma, p.w_down, p.w_up, p.w_write, dtype="f64")
    up, sp = orc.read(Rp, gp, wdp, wup, wwp, dtype="f64")
    np.testing.assert_allclose(up, u, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sp, s[:, perm], rtol=1e-13)
    np.testing.assert_allclose(orc.write(Rp, X.y, sp, "f64"),
                               orc.write(X.X, X.y, s, "f64")[:, perm], rtol=1e-13, atol=1e-15)


def test_branch_scale_invariance(orc):
    """eq:rms divides each branch by its own RMS, so with eps = 0 scaling branch
    i by c_i > 0 leaves the read unchanged (the prefill workload uses such
    scales)."""
    X = inputs.make_gr_inputs(5, 4, 32, 8, "f32", seed=23, n_param_sets=1, w_std=0.2)
    p = X.params[0]
    c = torch.tensor([1.0, 0.5, 2.0, 3.0], dtype=torch.float64)[None, :, None]
    u, s = orc.read(X.X, p.gamma, p.w_down, p.w_up, p.w_write, eps=0.0, dtype="f64")
    u2, s2 = orc.read(X.X.double() * c, p.gamma, p.w_down, p.w_up, p.w_write, eps=0.0,
                      dtype="f64")
    np.testing.assert_allclose(u2, u, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s2, s, rtol=1e-13)


# ---------------------------------------------------------------- P8 / P9: chain closed forms

def _chain_inputs(L=5, N=6, n=4, d=32, r=8):
    return inputs.make_gr_inputs(N, n, d, r, "bf16", seed=24, n_param_sets=L, with_y=False,
                                 w_std=0.2)


def test_branch_accumulator_closed_form(orc):
    """No branch mixing, so R_c^(v) = R_c^(0) + sum_{u<v} s_c^(u) y^(u) (eq:rcv),
    and x_L = x_0 + sum of the updates (residual-stream unrolling)."""
    X = _chain_inputs()
    R, ss, ys = orc.chain(X.X, X.params, dtype="f64", record=True)
    acc = X.X.double().numpy().copy()
    for s, y in zip(ss, ys):
        acc += s[:, :, None] * y[:, None, :]
    np.testing.assert_allclose(R, acc, rtol=1e-13, atol=1e-13)
    assert len(ss) == len(X.params)


def test_contribution_decomposition_is_exact(orc):
    """eq:auv: the read of block v splits exactly into the contribution of the
    initial state and of every earlier block's write."""
    X = _chain_inputs(L=4)
    n = X.n
    _, ss, ys = orc.chain(X.X, X.params, dtype="f64", record=True)
    R0 = X.X.double().numpy()
    v = 3
    Rv = R0 + sum(ss[u][:, :, None] * ys[u][:, None, :] for u in range(v))
    p = X.params[v]
    u_v, _, rho, G = orc.read(Rv, p.gamma, p.w_down, p.w_up, p.w_write, dtype="f64", detail=True)
    gam = p.gamma.double().numpy()[None]
    coef = G * gam * rho[:, :, None] / n                         # [N, n, d]
    parts = [(coef * R0).sum(1)]
    parts += [(coef * ss[u][:, :, None] * ys[u][:, None, :]).sum(1) for u in range(v)]
    np.testing.assert_allclose(sum(parts), u_v, rtol=1e-12, atol=1e-14)


def test_fused_is_write_then_read(orc):
    X = inputs.make_gr_inputs(8, 4, 64, 16, "bf16", seed=25, n_param_sets=2)
    p0, p1 = X.params
    _, s0 = orc.read(X.X, p0.gamma, p0.w_down, p0.w_up, p0.w_write)
    Rf, uf, sf = orc.fused(X.X, X.y, s0, p1.gamma, p1.w_down, p1.w_up, p1.w_write)
    Rw = orc.write(X.X, X.y, s0)
    u2, s2 = orc.read(Rw, p1.gamma, p1.w_down, p1.w_up, p1.w_write)
    np.testing.assert_array_equal(Rf, Rw)
    np.testing.assert_array_equal(uf, u2)
    np.testing.assert_array_equal(sf, s2)


def test_tanh_standin_vs_library(orc):
    u = np.random.default_rng(26).standard_normal(1000) * 3
    y = orc.tanh_standin(u, dtype="f64")
    np.testing.assert_allclose(y, 0.1 * np.tanh(u), rtol=1e-15, atol=1e-17)


def test_scalar_brute_force(orc):
    """n=1, d=1, r=1 by hand: R-hat = g R / sqrt(R^2 + eps), z = wd R-hat,
    G = sigmoid(wu SiLU(z)), u = G R-hat, s = 2 sigmoid(ww R-hat)."""
    for Rv, gv, wd, wu, ww, eps in [(0.7, 1.1, 0.9, -1.3, 0.4, 0.01), (-2.0, 0.8, -1.2, 2.0, 3.0, 0.5)]:
        u, s = orc.read(np.array([[[Rv]]]), np.array([[gv]]), np.array([[wd]]),
                        np.array([[wu]]), np.array([[ww]]), eps=eps, dtype="f64")
        rh = gv * Rv / math.sqrt(Rv * Rv + eps)
        z = wd * rh
        G = sig(wu * z * sig(z))
        assert abs(u[0, 0] - G * rh) < 1e-15
        assert abs(s[0, 0] - 2 * sig(ww * rh)) < 1e-15


# ---------------------------------------------------------------- variants on the same state
# "Paper reading: Qwen3.8 Flash Next", part 2: sec. 1 (AltUp-style static read
# eq:input, round-robin write eq:output), sec. 6 (eq:rcv: every branch starts at
# the embedding); "... architecture notes, 06 Residual", sec. 3 (per-channel
# write tried).  Collapse: sum of the branches, then RMSNorm (a reading).

def _bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g, dtype=torch.float64) * std).to(torch.bfloat16)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_expand_copies_the_embedding_into_every_branch(orc, dtype):
    e = _bf16((9, 48), 1.5, 1)
    R = orc.expand(e, 4, dtype)
    want = e.double() if dtype == "bf16" else e.float().clamp(-448, 448).to(torch.float8_e4m3fn).double()
    for i in range(4):
        np.testing.assert_array_equal(R[:, i, :], want.numpy())
    # then a unit-gate read of identical branches (gains 1) is RMSNorm(e)
    gamma = np.ones((4, 48))
    u, s = orc.read(R, gamma, None, None, None, 1e-6, "f64")
    np.testing.assert_allclose(u, rmsnorm_lib(R[:, 0, :], np.ones(48), 1e-6), rtol=1e-13)
    assert np.all(s == 1.0)


def test_static_read_closed_forms(orc):
    R = _bf16((11, 4, 40), 1.0, 2).double()
    for k in range(4):   # a one-hot h picks one branch exactly
        h = np.eye(4)[k]
        np.testing.assert_array_equal(orc.static_read(R, h, "bf16"), R[:, k, :].numpy())
    # the branch mean, stored as bf16: torch's mean in fp64, rounded to nearest even
    u = orc.static_read(R, np.full(4, 0.25), "bf16")
    np.testing.assert_array_equal(u, R.mean(dim=1).to(torch.bfloat16).double().numpy())
    # linear in h, exactly, before the store
    h1, h2 = np.array([0.5, -1.0, 2.0, 0.25]), np.array([1.0, 0.5, -0.75, 3.0])
    a = orc.static_read(R, h1, "f64") + orc.static_read(R, h2, "f64")
    np.testing.assert_allclose(orc.static_read(R, h1 + h2, "f64"), a, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("layer", [0, 1, 5, 11])
def test_round_robin_write_touches_one_branch(orc, layer):
    R = _bf16((7, 4, 32), 1.0, 3)
    y = _bf16((7, 32), 0.3, 4)
    R2 = orc.round_robin_write(R, y, layer, "bf16")
    k = layer % 4
    for i in range(4):
        if i == k:   # fp32 add, then bf16 round to nearest even (torch's casts)
            want = (R[:, i, :].float() + y.float()).to(torch.bfloat16).double().numpy()
        else:
            want = R[:, i, :].double().numpy()
        np.testing.assert_array_equal(R2[:, i, :], want)


def test_per_channel_write_closed_forms(orc):
    R = _bf16((6, 4, 24), 1.0, 5)
    y = _bf16((6, 24), 0.2, 6)
    s = torch.rand(4, 24, generator=torch.Generator().manual_seed(7), dtype=torch.float64).float() * 2
    got = orc.write_per_channel(R, y, s, "bf16")
    # exact product and sum in fp64, rounded to fp32 then bf16 (torch's casts)
    exact = R.double() + s.double()[None] * y.double()[:, None, :]
    np.testing.assert_array_equal(got, exact.float().to(torch.bfloat16).double().numpy())
    # strengths constant along channels are the per-branch scalar write
    sb = torch.tensor([0.5, 1.25, 2.0, 0.0]).float()
    got2 = orc.write_per_channel(R, y, sb[:, None].expand(4, 24), "bf16")
    np.testing.assert_array_equal(got2, orc.write(R, y, sb[None].expand(6, 4), "bf16"))


def test_collapse_closed_forms(orc):
    w = (1 + 0.05 * torch.randn(40, generator=torch.Generator().manual_seed(8), dtype=torch.float64)).numpy()
    R = _bf16((5, 1, 40), 1.0, 9).double().numpy()
    # one branch: the library RMSNorm
    np.testing.assert_allclose(orc.collapse(R, w, 1e-6, "f64"), rmsnorm_lib(R[:, 0, :], w, 1e-6), rtol=1e-13)
    # four branches: RMSNorm of their sum
    R4 = _bf16((5, 4, 40), 1.0, 10).double().numpy()
    np.testing.assert_allclose(orc.collapse(R4, w, 1e-6, "f64"), rmsnorm_lib(R4.sum(axis=1), w, 1e-6), rtol=1e-13)
    # expand then collapse is RMSNorm(e) when eps = 0 (scale invariance: sum = n e)
    e = _bf16((5, 40), 0.7, 11)
    out = orc.collapse(orc.expand(e, 4, "bf16"), w, 0.0, "f64")
    np.testing.assert_allclose(out, rmsnorm_lib(e.double().numpy(), w, 0.0), rtol=1e-13)
