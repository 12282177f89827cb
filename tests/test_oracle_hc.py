"""Pins of the oracle's Hyper-Connections (HC) and mHC functions against what the
pages and the mathematics fix, independently of the oracle's own code.

Sources: "Paper reading: Qwen3.8 Flash Next", part 2 (Residual), sec. 1 (the
AltUp-style widened stream, eq:input / eq:output) and sec. 2 (Hyper-Connections:
eq:block, eq:mix, eq:combine; the static terms e_(l mod n), 1, I with W = 0 give
back the Pre-Norm network, and with the dynamic terms kept at zero the AltUp
variant); "DepthBench", sec. 2.5 (mHC: sigmoid reads, twice-sigmoid writes,
20 Sinkhorn-Knopp iterations to an approximately doubly stochastic matrix).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle

EPS = 1e-6


def rms_norm_lib(x, w, eps=EPS):
    """torch's own RMSNorm in float64 (a library routine, not the oracle)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return torch.nn.functional.rms_norm(t, (t.shape[-1],), torch.from_numpy(w), eps).numpy()


def hc_params(rng, n, d, w_scale=0.5, lam=(0.7, 1.1, 0.9), static=None):
    g = 1.0 + 0.1 * rng.standard_normal((n, d))
    w = 1.0 + 0.1 * rng.standard_normal(d)
    P = w_scale * rng.standard_normal((n + 2, d))
    hs = rng.standard_normal(2 * n + n * n) if static is None else static
    return g, w, P, hs, np.asarray(lam, dtype=np.float64)


# ---------------------------------------------------------------- Sinkhorn-Knopp

def test_sinkhorn_two_by_two_closed_form():
    """A positive 2x2 matrix [[a, b], [c, d]] has the doubly stochastic scaling
    [[p, 1-p], [1-p, p]] with p / (1-p) = sqrt(ad / bc); the iteration converges
    to it geometrically (within 1e-9 after 20 steps for these entries)."""
    rng = np.random.default_rng(1)
    for _ in range(20):
        L = rng.uniform(-1.0, 1.0, (2, 2))
        a, b, c, d = np.exp(L).ravel()
        p = np.sqrt(a * d) / (np.sqrt(a * d) + np.sqrt(b * c))
        want = [[p, 1 - p], [1 - p, p]]
        np.testing.assert_allclose(oracle.sinkhorn(L, 20), want, rtol=0, atol=1e-9)
        np.testing.assert_allclose(oracle.sinkhorn(L, 60), want, rtol=0, atol=1e-14)


def test_sinkhorn_rank_one_is_uniform_after_one_iteration():
    """exp(a_i + b_j) is rank one: one row-then-column scaling gives 1/n exactly."""
    rng = np.random.default_rng(2)
    for n in (1, 2, 3, 4, 8):
        L = rng.standard_normal(n)[:, None] + rng.standard_normal(n)[None, :]
        for iters in (1, 20):
            np.testing.assert_allclose(oracle.sinkhorn(L, iters), np.full((n, n), 1.0 / n),
                                       rtol=0, atol=1e-15)


def test_sinkhorn_zero_iterations_is_exp():
    L = np.random.default_rng(3).standard_normal((4, 4))
    np.testing.assert_allclose(oracle.sinkhorn(L, 0), np.exp(L), rtol=4e-16, atol=0)


def test_sinkhorn_fixed_point_and_doubly_stochastic():
    """A doubly stochastic matrix is left unchanged; a generic one ends with
    columns summing to 1 (the last step) and rows within the convergence error."""
    D = 0.7 * np.eye(4) + 0.3 * np.full((4, 4), 0.25)
    np.testing.assert_allclose(oracle.sinkhorn(np.log(D), 20), D, rtol=0, atol=1e-15)
    rng = np.random.default_rng(4)
    for n in (2, 3, 4, 6):
        M = oracle.sinkhorn(rng.uniform(-2, 2, (n, n)), 20)
        np.testing.assert_allclose(M.sum(axis=0), 1.0, rtol=0, atol=1e-14)
        np.testing.assert_allclose(M.sum(axis=1), 1.0, rtol=0, atol=1e-6)
        assert (M > 0).all()


def test_sinkhorn_permutation_equivariant():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((4, 4))
    p, q = rng.permutation(4), rng.permutation(4)
    np.testing.assert_allclose(oracle.sinkhorn(L[p][:, q], 20), oracle.sinkhorn(L, 20)[p][:, q],
                               rtol=0, atol=1e-14)


# ---------------------------------------------------------------- HC reductions

@pytest.mark.parametrize("mode", ["hc"])
def test_hc_static_identity_is_pre_norm(mode):
    """Static terms e_k, 1, I and W = 0 on equal branches: the block input is
    RMSNorm of the shared branch and every branch receives r + y, which is
    x + F(Norm(x)) of the Pre-Norm network (paper reading, sec. 2)."""
    rng = np.random.default_rng(10)
    N, n, d, k = 3, 4, 16, 2
    r = rng.standard_normal((N, d))
    R = np.repeat(r[:, None, :], n, axis=1)
    y = rng.standard_normal((N, d))
    g, w, _, _, lam = hc_params(rng, n, d)
    hs = np.concatenate([np.eye(n)[k], np.ones(n), np.eye(n).ravel()])
    u, coeff = oracle.hc_read(R, g, w, np.zeros((n + 2, d)), hs, lam, mode, dtype="f64")
    np.testing.assert_allclose(u, rms_norm_lib(r, w), rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(coeff, np.tile(np.concatenate([np.ones(n), np.eye(n).ravel()]), (N, 1)))
    R2 = oracle.hc_write(R, y, coeff, dtype="f64")
    np.testing.assert_array_equal(R2, np.repeat((r + y)[:, None, :], n, axis=1))
    h, out = oracle.add_rmsnorm(r, y, w, dtype="f64")
    np.testing.assert_array_equal(h, R2[:, 0])


def test_hc_static_is_altup():
    """Dynamic terms zero, H_res = I, H_comb = e_(l mod n): the read is
    x = sum_i h_i R_i (eq:input) and the write adds y to one branch (eq:output)."""
    rng = np.random.default_rng(11)
    N, n, d, layer = 5, 4, 24, 7
    R = rng.standard_normal((N, n, d))
    y = rng.standard_normal((N, d))
    h = rng.standard_normal(n)
    g, w, P, _, _ = hc_params(rng, n, d)
    hs = np.concatenate([h, np.eye(n)[layer % n], np.eye(n).ravel()])
    u, coeff = oracle.hc_read(R, g, w, P, hs, np.zeros(3), "hc", dtype="f64")
    x = np.einsum("i,tic->tc", h, R)
    np.testing.assert_allclose(u, rms_norm_lib(x, w), rtol=1e-13, atol=1e-14)
    R2 = oracle.hc_write(R, y, coeff, dtype="f64")
    want = R.copy()
    want[:, layer % n] += y
    np.testing.assert_array_equal(R2, want)


def test_mhc_one_branch_is_rmsnorm_and_sigmoid_write():
    """n = 1, eps = 0: the read weight is a positive scalar, so u = RMSNorm(R);
    H_res is the 1x1 Sinkhorn result 1, so the write is R + 2 sigmoid(.) y."""
    rng = np.random.default_rng(12)
    N, d = 4, 32
    R = rng.standard_normal((N, 1, d))
    y = rng.standard_normal((N, d))
    g, w, P, hs, lam = hc_params(rng, 1, d)
    u, coeff = oracle.hc_read(R, g, w, P, hs, lam, "mhc", eps=0.0, dtype="f64")
    np.testing.assert_allclose(u, rms_norm_lib(R[:, 0], w, eps=0.0), rtol=1e-13, atol=1e-14)
    assert np.all(coeff[:, 1] == 1.0)
    assert np.all((coeff[:, 0] > 0) & (coeff[:, 0] < 2))


def test_mhc_operators_are_nonnegative_and_conserve_the_branch_sum():
    """mHC: H_mix in (0,1), H_comb in (0,2), H_res doubly stochastic; since its
    columns sum to 1, the write conserves sum_i R_i up to (sum_i H_comb_i) y."""
    rng = np.random.default_rng(13)
    N, n, d = 6, 4, 40
    R = rng.standard_normal((N, n, d))
    y = rng.standard_normal((N, d))
    g, w, P, hs, lam = hc_params(rng, n, d)
    u, coeff, hm = oracle.hc_read(R, g, w, P, hs, lam, "mhc", detail=True, dtype="f64")
    Hc, Hr = coeff[:, :n], coeff[:, n:].reshape(N, n, n)
    assert ((hm > 0) & (hm < 1)).all() and ((Hc > 0) & (Hc < 2)).all()
    np.testing.assert_allclose(Hr.sum(axis=1), 1.0, rtol=0, atol=1e-6)   # columns: the last step
    row_err = np.abs(Hr.sum(axis=2) - 1).max()
    assert row_err < 0.05        # rows: approximately, after 20 iterations on logits of +-6
    L = np.random.default_rng(16).uniform(-6, 6, (4, 4))
    errs = [np.abs(oracle.sinkhorn(L, k).sum(axis=1) - 1).max() for k in (5, 20, 80, 320)]
    assert errs[0] > errs[1] > errs[2] > errs[3] and errs[3] < 1e-9
    R2 = oracle.hc_write(R, y, coeff, dtype="f64")
    lhs = R2.sum(axis=1)
    rhs = np.einsum("tj,tjc->tc", Hr.sum(axis=1), R) + Hc.sum(axis=1)[:, None] * y
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lhs, R.sum(axis=1) + Hc.sum(axis=1)[:, None] * y, rtol=0, atol=1e-4)


@pytest.mark.parametrize("mode", ["hc", "mhc"])
def test_hc_permuting_branches(mode):
    """Branches are exchangeable: permuting them together with every per-branch
    parameter (gains, static terms, the columns of W_res) leaves u unchanged and
    permutes H_comb and H_res (P H P^T) and the written state."""
    rng = np.random.default_rng(14)
    N, n, d = 3, 4, 16
    R = rng.standard_normal((N, n, d))
    y = rng.standard_normal((N, d))
    g, w, P, hs, lam = hc_params(rng, n, d)
    p = np.array([2, 0, 3, 1])
    hs_p = np.concatenate([hs[:n][p], hs[n:2 * n][p], hs[2 * n:].reshape(n, n)[p][:, p].ravel()])
    P_p = np.concatenate([P[:2], P[2:][p]])
    u, c = oracle.hc_read(R, g, w, P, hs, lam, mode, dtype="f64")
    u2, c2 = oracle.hc_read(R[:, p], g[p], w, P_p, hs_p, lam, mode, dtype="f64")
    np.testing.assert_allclose(u2, u, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(c2[:, :n], c[:, :n][:, p], rtol=1e-7)
    Hr, Hr2 = c[:, n:].reshape(N, n, n), c2[:, n:].reshape(N, n, n)
    np.testing.assert_allclose(Hr2, Hr[:, p][:, :, p], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(oracle.hc_write(R[:, p], y, c2, dtype="f64"),
                               oracle.hc_write(R, y, c, dtype="f64")[:, p], rtol=1e-12, atol=1e-12)


# ------------------------------------------------- brute force vs a matrix form

def numpy_sinkhorn(L, iters):
    M = np.exp(L)
    for _ in range(iters):
        M = M / M.sum(axis=-1, keepdims=True)
        M = M / M.sum(axis=-2, keepdims=True)
    return M


def numpy_hc(R, y, coeff_in, g, w, P, hs, lam, mode, iters=20, eps=EPS):
    """The same definitions written as whole-array numpy (einsum) operations."""
    N, n, d = R.shape
    if y is not None:
        Hc_in, Hr_in = coeff_in[:, :n], coeff_in[:, n:].reshape(N, n, n)
        R = np.einsum("tij,tjc->tic", Hr_in, R) + Hc_in[:, :, None] * y[:, None, :]
    rbar = g[None] * R / np.sqrt((R ** 2).mean(axis=-1, keepdims=True) + eps)
    proj = np.einsum("tic,kc->tik", rbar, P)
    sm, sc, sr = hs[:n], hs[n:2 * n], hs[2 * n:].reshape(n, n)
    if mode == "hc":
        hm = sm + lam[0] * np.tanh(proj[:, :, 0])
        hc = sc + lam[1] * np.tanh(proj[:, :, 1])
        hr = sr + lam[2] * np.tanh(proj[:, :, 2:])
    else:
        sig = lambda z: 1.0 / (1.0 + np.exp(-z))
        hm = sig(sm + lam[0] * proj[:, :, 0])
        hc = 2.0 * sig(sc + lam[1] * proj[:, :, 1])
        hr = numpy_sinkhorn(sr + lam[2] * proj[:, :, 2:], iters)
    x = np.einsum("ti,tic->tc", hm, R)
    u = w * x / np.sqrt((x ** 2).mean(axis=-1, keepdims=True) + eps)
    return R, u, np.concatenate([hc, hr.reshape(N, n * n)], axis=1)


CASES = list(itertools.product([1, 2, 3, 4], [1, 2, 3, 8, 16], [1, 3], ["hc", "mhc"]))


@pytest.mark.parametrize("n,d,N,mode", CASES)
def test_hc_bruteforce_matches_matrix_form(n, d, N, mode):
    rng = np.random.default_rng(1000 * n + 10 * d + N)
    R = rng.standard_normal((N, n, d))
    y = rng.standard_normal((N, d))
    g, w, P, hs, lam = hc_params(rng, n, d)
    cin = rng.uniform(0.2, 1.5, (N, n + n * n))
    u, c = oracle.hc_read(R, g, w, P, hs, lam, mode, dtype="f64")
    _, u_np, c_np = numpy_hc(R, None, None, g, w, P, hs, lam, mode)
    np.testing.assert_allclose(u, u_np, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c, c_np, rtol=1e-7, atol=1e-7)   # coeff is stored in fp32
    R2, u2, c2 = oracle.hc_fused(R, y, cin, g, w, P, hs, lam, mode, dtype="f64")
    R2_np, u2_np, c2_np = numpy_hc(R, y, cin, g, w, P, hs, lam, mode)
    np.testing.assert_allclose(R2, R2_np, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(u2, u2_np, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c2, c2_np, rtol=1e-7, atol=1e-7)


def test_hc_bruteforce_has_teeth():
    """A plausible slip in the matrix form (W_res read transposed, i.e. the
    branch index and the output index swapped) is caught by the comparison."""
    rng = np.random.default_rng(77)
    n, d, N = 3, 8, 3
    R = rng.standard_normal((N, n, d))
    g, w, P, hs, lam = hc_params(rng, n, d)
    _, c = oracle.hc_read(R, g, w, P, hs, lam, "hc", dtype="f64")
    _, _, c_np = numpy_hc(R, None, None, g, w, P, hs, lam, "hc")
    Hr_np = c_np[:, n:].reshape(N, n, n)
    c_bad = np.concatenate([c_np[:, :n], Hr_np.transpose(0, 2, 1).reshape(N, n * n)], axis=1)
    assert not np.allclose(c, c_bad, rtol=1e-7, atol=1e-7)


def test_hc_rounding_points():
    """bf16 storage: the written state and u are bf16 values; the coefficients
    are fp32; the write is the exact sum rounded once."""
    rng = np.random.default_rng(15)
    N, n, d = 2, 4, 8
    bf = lambda a: torch.from_numpy(np.asarray(a)).to(torch.bfloat16).double().numpy()
    R = bf(rng.standard_normal((N, n, d)))
    y = bf(rng.standard_normal((N, d)))
    g, w, P, hs, lam = [bf(a) if i < 3 else a for i, a in enumerate(hc_params(rng, n, d))]
    cin = np.float32(rng.uniform(0.2, 1.5, (N, n + n * n))).astype(np.float64)
    R2, u, c = oracle.hc_fused(R, y, cin, g, w, P, hs, lam, "mhc", dtype="bf16")
    exact, _, _ = numpy_hc(R, y, cin, g, w, P, hs, lam, "mhc")
    np.testing.assert_array_equal(R2, bf(exact))
    np.testing.assert_array_equal(u, bf(u))
    np.testing.assert_array_equal(c, np.float32(c).astype(np.float64))
