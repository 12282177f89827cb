"""Brute-force pin of the oracle on tiny shapes with dense random weights.

The oracle (plain loops in C) is compared with a second, independent
formulation of the same equations written here as whole-array numpy
contractions ("Paper reading: Qwen3.8 Flash Next", part 2 Residual, sec. 4:
eq:rms, eq:gate, eq:use_gate, eq:s, eq:write; the fused call is eq:write
followed by the read of the next module, sec. 7).  The two share nothing but
the equations: here the branch stack vec() is a reshape of the [n, d] block,
the projections are einsum contractions over that stacked axis, and the
sigmoid is numpy's.  A transposed weight, a wrong vec index, a dropped 1/n or
a per-branch norm taken over the wrong axis moves results far beyond the
1e-12 agreement asserted, for every n in {1, 2, 3, 4}, d in {1, 2, 3, 8, 16},
r in {0, 1, 2, 5} and N in {1, 3}, with and without a write projection.
Storage dtype "f64" (no store rounding) makes the comparison exact up to the
order of fp64 sums.
"""
import itertools

import numpy as np
import pytest


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def read_matrix(R, gamma, wd, wu, ww, eps):
    """GR read of a [N, n, d] state as array contractions; returns (u, s)."""
    N, n, d = R.shape
    rho = 1.0 / np.sqrt(np.mean(R * R, axis=2, keepdims=True) + eps)   # eq:rms, per branch
    Rhat = gamma[None, :, :] * R * rho
    v = Rhat.reshape(N, n * d)                                          # vec: branches stacked
    if wd is None:
        G = np.ones_like(Rhat)                                          # r = 0: unit gate
    else:
        z = np.einsum("kj,tj->tk", wd, v) / n                           # eq:gate, down projection
        a = z * sigmoid(z)                                              # SiLU
        G = sigmoid(np.einsum("jk,tk->tj", wu, a)).reshape(N, n, d)     # up projection, unvec
    u = np.mean(G * Rhat, axis=1)                                       # eq:use_gate
    if ww is None:
        s = np.ones((N, n))
    else:
        s = 2.0 * sigmoid(np.einsum("ij,tj->ti", ww, v) / n)           # eq:s
    return u, s


CASES = list(itertools.product([1, 2, 3, 4], [1, 2, 3, 8, 16], [0, 1, 2, 5], [1, 3]))


@pytest.mark.parametrize("n,d,r,N", CASES)
def test_oracle_matches_matrix_formulation(orc, n, d, r, N):
    rng = np.random.default_rng(1000 * n + 100 * d + 10 * r + N)
    R = rng.standard_normal((N, n, d)) * rng.uniform(0.3, 3.0, size=(1, n, 1))
    gamma = 1.0 + 0.3 * rng.standard_normal((n, d))
    wd = rng.standard_normal((r, n * d)) if r else None
    wu = rng.standard_normal((n * d, r)) if r else None
    ww = rng.standard_normal((n, n * d))
    y = 0.5 * rng.standard_normal((N, d))
    s_in = rng.uniform(0.0, 2.0, size=(N, n))
    eps = 1e-3
    for w_write in (ww, None):
        u, s = orc.read(R, gamma, wd, wu, w_write, eps=eps, dtype="f64")
        u_m, s_m = read_matrix(R, gamma, wd, wu, w_write, eps)
        scale_u = max(np.abs(u_m).max(), 1e-300)
        assert np.abs(u - u_m).max() <= 1e-12 * scale_u, (u, u_m)
        np.testing.assert_allclose(s, s_m, rtol=1e-12, atol=0)
        # fused: eq:write first (exact in f64), then the read of the stored state
        Rw, uf, sf = orc.fused(R, y, s_in, gamma, wd, wu, w_write, eps=eps, dtype="f64")
        Rw_m = R + s_in[:, :, None] * y[:, None, :]
        np.testing.assert_allclose(Rw, Rw_m, rtol=1e-15, atol=1e-15)
        uf_m, sf_m = read_matrix(Rw_m, gamma, wd, wu, w_write, eps)
        assert np.abs(uf - uf_m).max() <= 1e-12 * max(np.abs(uf_m).max(), 1e-300)
        np.testing.assert_allclose(sf, sf_m, rtol=1e-12, atol=0)


def test_matrix_formulation_is_not_trivially_equal(orc):
    """The pin has teeth: a transposed W_up (same shape when n*d == r) or the
    1/n dropped from the down projection changes u by far more than 1e-12."""
    rng = np.random.default_rng(5)
    n, d, r = 2, 2, 4
    R = rng.standard_normal((3, n, d))
    gamma = 1.0 + 0.3 * rng.standard_normal((n, d))
    wd = rng.standard_normal((r, n * d))
    wu = rng.standard_normal((n * d, r))
    u, _ = orc.read(R, gamma, wd, wu, None, eps=1e-3, dtype="f64")
    u_t, _ = read_matrix(R, gamma, wd, wu.T.copy(), None, 1e-3)
    u_n, _ = read_matrix(R, gamma, wd * n, wu, None, 1e-3)
    assert np.abs(u - u_t).max() > 1e-6
    assert np.abs(u - u_n).max() > 1e-6
