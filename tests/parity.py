"""Parity helpers: compare GPU results with the fp64 oracle's.

Tolerances (written here, used by every GPU parity test):
  * fp32 state:  max |g - o| <= 1e-5 * RMS(o), per output tensor.
  * bf16 state (and u / y with an e4m3 state):
    |g - o| <= 2e-2 * max(|o|, RMS(o)/16) element by element (the per-element
    relative bound with a floor near zero), and relative L2 error
    ||g - o|| / ||o|| <= 4e-3, with fp32 accumulation on the GPU.  Also
    reported: max|g-o|/RMS(o).  (An earlier form also allowed the combine's
    term scale (1/n) sum_i |G_i R-hat_i| in the per-element bound; measured on
    every GPU check, no element needed it, so it is gone.)
  * written state (eq:write): bit for bit (check_exact).  Both sides form
    R + s y in fp32 (the exact value rounded once, as one fp32 FMA does) and
    store that rounded to the state dtype.
  * state written by the HC / mHC write (check_sum_store): R'_i is a sum of
    n + 1 products, formed in fp32 on the GPU and exactly in the oracle, then
    rounded once to the state dtype, so the two may differ by the fp32 sum's
    error and one rounding: |g - o| <= ulp(max(|g|, |o|)) + (n + 2) 2^-24 T,
    T = sum_j |H_res_ij R_j| + |H_comb_i y| (ulp of the state dtype).
  * chained bf16 state after L sublayers (check_chain): each stored value is
    rounded L times, and a rounding decision that differs between the two
    sides (a pre-rounding difference of 1e-7 lands on a bf16 rounding
    boundary) moves that element by one ulp for good; such flips cascade
    through y = F(u).  So: every element within 6e-2 * max(|o|, A), at least
    99.9 % of elements within 2e-2 * max(|o|, A), relative L2 error <= 2e-3,
    where A = |R^(0)| + sum_u |s^(u) y^(u)| (eq:rcv); the per-element A13
    figures (against max(|o|, RMS/16)) are reported beside them.
"""
import numpy as np
import torch

# Every check's statistics, for the session summary (tests/conftest.py):
# (name, dtype, max|g-o|/RMS(o), relative L2, elements past the A13 bound
# without the combine scale A, elements compared).
RECORDS = []


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def check(name: str, got, ref, dtype: str, rms=None):
    """Assert ``got`` (GPU) matches ``ref`` (oracle) at the stated tolerance.

    ``rms`` overrides the RMS used for the floor (e.g. the RMS of the whole
    output when only sampled tokens are compared)."""
    g, o = to64(got), to64(ref)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    if g.size == 0:
        return {}
    rms = float(np.sqrt(np.mean(o * o))) if rms is None else float(rms)
    err = np.abs(g - o)
    stats = {"max_abs": float(err.max()), "max_over_rms": float(err.max() / max(rms, 1e-300)),
             "rel_l2": float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))}
    strict_over = int((err > 2e-2 * np.maximum(np.abs(o), rms / 16)).sum()) if dtype != "f32" else 0
    stats["strict_over"] = strict_over
    RECORDS.append((name, dtype, stats["max_over_rms"], stats["rel_l2"], strict_over, int(g.size)))
    if dtype == "f32":
        assert err.max() <= 1e-5 * rms, f"{name}: fp32 max err {err.max():.3e} > 1e-5*RMS {rms:.3e}"
    else:
        # A13: relative L2 error of a bf16-stored result within ~3 half-ulps
        assert stats["rel_l2"] <= 4e-3, f"{name}: relative L2 error {stats['rel_l2']:.3e} > 4e-3"
        bound = 2e-2 * np.maximum(np.abs(o), rms / 16)
        bad = err > bound
        if bad.any():
            k = int(np.argmax(err / bound))
            idx = np.unravel_index(k, err.shape)
            raise AssertionError(f"{name}: {int(bad.sum())} elements outside 2e-2 rel (worst at "
                                 f"{idx}: gpu {g[idx]!r} oracle {o[idx]!r}); stats {stats}")
    return stats


def check_exact(name: str, got, ref):
    """Assert bit-for-bit equality of a stored tensor with the oracle's value
    (the oracle returns the stored values widened to fp64)."""
    g, o = to64(got), to64(ref)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    diff = g != o
    if diff.any():
        idx = tuple(int(v) for v in np.argwhere(diff)[0])
        raise AssertionError(f"{name}: {int(diff.sum())} of {diff.size} elements differ "
                             f"(first at {idx}: gpu {g[idx]!r} oracle {o[idx]!r})")


def _ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    bits = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - (bits - 1))


def check_sum_store(name: str, got, ref, terms, n: int, dtype: str):
    """The HC write's criterion stated in the module docstring; ``terms`` is T."""
    g, o, T = to64(got), to64(ref), to64(terms)
    assert g.shape == o.shape == T.shape, f"{name}: shapes {g.shape} {o.shape} {T.shape}"
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    err = np.abs(g - o)
    bound = _ulp(np.maximum(np.abs(g), np.abs(o)), dtype) + (n + 2) * 2.0 ** -24 * T
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 1.0
    exact = float((err == 0).mean()) if o.size else 1.0
    RECORDS.append((name, dtype + "-hc-state", float(err.max() / max(rms, 1e-300)) if o.size else 0.0,
                    float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300)), 0, int(g.size)))
    bad = err > bound
    if bad.any():
        idx = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} elements beyond one rounding "
                             f"(first at {idx}: gpu {g[idx]!r} oracle {o[idx]!r} bound {bound[idx]:.3e})")
    return {"exact_fraction": exact}


def sample_tokens(N: int, k: int, seed: int = 0) -> np.ndarray:
    """A sorted sample of k token indices including the first and last ones."""
    if N <= k:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(2, N - 2), size=k - 4, replace=False)
    return np.unique(np.concatenate([[0, 1, N - 2, N - 1], mid]))


def combine_scale(R, gamma, rho, G) -> np.ndarray:
    """A for u: (1/n) sum_i |G_i (.) gamma_i (.) R_i| rho_i, from the oracle's
    stored state R [N,n,d], gains, 1/rms per branch and gate G."""
    R, gamma, rho, G = to64(R), to64(gamma), to64(rho), to64(G)
    n = R.shape[1]
    return np.abs(G * gamma[None] * R * rho[:, :, None]).sum(1) / n


def check_chain(name: str, got, ref, scale):
    """The chained-state criterion stated in the module docstring."""
    g, o, A = to64(got), to64(ref), to64(scale)
    assert g.shape == o.shape == A.shape
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    err = np.abs(g - o)
    q = err / np.maximum(np.abs(o), A)
    rms = float(np.sqrt(np.mean(o * o)))
    strict = err / np.maximum(np.abs(o), rms / 16)
    rel_l2 = float(np.linalg.norm(g - o) / np.linalg.norm(o))
    frac = float((q > 2e-2).mean())
    stats = {"max_err_over_scale": float(q.max()), "frac_over_2e-2": frac, "rel_l2": rel_l2,
             "a13_max_ratio": float(strict.max()), "a13_frac_over_2e-2": float((strict > 2e-2).mean())}
    RECORDS.append((name, "bf16-chain", float(err.max() / max(rms, 1e-300)), rel_l2,
                    int((strict > 2e-2).sum()), int(g.size)))
    assert q.max() <= 6e-2, f"{name}: element off by {q.max():.3e} of its scale; {stats}"
    assert frac <= 1e-3, f"{name}: {frac:.2e} of elements beyond 2e-2; {stats}"
    assert rel_l2 <= 2e-3, f"{name}: relative L2 error {rel_l2:.2e}; {stats}"
    return stats
