"""fp64 CPU oracle of the Gated Residual read/write path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (``write_gr_read_amd``)
never does.  The arithmetic lives in ``gr_oracle.c`` (plain loops, fp64,
built with ``-O2 -ffp-contract=off``); this file only marshals numpy arrays.

Functions take and return float64 numpy arrays holding the exact stored values
(a bfloat16, float32 or e4m3 input widened to float64 is exact).  Storage
dtypes: "f32", "bf16", "f64" (no rounding at store points, for closed-form
checks), or "fp8" (the branch state in OCP e4m3, saturating at +-448; u, y,
gains and weights in bf16).

Every function follows a passage of the pages:
  read / write / fused  -- "Paper reading: Qwen3.8 Flash Next", part 2
                           (Residual), sec. 4 Gated Residual, eq:rms, eq:gate,
                           eq:use_gate, eq:s, eq:write; sec. 7 for the fusion.
  add_rmsnorm           -- "Residual" (LLM inference), sec. 3.3.
  chain                 -- the same page of the paper reading, sec. 4 (one GR
                           module around each sublayer) and sec. 6 (each branch
                           accumulates the writes, eq:rcv).
  expand                -- the paper reading, sec. 6 (eq:rcv: branches start at
                           the token embedding).
  static_read,          -- the paper reading, sec. 1 (the AltUp-style widened
  round_robin_write        stream: eq:input, eq:output).
  write_per_channel     -- the architecture notes, sec. 3 (a per-channel write
                           was tried); strengths a learned [n, d] parameter.
  collapse              -- read-out after the last block: sum of the branches,
                           then RMSNorm (a reading; the GR pages give none).
  sinkhorn, hc_read,    -- Hyper-Connections and mHC: the paper reading, sec. 2
  hc_write, hc_fused       (eq:block, eq:mix, eq:combine; phi = tanh), and
                           "DepthBench" sec. 2.5 (mHC: sigmoid reads, twice-
                           sigmoid writes, 20 Sinkhorn-Knopp iterations).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gr_oracle.c")
_LIB = os.path.join(_HERE, "libgr_oracle.so")
_DT = {"f32": 0, "bf16": 1, "f64": 2, "fp8": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64, I, D = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.gro_read.argtypes = [I64, I, I, I, D, I, P, P, P, P, P, P, P, P, P]
        lib.gro_write.argtypes = [I64, I, I, I, P, P, P]
        lib.gro_fused.argtypes = [I64, I, I, I, D, I, P, P, P, P, P, P, P, P, P]
        lib.gro_add_rmsnorm.argtypes = [I64, I, D, I, P, P, P, P]
        lib.gro_tanh_standin.argtypes = [I64, I, P, P]
        lib.gro_expand.argtypes = [I64, I, I, I, P, P]
        lib.gro_static_read.argtypes = [I64, I, I, I, P, P, P]
        lib.gro_round_robin_write.argtypes = [I64, I, I, I, I, P, P]
        lib.gro_write_per_channel.argtypes = [I64, I, I, I, P, P, P]
        lib.gro_collapse.argtypes = [I64, I, I, D, I, P, P, P]
        lib.gro_sinkhorn.argtypes = [I, I, P, P]
        lib.gro_hc_read.argtypes = [I64, I, I, I, I, D, I, P, P, P, P, P, P, P, P, P]
        lib.gro_hc_write.argtypes = [I64, I, I, I, P, P, P]
        lib.gro_hc_fused.argtypes = [I64, I, I, I, I, D, I, P, P, P, P, P, P, P, P, P, P]
        for f in (lib.gro_sinkhorn, lib.gro_hc_read, lib.gro_hc_write, lib.gro_hc_fused):
            f.restype = ctypes.c_int
        lib.orc_round_bf16.argtypes = [D]
        lib.orc_round_bf16.restype = D
        lib.orc_round_e4m3.argtypes = [D]
        lib.orc_round_e4m3.restype = D
        for f in (lib.gro_read, lib.gro_write, lib.gro_fused, lib.gro_add_rmsnorm,
                  lib.gro_tanh_standin, lib.gro_expand, lib.gro_static_read,
                  lib.gro_round_robin_write, lib.gro_write_per_channel, lib.gro_collapse):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a, shape=None) -> np.ndarray:
    """float64, C-contiguous copy of a numpy array or CPU torch tensor."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None:
        a = a.reshape(shape)
    return a


def _p(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments")


def round_bf16(x: float) -> float:
    return _load().orc_round_bf16(float(x))


def round_e4m3(x: float) -> float:
    """Nearest OCP e4m3 value, ties to even, saturating at +-448."""
    return _load().orc_round_e4m3(float(x))


def read(R, gamma, w_down, w_up, w_write, eps: float = 1e-6, dtype: str = "bf16",
         detail: bool = False):
    """GR read: returns (u [N,d], s [N,n]) and, with ``detail``, (rho, G)."""
    R = _f64(R)
    N, n, d = R.shape
    gamma = _f64(gamma, (n, d))
    r = 0 if w_down is None else int(np.shape(w_down)[0])
    wd = _f64(w_down, (r, n * d)) if r else None
    wu = _f64(w_up, (n * d, r)) if r else None
    ww = _f64(w_write, (n, n * d))
    u = np.empty((N, d))
    s = np.empty((N, n))
    rho = np.empty((N, n)) if detail else None
    G = np.empty((N, n, d)) if detail else None
    _check(_load().gro_read(N, n, d, r, eps, _DT[dtype], _p(R), _p(gamma), _p(wd), _p(wu),
                            _p(ww), _p(u), _p(s), _p(rho), _p(G)), "read")
    return (u, s, rho, G) if detail else (u, s)


def write(R, y, s, dtype: str = "bf16") -> np.ndarray:
    """GR write: returns R' = R + s_i y per branch (a new array)."""
    R = _f64(R).copy()
    N, n, d = R.shape
    y = _f64(y, (N, d))
    s = _f64(s, (N, n))
    _check(_load().gro_write(N, n, d, _DT[dtype], _p(R), _p(y), _p(s)), "write")
    return R


def fused(R, y, s_in, gamma, w_down, w_up, w_write, eps: float = 1e-6,
          dtype: str = "bf16"):
    """Write of sublayer l then read of sublayer l+1: returns (R', u, s_out)."""
    R = _f64(R).copy()
    N, n, d = R.shape
    y = _f64(y, (N, d))
    s_in = _f64(s_in, (N, n))
    gamma = _f64(gamma, (n, d))
    r = 0 if w_down is None else int(np.shape(w_down)[0])
    wd = _f64(w_down, (r, n * d)) if r else None
    wu = _f64(w_up, (n * d, r)) if r else None
    ww = _f64(w_write, (n, n * d))
    u = np.empty((N, d))
    s = np.empty((N, n))
    _check(_load().gro_fused(N, n, d, r, eps, _DT[dtype], _p(R), _p(y), _p(s_in), _p(gamma),
                             _p(wd), _p(wu), _p(ww), _p(u), _p(s)), "fused")
    return R, u, s


def add_rmsnorm(x, y, w, eps: float = 1e-6, dtype: str = "bf16"):
    """n = 1 fused residual add + RMSNorm: returns (h, out)."""
    x = _f64(x).copy()
    N, d = x.shape
    y = _f64(y, (N, d))
    w = _f64(w, (d,))
    out = np.empty((N, d))
    _check(_load().gro_add_rmsnorm(N, d, eps, _DT[dtype], _p(x), _p(y), _p(w), _p(out)),
           "add_rmsnorm")
    return x, out


def tanh_standin(u, dtype: str = "bf16") -> np.ndarray:
    """The chained workload's elementwise sublayer: y = 0.1 tanh(u)."""
    u = _f64(u)
    y = np.empty_like(u)
    _check(_load().gro_tanh_standin(u.size, _DT[dtype], _p(u), _p(y)), "tanh_standin")
    return y


def expand(e, n: int, dtype: str = "bf16") -> np.ndarray:
    """Every branch starts as the embedding e [N, d] (eq:rcv): returns [N, n, d]."""
    e = _f64(e)
    N, d = e.shape
    R = np.empty((N, n, d))
    _check(_load().gro_expand(N, n, d, _DT[dtype], _p(e), _p(R)), "expand")
    return R


def static_read(R, h, dtype: str = "bf16") -> np.ndarray:
    """AltUp-style static read (eq:input): u = sum_i h_i R_i."""
    R = _f64(R)
    N, n, d = R.shape
    h = _f64(h, (n,))
    u = np.empty((N, d))
    _check(_load().gro_static_read(N, n, d, _DT[dtype], _p(R), _p(h), _p(u)), "static_read")
    return u


def round_robin_write(R, y, layer: int, dtype: str = "bf16") -> np.ndarray:
    """Round-robin write (eq:output): y added to branch layer mod n only."""
    R = _f64(R).copy()
    N, n, d = R.shape
    y = _f64(y, (N, d))
    _check(_load().gro_round_robin_write(N, n, d, int(layer), _DT[dtype], _p(R), _p(y)),
           "round_robin_write")
    return R


def write_per_channel(R, y, s, dtype: str = "bf16") -> np.ndarray:
    """Per-channel write with a learned [n, d] strength: R'_ic = R_ic + s_ic y_c."""
    R = _f64(R).copy()
    N, n, d = R.shape
    y = _f64(y, (N, d))
    s = _f64(s, (n, d))
    _check(_load().gro_write_per_channel(N, n, d, _DT[dtype], _p(R), _p(y), _p(s)),
           "write_per_channel")
    return R


def collapse(R, w, eps: float = 1e-6, dtype: str = "bf16") -> np.ndarray:
    """Read-out of the widened stream: RMSNorm(sum_i R_i; w)."""
    R = _f64(R)
    N, n, d = R.shape
    w = _f64(w, (d,))
    out = np.empty((N, d))
    _check(_load().gro_collapse(N, n, d, eps, _DT[dtype], _p(R), _p(w), _p(out)), "collapse")
    return out


_HC_MODE = {"hc": 0, "mhc": 1}


def sinkhorn(L, iters: int = 20) -> np.ndarray:
    """Sinkhorn-Knopp on exp(L) (n x n): rows then columns scaled to sum 1, per iteration."""
    L = _f64(L)
    n = L.shape[0]
    M = np.empty((n, n))
    _check(_load().gro_sinkhorn(n, int(iters), _p(L), _p(M)), "sinkhorn")
    return M


def _hc_params(n, d, gamma, w_norm, w_proj, h_static, lam):
    return (_f64(gamma, (n, d)), _f64(w_norm, (d,)), _f64(w_proj, (n + 2, d)),
            _f64(h_static, (2 * n + n * n,)), _f64(lam, (3,)))


def hc_read(R, gamma, w_norm, w_proj, h_static, lam, mode: str = "mhc", iters: int = 20,
            eps: float = 1e-6, dtype: str = "bf16", detail: bool = False):
    """HC / mHC read: returns (u [N,d], coeff [N, n+n*n]) and, with ``detail``,
    H_mix [N, n].  coeff holds H_combine then H_res (row-major)."""
    R = _f64(R)
    N, n, d = R.shape
    g, w, P, hs, lm = _hc_params(n, d, gamma, w_norm, w_proj, h_static, lam)
    u = np.empty((N, d))
    coeff = np.empty((N, n + n * n))
    hm = np.empty((N, n)) if detail else None
    _check(_load().gro_hc_read(N, n, d, _HC_MODE[mode], int(iters), eps, _DT[dtype], _p(R), _p(g),
                               _p(w), _p(P), _p(hs), _p(lm), _p(u), _p(coeff), _p(hm)), "hc_read")
    return (u, coeff, hm) if detail else (u, coeff)


def hc_write(R, y, coeff, dtype: str = "bf16") -> np.ndarray:
    """HC / mHC write: R'_i = sum_j H_res[i,j] R_j + H_comb[i] y (a new array)."""
    R = _f64(R).copy()
    N, n, d = R.shape
    y = _f64(y, (N, d))
    coeff = _f64(coeff, (N, n + n * n))
    _check(_load().gro_hc_write(N, n, d, _DT[dtype], _p(R), _p(y), _p(coeff)), "hc_write")
    return R


def hc_fused(R, y, coeff_in, gamma, w_norm, w_proj, h_static, lam, mode: str = "mhc",
             iters: int = 20, eps: float = 1e-6, dtype: str = "bf16"):
    """Write of block l, then the read of block l+1: returns (R', u, coeff_out)."""
    R = _f64(R).copy()
    N, n, d = R.shape
    y = _f64(y, (N, d))
    cin = _f64(coeff_in, (N, n + n * n))
    g, w, P, hs, lm = _hc_params(n, d, gamma, w_norm, w_proj, h_static, lam)
    u = np.empty((N, d))
    cout = np.empty((N, n + n * n))
    _check(_load().gro_hc_fused(N, n, d, _HC_MODE[mode], int(iters), eps, _DT[dtype], _p(R), _p(y),
                                _p(cin), _p(g), _p(w), _p(P), _p(hs), _p(lm), _p(u), _p(cout)),
           "hc_fused")
    return R, u, cout


def chain(X0, params: Sequence, eps: float = 1e-6, dtype: str = "bf16",
          record: bool = False):
    """A stack of len(params) sublayers, each read -> F -> write, where F is the
    stand-in y = 0.1 tanh(u) and consecutive write/read pairs are fused.

    ``params`` holds objects with gamma / w_down / w_up / w_write.  Returns the
    final state and, with ``record``, the lists of (s, y) that were written.
    """
    R = _f64(X0).copy()
    ss: List[np.ndarray] = []
    ys: List[np.ndarray] = []
    p0 = params[0]
    u, s = read(R, p0.gamma, p0.w_down, p0.w_up, p0.w_write, eps, dtype)
    y = tanh_standin(u, dtype)
    for p in params[1:]:
        if record:
            ss.append(s); ys.append(y)
        R, u, s = fused(R, y, s, p.gamma, p.w_down, p.w_up, p.w_write, eps, dtype)
        y = tanh_standin(u, dtype)
    if record:
        ss.append(s); ys.append(y)
    R = write(R, y, s, dtype)
    return (R, ss, ys) if record else R


def parallel_tokens(fn, arrays_by_token: Sequence[np.ndarray], threads: int, **kw):
    """Run ``fn`` over disjoint token ranges in ``threads`` threads (ctypes
    releases the GIL).  Tokens are independent, so results equal one call."""
    N = arrays_by_token[0].shape[0]
    threads = max(1, min(threads, N))
    bounds = np.linspace(0, N, threads + 1).astype(int)
    def run(k):
        lo, hi = bounds[k], bounds[k + 1]
        return fn(*[a[lo:hi] for a in arrays_by_token], **kw)
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(run, range(threads)))
