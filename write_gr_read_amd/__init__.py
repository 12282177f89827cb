"""MI355X-native Gated Residual (GR) read/write path.

Thin Python binding of ``libgr.so`` (the C ABI in ``include/gr.h``).  It only
marshals arguments: checks that tensors live on the GPU with the shapes, dtype
and contiguity the kernels assume, allocates outputs and the workspace with
torch, and passes raw device pointers plus the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is missing the first call raises.

GR ("Paper reading: Qwen3.8 Flash Next", part 2 Residual, sec. 4):
  read   u = (1/n) sum_i G_i (.) RMSNorm(R_i; gamma_i), s = 2 sigmoid(...)
  write  R_i += s_i y
  fused  write of sublayer l, then read of sublayer l+1, in one call (by
         default two kernels over R: the write with the projections, then
         the gated combine reading R' back).
n = 1 fused residual add + RMSNorm: "Residual" (LLM inference), sec. 3.3.
Hyper-Connections / mHC (same paper reading, sec. 2; "DepthBench", sec. 2.5):
  hc_read, hc_write, hc_fused_write_read with an ``HCLayer``.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

__all__ = ["read", "write", "fused_write_read", "residual_add_rmsnorm", "tanh_standin",
           "copy", "workspace_size", "library_path", "device_error_word", "GRError",
           "hc_read", "hc_write", "hc_fused_write_read", "HC_TANH", "HC_MHC"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgr.so")

GR_F32, GR_BF16, GR_FP8_E4M3 = 0, 1, 2
GR_OP_READ, GR_OP_FUSED_WRITE_READ = 0, 1
HC_TANH, HC_MHC = 0, 1
_HC_MODES = {"hc": HC_TANH, "mhc": HC_MHC, HC_TANH: HC_TANH, HC_MHC: HC_MHC}


class GRError(RuntimeError):
    """A GR library call returned a non-success status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


class _Layer(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("d", ctypes.c_int32), ("r", ctypes.c_int32),
                ("eps", ctypes.c_float), ("gamma", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_write", ctypes.c_void_p)]


class _HcLayer(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("d", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("sinkhorn_iters", ctypes.c_int32), ("eps", ctypes.c_float),
                ("lambda_mix", ctypes.c_float), ("lambda_comb", ctypes.c_float),
                ("lambda_res", ctypes.c_float), ("gamma", ctypes.c_void_p),
                ("w_norm", ctypes.c_void_p), ("w_proj", ctypes.c_void_p),
                ("h_static", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"GR HIP library not built ({_LIB_PATH}); run "
                               "`python -m write_gr_read_amd.build` first")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        LP = ctypes.POINTER(_Layer)
        L.gr_read.argtypes = [P, ctypes.c_int, I64, LP, P, P, P, ctypes.c_size_t, P]
        L.gr_write.argtypes = [P, P, P, ctypes.c_int, I64, I32, I32, P]
        L.gr_fused_write_read.argtypes = [P, P, P, ctypes.c_int, I64, LP, P, P, P,
                                          ctypes.c_size_t, P]
        L.residual_add_rmsnorm.argtypes = [P, P, P, F, P, ctypes.c_int, I64, I32, P]
        L.gr_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, I64, LP,
                                        ctypes.POINTER(ctypes.c_size_t)]
        L.gr_expand.argtypes = [P, P, ctypes.c_int, I64, I32, I32, P]
        L.gr_static_read.argtypes = [P, P, P, ctypes.c_int, I64, I32, I32, P]
        L.gr_round_robin_write.argtypes = [P, P, I32, ctypes.c_int, I64, I32, I32, P]
        L.gr_write_per_channel.argtypes = [P, P, P, ctypes.c_int, I64, I32, I32, P]
        L.gr_collapse.argtypes = [P, P, F, P, ctypes.c_int, I64, I32, I32, P]
        L.gr_bench_tanh_standin.argtypes = [P, P, ctypes.c_int, I64, P]
        L.gr_bench_copy.argtypes = [P, P, ctypes.c_size_t, P]
        L.gr_device_error_word.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
        HP = ctypes.POINTER(_HcLayer)
        L.gr_hc_read.argtypes = [P, ctypes.c_int, I64, HP, P, P, P]
        L.gr_hc_write.argtypes = [P, P, P, ctypes.c_int, I64, I32, I32, P]
        L.gr_hc_fused_write_read.argtypes = [P, P, P, ctypes.c_int, I64, HP, P, P, P]
        L.gr_status_string.argtypes = [ctypes.c_int]
        L.gr_status_string.restype = ctypes.c_char_p
        L.gr_last_error.argtypes = []
        L.gr_last_error.restype = ctypes.c_char_p
        for f in ("gr_read", "gr_write", "gr_fused_write_read", "residual_add_rmsnorm",
                  "gr_workspace_size", "gr_bench_tanh_standin", "gr_bench_copy", "gr_expand",
                  "gr_static_read", "gr_round_robin_write", "gr_write_per_channel", "gr_collapse",
                  "gr_device_error_word", "gr_hc_read", "gr_hc_write", "gr_hc_fused_write_read"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _call(fn: str, *args):
    st = getattr(lib(), fn)(*args)
    if st != 0:
        raise GRError(fn, st, lib().gr_last_error().decode())


# ------------------------------------------------------------------ argument checks

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GR_F32
    if t.dtype == torch.bfloat16:
        return GR_BF16
    if t.dtype == torch.float8_e4m3fn:
        return GR_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, or float8_e4m3fn state)")


def _pdt(state: torch.Tensor) -> torch.dtype:
    """dtype of y, u, gamma and weights for a given state (bf16 with an fp8 state)."""
    return torch.bfloat16 if state.dtype == torch.float8_e4m3fn else state.dtype


def _dev(t: torch.Tensor, name: str, shape, dtype, device) -> int:
    # one combined test for the usual case; the checks below name what is wrong
    if (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.shape == shape
            and (device is None or t.device == device) and t.is_contiguous()):
        return t.data_ptr()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _layer(layer, n: int, d: int, dtype, device, eps: float) -> _Layer:
    g = _dev(layer.gamma, "gamma", (n, d), dtype, device)
    r = 0 if layer.w_down is None else int(layer.w_down.shape[0])
    wd = wu = None
    if r:
        wd = _dev(layer.w_down, "w_down", (r, n * d), dtype, device)
        if layer.w_up is None:
            raise ValueError("w_up is required when w_down is given")
        wu = _dev(layer.w_up, "w_up", (n * d, r), dtype, device)
    elif layer.w_up is not None:
        raise ValueError("w_up given without w_down")
    ww = None
    if layer.w_write is not None:
        ww = _dev(layer.w_write, "w_write", (n, n * d), dtype, device)
    return _Layer(n, d, r, float(eps), g, wd, wu, ww)


# The current HIP stream of a device as a raw pointer; torch's accessor that
# skips building a Stream object (about 0.2 instead of 1.8 us per call) where
# this torch has it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


_workspaces = {}


def _workspace(device, nbytes: int, stream: Optional[int] = None) -> Tuple[int, int]:
    """Scratch buffer per (device, stream), grown on demand: calls on one
    stream are ordered, so they may share it; calls on different streams get
    their own.  The library needs no initialisation of it.  (Under graph
    capture, make one eager call first so that no allocation happens inside
    the capture.)"""
    if nbytes == 0:
        return 0, 0
    key = (device, _stream(device) if stream is None else stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf.data_ptr(), buf.numel()


@functools.lru_cache(maxsize=512)
def _workspace_size(op: int, code: int, N: int, n: int, d: int, r: int, has_write: bool,
                    variant: Optional[str]) -> int:
    L = _Layer(n, d, r, 1e-6, None, None, None, 16 if has_write else None)
    out = ctypes.c_size_t(0)
    _call("gr_workspace_size", op, code, N, ctypes.byref(L), ctypes.byref(out))
    return out.value


def workspace_size(op: int, dtype: torch.dtype, N: int, n: int, d: int, r: int,
                   has_write: bool = True) -> int:
    """Workspace bytes of a call (a pure function of its shape and of the
    GR_KERNEL_VARIANT setting, so remembered per distinct argument set)."""
    code = {torch.bfloat16: GR_BF16, torch.float8_e4m3fn: GR_FP8_E4M3}.get(dtype, GR_F32)
    return _workspace_size(int(op), code, int(N), int(n), int(d), int(r), bool(has_write),
                           os.environ.get("GR_KERNEL_VARIANT"))


# ------------------------------------------------------------------ public API

def device_error_word(reset: bool = False) -> int:
    """The single-pass path's device error word on the current GPU (bit 0: a
    bounded wait on another workgroup timed out).  Synchronous."""
    w = ctypes.c_uint32(0)
    _call("gr_device_error_word", ctypes.byref(w), 1 if reset else 0)
    return w.value


def read(state: torch.Tensor, layer, eps: float = 1e-6, u: Optional[torch.Tensor] = None,
         s: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """GR read of ``state`` [N, n, d]: returns (u [N, d], s [N, n] fp32).
    An fp8 (float8_e4m3fn) state takes bf16 parameters and gives a bf16 u."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    dt = _pdt(state)
    L = _layer(layer, n, d, dt, dev, eps)
    u = torch.empty((N, d), dtype=dt, device=dev) if u is None else u
    s = torch.empty((N, n), dtype=torch.float32, device=dev) if s is None else s
    up = _dev(u, "u", (N, d), dt, dev)
    spo = _dev(s, "s", (N, n), torch.float32, dev)
    need = workspace_size(GR_OP_READ, state.dtype, N, n, d, L.r, layer.w_write is not None)
    st = _stream(dev)
    wp, wn = _workspace(dev, need, st)
    _call("gr_read", sp, _dt(state), N, ctypes.byref(L), up, spo, wp, wn, st)
    return u, s


def write(state: torch.Tensor, y: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """GR write, in place: state[t, i, :] += s[t, i] * y[t, :].  Returns state."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    yp = _dev(y, "y", (N, d), _pdt(state), dev)
    s_p = _dev(s, "s", (N, n), torch.float32, dev)
    _call("gr_write", sp, yp, s_p, _dt(state), N, n, d, _stream(dev))
    return state


def fused_write_read(state: torch.Tensor, y: torch.Tensor, s_in: torch.Tensor, layer,
                     eps: float = 1e-6, u: Optional[torch.Tensor] = None,
                     s: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Write (y, s_in) into ``state`` in place, then read it with ``layer``:
    returns (u_next [N, d], s_next [N, n])."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    dt = _pdt(state)
    yp = _dev(y, "y", (N, d), dt, dev)
    sip = _dev(s_in, "s_in", (N, n), torch.float32, dev)
    L = _layer(layer, n, d, dt, dev, eps)
    u = torch.empty((N, d), dtype=dt, device=dev) if u is None else u
    s = torch.empty((N, n), dtype=torch.float32, device=dev) if s is None else s
    up = _dev(u, "u_next", (N, d), dt, dev)
    spo = _dev(s, "s_next", (N, n), torch.float32, dev)
    need = workspace_size(GR_OP_FUSED_WRITE_READ, state.dtype, N, n, d, L.r, layer.w_write is not None)
    st = _stream(dev)
    wp, wn = _workspace(dev, need, st)
    _call("gr_fused_write_read", sp, yp, sip, _dt(state), N, ctypes.byref(L), up, spo, wp, wn, st)
    return u, s


def residual_add_rmsnorm(x: torch.Tensor, y: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """n = 1: x += y in place (stored), returns out = RMSNorm(x; w)."""
    N, d = x.shape
    dev, dt = x.device, x.dtype
    _dt(x)
    xp = _dev(x, "x", (N, d), dt, None)
    yp = _dev(y, "y", (N, d), dt, dev)
    wp = _dev(w, "w", (d,), dt, dev)
    out = torch.empty_like(x) if out is None else out
    op = _dev(out, "out", (N, d), dt, dev)
    _call("residual_add_rmsnorm", xp, yp, wp, float(eps), op, _dt(x), N, d, _stream(dev))
    return out


# ------------------------------------------------------------------ variants
def expand(e: torch.Tensor, n: int, dtype: Optional[torch.dtype] = None,
           state: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Every branch starts at the embedding: returns state [N, n, d] with
    state[:, i] = e for all i.  ``dtype`` is the state dtype (default e's;
    torch.float8_e4m3fn takes a bf16 e)."""
    N, d = e.shape
    dev = e.device
    dtype = e.dtype if dtype is None else dtype
    if state is None:
        state = torch.empty((N, n, d), dtype=dtype, device=dev)
    sp = _dev(state, "state", (N, n, d), dtype, dev)
    ep = _dev(e, "e", (N, d), _pdt(state), dev)
    _call("gr_expand", ep, sp, _dt(state), N, n, d, _stream(dev))
    return state


def static_read(state: torch.Tensor, h: torch.Tensor, u: Optional[torch.Tensor] = None) -> torch.Tensor:
    """AltUp-style static read: u = sum_i h[i] * state[:, i] (h: n fp32 values)."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    hp = _dev(h, "h", (n,), torch.float32, dev)
    u = torch.empty((N, d), dtype=_pdt(state), device=dev) if u is None else u
    up = _dev(u, "u", (N, d), _pdt(state), dev)
    _call("gr_static_read", sp, hp, up, _dt(state), N, n, d, _stream(dev))
    return u


def round_robin_write(state: torch.Tensor, y: torch.Tensor, layer: int) -> torch.Tensor:
    """AltUp-style write, in place: state[:, layer % n] += y.  Returns state."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    yp = _dev(y, "y", (N, d), _pdt(state), dev)
    _call("gr_round_robin_write", sp, yp, int(layer), _dt(state), N, n, d, _stream(dev))
    return state


def write_per_channel(state: torch.Tensor, y: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """Per-channel write, in place: state[t, i, c] += s[i, c] * y[t, c] (s: [n, d] fp32)."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    yp = _dev(y, "y", (N, d), _pdt(state), dev)
    s_p = _dev(s, "s", (n, d), torch.float32, dev)
    _call("gr_write_per_channel", sp, yp, s_p, _dt(state), N, n, d, _stream(dev))
    return state


def collapse(state: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read-out after the last block: RMSNorm(sum_i state[:, i]; w)."""
    N, n, d = state.shape
    dev = state.device
    _dt(state)
    sp = _dev(state, "state", (N, n, d), state.dtype, None)
    wp = _dev(w, "w", (d,), _pdt(state), dev)
    out = torch.empty((N, d), dtype=_pdt(state), device=dev) if out is None else out
    op = _dev(out, "out", (N, d), _pdt(state), dev)
    _call("gr_collapse", sp, wp, float(eps), op, _dt(state), N, n, d, _stream(dev))
    return out


def tanh_standin(u: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The chained workload's sublayer stand-in, y = 0.1 tanh(u) (HIP kernel)."""
    y = torch.empty_like(u) if y is None else y
    up = _dev(u, "u", tuple(u.shape), u.dtype, None)
    yp = _dev(y, "y", tuple(u.shape), u.dtype, u.device)
    _call("gr_bench_tanh_standin", up, yp, _dt(u), u.numel(), _stream(u.device))
    return y


def copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Streaming 16-byte copy probe (HBM bandwidth reference)."""
    nbytes = src.numel() * src.element_size()
    sp = _dev(src, "src", tuple(src.shape), src.dtype, None)
    dp = _dev(dst, "dst", tuple(src.shape), src.dtype, src.device)
    _call("gr_bench_copy", sp, dp, nbytes, _stream(src.device))
    return dst


# ------------------------------------------------------------------ Hyper-Connections / mHC
def _hc_layer(layer, n: int, d: int, dtype, device) -> _HcLayer:
    """``layer`` has mode ("hc" / "mhc"), iters, eps, lam (3 floats), gamma [n, d],
    w_norm [d], w_proj [n+2, d] (state dtype) and h_static [2n + n*n] fp32."""
    g = _dev(layer.gamma, "gamma", (n, d), dtype, device)
    wn = _dev(layer.w_norm, "w_norm", (d,), dtype, device)
    wp = _dev(layer.w_proj, "w_proj", (n + 2, d), dtype, device)
    hs = _dev(layer.h_static, "h_static", (2 * n + n * n,), torch.float32, device)
    lm, lc, lr = (float(v) for v in layer.lam)
    return _HcLayer(n, d, _HC_MODES[layer.mode], int(layer.iters), float(layer.eps), lm, lc, lr,
                    g, wn, wp, hs)


def _hc_dt(state: torch.Tensor) -> int:
    if state.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"the HC calls take a float32 or bfloat16 state, not {state.dtype}")
    return _dt(state)


def hc_read(state: torch.Tensor, layer, u: Optional[torch.Tensor] = None,
            coeff: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """HC / mHC read of ``state`` [N, n, d]: returns (u [N, d], coeff [N, n + n*n] fp32),
    coeff = [H_comb | H_res row-major] for the write."""
    N, n, d = state.shape
    dev, dt = state.device, state.dtype
    code = _hc_dt(state)
    sp = _dev(state, "state", (N, n, d), dt, None)
    L = _hc_layer(layer, n, d, dt, dev)
    u = torch.empty((N, d), dtype=dt, device=dev) if u is None else u
    coeff = torch.empty((N, n + n * n), dtype=torch.float32, device=dev) if coeff is None else coeff
    up = _dev(u, "u", (N, d), dt, dev)
    cp = _dev(coeff, "coeff", (N, n + n * n), torch.float32, dev)
    _call("gr_hc_read", sp, code, N, ctypes.byref(L), up, cp, _stream(dev))
    return u, coeff


def hc_write(state: torch.Tensor, y: torch.Tensor, coeff: torch.Tensor) -> torch.Tensor:
    """HC / mHC write, in place: R'_i = sum_j H_res[i, j] R_j + H_comb[i] y.  Returns state."""
    N, n, d = state.shape
    dev, dt = state.device, state.dtype
    code = _hc_dt(state)
    sp = _dev(state, "state", (N, n, d), dt, None)
    yp = _dev(y, "y", (N, d), dt, dev)
    cp = _dev(coeff, "coeff", (N, n + n * n), torch.float32, dev)
    _call("gr_hc_write", sp, yp, cp, code, N, n, d, _stream(dev))
    return state


def hc_fused_write_read(state: torch.Tensor, y: torch.Tensor, coeff_in: torch.Tensor, layer,
                        u: Optional[torch.Tensor] = None,
                        coeff: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """HC / mHC write of block l (y, coeff_in) in place, then the read of block
    l+1 with ``layer``: returns (u_next [N, d], coeff_next [N, n + n*n])."""
    N, n, d = state.shape
    dev, dt = state.device, state.dtype
    code = _hc_dt(state)
    sp = _dev(state, "state", (N, n, d), dt, None)
    yp = _dev(y, "y", (N, d), dt, dev)
    cip = _dev(coeff_in, "coeff_in", (N, n + n * n), torch.float32, dev)
    L = _hc_layer(layer, n, d, dt, dev)
    u = torch.empty((N, d), dtype=dt, device=dev) if u is None else u
    coeff = torch.empty((N, n + n * n), dtype=torch.float32, device=dev) if coeff is None else coeff
    up = _dev(u, "u_next", (N, d), dt, dev)
    cp = _dev(coeff, "coeff_next", (N, n + n * n), torch.float32, dev)
    _call("gr_hc_fused_write_read", sp, yp, cip, code, N, ctypes.byref(L), up, cp, _stream(dev))
    return u, coeff
