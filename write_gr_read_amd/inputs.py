"""Seeded synthetic inputs for the Gated Residual (GR) workloads.

This module only draws random numbers and stores them in the storage dtype.
It holds none of the method's arithmetic, so both the fp64 CPU oracle (a test
tool) and the HIP path can be fed from it without sharing any computation.

Recipe (the same for every workload):
  * numpy ``Generator(PCG64(SeedSequence(seed)))``; one child stream per tensor,
    spawned in the fixed order: state X, sublayer output y, then for every
    parameter set (gamma, W_down, W_up, W_write).
  * ``standard_normal`` in float64, times the stated standard deviation (plus
    the stated mean), rounded to float32, then to bfloat16 by round-to-nearest-
    even (torch's conversion) when the storage dtype is bfloat16.  Storage
    dtype "fp8": the state X in OCP e4m3 (torch's float8_e4m3fn conversion,
    round to nearest even, values clamped to +-448 first), everything else in
    bfloat16.
  * Shapes follow the pages' notation: state ``[N, n, d]`` (token, branch,
    channel), ``gamma [n, d]``, ``W_down [r, n*d]``, ``W_up [n*d, r]``,
    ``W_write [n, n*d]`` (the vec index of branch i, channel c is ``i*d + c``).

Hyper-Connections / mHC inputs (make_hc_inputs) follow the same recipe with
their own parameter streams (gamma, w_norm, w_proj, h_static).

Workload sizes are the synthetic configurations the GR measurements use
(tiny fp32 read/write, n=1 fused add+RMSNorm, prefill, decode, a 32-sublayer
chain, the prefill shape with an e4m3 state, and the pages' own model shape
d = 2560 with gate rank r = d/8 = 320). No dataset is involved anywhere.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

_CHUNK = 1 << 24  # values generated per numpy call (bounds host memory)


def _dtype(name: str) -> torch.dtype:
    if name == "f32":
        return torch.float32
    if name == "bf16":
        return torch.bfloat16
    if name == "fp8":
        return torch.float8_e4m3fn
    raise ValueError(f"unknown storage dtype {name!r}")


def param_dtype(name: str) -> str:
    """Storage dtype of y, u, gains and weights for a state dtype."""
    return "bf16" if name == "fp8" else name


def normal(rng: np.random.Generator, shape: Sequence[int], std: float,
           mean: float = 0.0, dtype: str = "bf16",
           scale_rows: Optional[Sequence[float]] = None) -> torch.Tensor:
    """Draw N(mean, std^2) values of ``shape`` into a CPU tensor of ``dtype``.

    ``scale_rows`` multiplies the draws along axis 1 (the branch axis of a
    ``[N, n, d]`` state) before rounding; it is how per-branch scales enter.
    Values are produced in row-major order in chunks, which yields exactly the
    stream a single call would.
    """
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape)) if shape else 1
    out = torch.empty(total, dtype=_dtype(dtype))
    if scale_rows is not None:
        assert len(shape) == 3 and len(scale_rows) == shape[1]
        per_row = shape[2]
        scales = np.asarray(scale_rows, dtype=np.float64)
    pos = 0
    while pos < total:
        cnt = min(_CHUNK, total - pos)
        v = rng.standard_normal(cnt, dtype=np.float64) * std
        if scale_rows is not None:
            idx = np.arange(pos, pos + cnt) // per_row % shape[1]
            v = v * scales[idx]
        if mean:
            v = v + mean
        t = torch.from_numpy(v.astype(np.float32))
        if out.dtype == torch.float8_e4m3fn:
            t = t.clamp(-448.0, 448.0)
        out[pos:pos + cnt] = t.to(out.dtype)
        pos += cnt
    return out.view(shape)


@dataclass
class LayerParams:
    """One GR module's parameters, in the storage dtype (CPU tensors)."""
    gamma: torch.Tensor                 # [n, d]  effective RMSNorm gains
    w_down: Optional[torch.Tensor]      # [r, n*d] or None when r == 0
    w_up: Optional[torch.Tensor]        # [n*d, r] or None when r == 0
    w_write: Optional[torch.Tensor]     # [n, n*d] or None (unit write strengths)

    @property
    def n(self) -> int:
        return self.gamma.shape[0]

    @property
    def d(self) -> int:
        return self.gamma.shape[1]

    @property
    def r(self) -> int:
        return 0 if self.w_down is None else self.w_down.shape[0]

    def to(self, device) -> "LayerParams":
        f = lambda t: None if t is None else t.to(device)
        return LayerParams(f(self.gamma), f(self.w_down), f(self.w_up), f(self.w_write))


@dataclass
class GRInputs:
    """A full synthetic workload: state, sublayer output and parameter sets."""
    N: int
    n: int
    d: int
    r: int
    dtype: str
    eps: float
    X: torch.Tensor                     # [N, n, d]
    y: Optional[torch.Tensor]           # [N, d]
    params: List[LayerParams] = field(default_factory=list)


def make_layer(rngs, n: int, d: int, r: int, dtype: str, w_std: float = 0.02,
               gamma_std: float = 0.01, with_write: bool = True) -> LayerParams:
    """Parameters from four child streams (gamma, W_down, W_up, W_write)."""
    g_rng, d_rng, u_rng, w_rng = rngs
    gamma = normal(g_rng, (n, d), gamma_std, mean=1.0, dtype=dtype)
    w_down = normal(d_rng, (r, n * d), w_std, dtype=dtype) if r > 0 else None
    w_up = normal(u_rng, (n * d, r), w_std, dtype=dtype) if r > 0 else None
    w_write = normal(w_rng, (n, n * d), w_std, dtype=dtype) if with_write else None
    return LayerParams(gamma, w_down, w_up, w_write)


def make_gr_inputs(N: int, n: int, d: int, r: int, dtype: str = "bf16", seed: int = 0,
                   n_param_sets: int = 2, x_std: float = 1.0, y_std: float = 0.05,
                   w_std: float = 0.02, gamma_std: float = 0.01,
                   branch_scale: Optional[Sequence[float]] = None,
                   with_write: bool = True, with_y: bool = True,
                   eps: float = 1e-6) -> GRInputs:
    """Seeded inputs of any shape (the five workloads below are instances)."""
    children = np.random.SeedSequence(seed).spawn(2 + 4 * n_param_sets)
    rngs = [np.random.Generator(np.random.PCG64(c)) for c in children]
    X = normal(rngs[0], (N, n, d), x_std, dtype=dtype, scale_rows=branch_scale)
    pdt = param_dtype(dtype)
    y = normal(rngs[1], (N, d), y_std, dtype=pdt) if with_y else None
    params = [make_layer(rngs[2 + 4 * p: 6 + 4 * p], n, d, r, pdt, w_std, gamma_std,
                         with_write) for p in range(n_param_sets)]
    return GRInputs(N, n, d, r, dtype, eps, X, y, params)


@dataclass
class AddNormInputs:
    """Inputs of the n=1 fused residual add + RMSNorm."""
    N: int
    d: int
    dtype: str
    eps: float
    x: torch.Tensor   # [N, d] residual stream
    y: torch.Tensor   # [N, d] sublayer output
    w: torch.Tensor   # [d]    RMSNorm gain


def make_addnorm_inputs(N: int, d: int, dtype: str = "bf16", seed: int = 0,
                        x_std: float = 1.0, y_std: float = 0.05,
                        w_std: float = 0.01, eps: float = 1e-6) -> AddNormInputs:
    children = np.random.SeedSequence(seed).spawn(3)
    rngs = [np.random.Generator(np.random.PCG64(c)) for c in children]
    x = normal(rngs[0], (N, d), x_std, dtype=dtype)
    y = normal(rngs[1], (N, d), y_std, dtype=dtype)
    w = normal(rngs[2], (d,), w_std, mean=1.0, dtype=dtype)
    return AddNormInputs(N, d, dtype, eps, x, y, w)


@dataclass
class VariantInputs:
    """Inputs of the variants on the widened state (expand, static read,
    round-robin write, per-channel write, collapse)."""
    N: int
    n: int
    d: int
    dtype: str               # state dtype
    X: torch.Tensor          # [N, n, d] state
    e: torch.Tensor          # [N, d]    embedding (activation dtype)
    y: torch.Tensor          # [N, d]    sublayer output (activation dtype)
    h: torch.Tensor          # [n]       static read weights, fp32
    s: torch.Tensor          # [n, d]    per-channel write strengths, fp32
    w: torch.Tensor          # [d]       collapse RMSNorm gain (activation dtype)


def make_variant_inputs(N: int, n: int, d: int, dtype: str = "bf16", seed: int = 0,
                        x_std: float = 1.0, y_std: float = 0.05,
                        branch_scale: Optional[Sequence[float]] = None) -> VariantInputs:
    """Seeded inputs of the variants: X ~ N(0, x_std^2) (per-branch scales
    optional), e ~ N(0, 1), y ~ N(0, y_std^2), h ~ N(1/n, (0.5/n)^2) and
    s ~ N(1, 0.25^2) in fp32, w = 1 + N(0, 0.01^2)."""
    children = np.random.SeedSequence(seed).spawn(6)
    rngs = [np.random.Generator(np.random.PCG64(c)) for c in children]
    pdt = param_dtype(dtype)
    X = normal(rngs[0], (N, n, d), x_std, dtype=dtype, scale_rows=branch_scale)
    e = normal(rngs[1], (N, d), 1.0, dtype=pdt)
    y = normal(rngs[2], (N, d), y_std, dtype=pdt)
    h = normal(rngs[3], (n,), 0.5 / n, mean=1.0 / n, dtype="f32")
    s = normal(rngs[4], (n, d), 0.25, mean=1.0, dtype="f32")
    w = normal(rngs[5], (d,), 0.01, mean=1.0, dtype=pdt)
    return VariantInputs(N, n, d, dtype, X, e, y, h, s, w)


@dataclass
class HCLayer:
    """One Hyper-Connections / mHC module's parameters (CPU tensors).  The
    fields match the library's ``gr_hc_layer``."""
    mode: str                  # "hc" (tanh) or "mhc" (sigmoid, twice sigmoid, Sinkhorn)
    gamma: torch.Tensor        # [n, d]   per-branch gains (state dtype)
    w_norm: torch.Tensor       # [d]      gain of the block's RMSNorm (state dtype)
    w_proj: torch.Tensor       # [n+2, d] W_mix, W_comb, columns of W_res (state dtype)
    h_static: torch.Tensor     # [2n + n*n] fp32: H^s_mix | H^s_comb | H^s_res
    lam: tuple                 # (lambda_mix, lambda_comb, lambda_res)
    iters: int = 20
    eps: float = 1e-6

    def to(self, device) -> "HCLayer":
        return HCLayer(self.mode, self.gamma.to(device), self.w_norm.to(device), self.w_proj.to(device),
                       self.h_static.to(device), self.lam, self.iters, self.eps)


@dataclass
class HCInputs:
    N: int
    n: int
    d: int
    dtype: str
    X: torch.Tensor            # [N, n, d]
    y: torch.Tensor            # [N, d]
    params: List[HCLayer] = field(default_factory=list)


def hc_static_terms(mode: str, n: int, layer: int = 0) -> torch.Tensor:
    """Static terms that start the widened network as the Pre-Norm one: HC takes
    e_(layer mod n), 1 and I for H_mix, H_comb and H_res; mHC takes logits 0
    (sigmoid 1/2), 0 (twice sigmoid 1) and a gap of 8 on the diagonal of H_res."""
    eye = torch.eye(n, dtype=torch.float32)
    if mode == "hc":
        return torch.cat([eye[layer % n], torch.ones(n), eye.reshape(-1)])
    return torch.cat([torch.zeros(n), torch.zeros(n), (8.0 * eye).reshape(-1)])


def make_hc_inputs(N: int, n: int, d: int, mode: str = "mhc", dtype: str = "bf16", seed: int = 0,
                   n_param_sets: int = 2, x_std: float = 1.0, y_std: float = 0.05,
                   w_std: float = 0.02, gamma_std: float = 0.01, lam=(1.0, 1.0, 1.0),
                   static: str = "init", branch_scale: Optional[Sequence[float]] = None,
                   iters: int = 20) -> HCInputs:
    """Seeded inputs of the HC / mHC calls.  Child streams: X, y, then per
    parameter set (gamma, w_norm, w_proj, h_static).  ``static`` = "init" uses
    hc_static_terms (layer = the set's index), "random" draws N(0, 1) fp32."""
    children = np.random.SeedSequence(seed).spawn(2 + 4 * n_param_sets)
    rngs = [np.random.Generator(np.random.PCG64(c)) for c in children]
    X = normal(rngs[0], (N, n, d), x_std, dtype=dtype, scale_rows=branch_scale)
    y = normal(rngs[1], (N, d), y_std, dtype=dtype)
    params = []
    for p in range(n_param_sets):
        g_rng, w_rng, p_rng, h_rng = rngs[2 + 4 * p: 6 + 4 * p]
        gamma = normal(g_rng, (n, d), gamma_std, mean=1.0, dtype=dtype)
        w_norm = normal(w_rng, (d,), gamma_std, mean=1.0, dtype=dtype)
        w_proj = normal(p_rng, (n + 2, d), w_std, dtype=dtype)
        hs = (hc_static_terms(mode, n, p) if static == "init"
              else normal(h_rng, (2 * n + n * n,), 1.0, dtype="f32"))
        params.append(HCLayer(mode, gamma, w_norm, w_proj, hs, tuple(float(v) for v in lam), iters))
    return HCInputs(N, n, d, dtype, X, y, params)


def make_device_state(N: int, n: int, d: int, dtype: str = "bf16", seed: int = 0, device="cuda:0",
                      x_std: float = 1.0, y_std: float = 0.05,
                      branch_scale: Optional[Sequence[float]] = (1.0, 0.5, 2.0, 1.0)):
    """State [N, n, d] and y [N, d] drawn on ``device`` with torch's seeded
    generator of that device: for sizes whose host-side draw would be slow
    (billions of values).  Same distributions as make_gr_inputs; a test hands
    the oracle the rows it samples from these very tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    X = torch.randn((N, n, d), generator=g, device=device, dtype=torch.float32).mul_(x_std)
    if branch_scale is not None:
        X.mul_(torch.tensor(branch_scale[:n], device=device, dtype=torch.float32).view(1, n, 1))
    if _dtype(dtype) == torch.float8_e4m3fn:
        X.clamp_(-448.0, 448.0)
    X = X.to(_dtype(dtype))
    y = torch.randn((N, d), generator=g, device=device, dtype=torch.float32).mul_(y_std)
    return X, y.to(_dtype(param_dtype(dtype)))


# The synthetic workloads, by number. Seed of workload k is 1000*k.
WORKLOADS = {
    1: dict(name="gr_tiny_f32", kind="gr", N=64, n=4, d=256, r=16, dtype="f32",
            y_std=0.1, branch_scale=None, param_sets=2),
    2: dict(name="add_rmsnorm_n1_bf16", kind="addnorm", N=8192, d=4096, dtype="bf16",
            y_std=0.05),
    3: dict(name="gr_prefill_bf16", kind="gr", N=16384, n=4, d=4096, r=64, dtype="bf16",
            y_std=0.05, branch_scale=(1.0, 0.5, 2.0, 1.0), param_sets=2),
    4: dict(name="gr_decode_bf16", kind="gr", N=256, n=4, d=4096, r=64, dtype="bf16",
            y_std=0.05, branch_scale=(1.0, 0.5, 2.0, 1.0), param_sets=2),
    5: dict(name="gr_chain32_bf16", kind="chain", N=32768, n=4, d=2048, r=32, dtype="bf16",
            layers=32, branch_scale=None, param_sets=32),
    # the prefill shape with an fp8 (e4m3) branch state: the pages' FP8 state
    6: dict(name="gr_prefill_fp8", kind="gr", N=16384, n=4, d=4096, r=64, dtype="fp8",
            y_std=0.05, branch_scale=(1.0, 0.5, 2.0, 1.0), param_sets=2),
    # the pages' own model shape: d = 2560 and the gate rank r = d/8 = 320
    7: dict(name="gr_prefill_d2560_r320", kind="gr", N=16384, n=4, d=2560, r=320, dtype="bf16",
            y_std=0.05, branch_scale=(1.0, 0.5, 2.0, 1.0), param_sets=2),
    # the pages' model shape with the FP8 (e4m3) branch state
    8: dict(name="gr_prefill_fp8_d2560_r320", kind="gr", N=16384, n=4, d=2560, r=320, dtype="fp8",
            y_std=0.05, branch_scale=(1.0, 0.5, 2.0, 1.0), param_sets=2),
}


def workload(k: int, N: Optional[int] = None):
    """Inputs of workload ``k`` (optionally with fewer tokens, same recipe).

    Parameter set 0 feeds the untimed read that produces the write strengths of
    the fused call; parameter set 1 is the next sublayer's (workloads 1, 3, 4, 6, 7, 8).
    Workload 5 has one parameter set per sublayer and no y (F makes it).
    """
    w = WORKLOADS[k]
    seed = 1000 * k
    NN = w["N"] if N is None else N
    if w["kind"] == "addnorm":
        return make_addnorm_inputs(NN, w["d"], w["dtype"], seed, y_std=w["y_std"])
    return make_gr_inputs(NN, w["n"], w["d"], w["r"], w["dtype"], seed,
                          n_param_sets=w["param_sets"], y_std=w.get("y_std", 0.05),
                          branch_scale=w["branch_scale"], with_y=w["kind"] != "chain")
