#!/usr/bin/env python3
"""Benchmark of the Gated Residual fused write+read on one MI355X.

One step = one gr_fused_write_read over the prefill workload (N = 16384
tokens, d = 4096, n = 4 branches, gate rank r = 64, bf16 state with fp32
accumulation): the write of sublayer l and the whole read of sublayer l+1
(Group RMSNorm, low-rank gate, gated combine, write strengths), i.e. every
step of the hot path.  Inputs are seeded synthetic tensors already resident in
HBM.  Prints one JSON line on stdout; progress goes to stderr.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(N, n, d, r, elt=2, has_write=True):
    """Bytes the fused write+read must move: state in and out, y in, u out,
    s in and out (fp32), plus gamma and the gate/write weights once."""
    per_token = 2 * n * d * elt + 2 * d * elt + 2 * n * 4
    weights = n * d * elt + 2 * r * n * d * elt + (n * n * d * elt if has_write else 0)
    return N * per_token + weights


def kernel_source_digest():
    """Digest of the HIP sources, to tell whether stored counters still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "write_gr_read_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_name):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get(kernel_name)
    if not rec or rec.get("source_digest") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(Xin, threads, n_tokens):
    """The oracle (plain fp64 C) on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    p0, p1 = Xin.params
    R = Xin.X[:n_tokens].double().numpy()
    y = Xin.y[:n_tokens].double().numpy()
    _, s0 = oracle.read(Xin.X[:1], p0.gamma, p0.w_down, p0.w_up, p0.w_write)
    s_in = np.repeat(s0, n_tokens, axis=0)
    w = [oracle._f64(t) for t in (p1.gamma, p1.w_down, p1.w_up, p1.w_write)]
    fn = lambda R_, y_, s_: oracle.fused(R_, y_, s_, *w)
    t0 = time.perf_counter()
    oracle.parallel_tokens(fn, [R, y, s_in], threads)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fused write+read of the first {n_tokens} of {Xin.N} prefill tokens "
                      f"(fp64 C oracle, {threads} threads over disjoint token ranges, "
                      f"{dt:.2f} s wall)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--copy-probe", action="store_true", help="also time the copy probe")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GR path is per-token and is sharded over "
              "tokens with no communication; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import write_gr_read_amd as gr
    from write_gr_read_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = inputs.WORKLOADS[3]
    log(f"generating workload {W['name']} ...")
    Xin = inputs.workload(3)
    N, n, d, r = Xin.N, Xin.n, Xin.d, Xin.r
    p0, p1 = Xin.params[0].to(dev), Xin.params[1].to(dev)
    X = Xin.X.to(dev)
    y = Xin.y.to(dev)
    u = torch.empty((N, d), dtype=X.dtype, device=dev)
    s_next = torch.empty((N, n), dtype=torch.float32, device=dev)
    _, s_in = gr.read(X, p0)  # untimed: write strengths of the previous sublayer
    torch.cuda.synchronize()

    log(f"warmup {args.warmup} ...")
    for _ in range(args.warmup):
        gr.fused_write_read(X, y, s_in, p1, u=u, s=s_next)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps ...")
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        gr.fused_write_read(X, y, s_in, p1, u=u, s=s_next)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    tokens_per_s = N / (ms * 1e-3)
    alg = algorithmic_bytes(N, n, d, r)
    gbps = alg / (ms * 1e-3) / 1e9
    log(f"fused write+read: {ms * 1e3:.1f} us/call, {tokens_per_s / 1e6:.2f} M tok/s, "
        f"{gbps:.0f} GB/s algorithmic ({gbps / PEAK_HBM_GBPS:.1%} of peak); wall {wall:.2f}s")

    kname = "gr_fused_write_read"
    out = {
        "metric": "GR fused write+read tokens/s (prefill, d=4096, n=4, r=64, bf16 state)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W["name"], "N": N, "d": d, "n": n, "r": r,
                   "state_dtype": "bf16", "accumulation": "fp32"},
        "hbm_GBps_algorithmic": gbps,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": stored_traffic(kname),
                     "kernel": kname, "algorithmic_bytes_per_launch": alg},
    }

    if args.copy_probe:
        nbytes = 1 << 30
        a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            gr.copy(a, b)
        start.record(stream)
        for _ in range(10):
            gr.copy(a, b)
        stop.record(stream)
        torch.cuda.synchronize()
        cms = start.elapsed_time(stop) / 10
        out["copy_probe_GBps"] = 2 * nbytes / (cms * 1e-3) / 1e9
        log(f"copy probe: {out['copy_probe_GBps']:.0f} GB/s (read + write of 1 GiB)")
        del a, b

    if not args.no_cpu:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"CPU baseline: oracle on {args.cpu_tokens} tokens, {threads} threads ...")
        out["cpu_baseline"] = cpu_baseline(Xin, threads, args.cpu_tokens)
        log(f"CPU baseline: {out['cpu_baseline']['value']:.0f} tokens/s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
