#!/usr/bin/env python3
"""Benchmark of the Gated Residual fused write+read on one MI355X.

One step = one gr_fused_write_read over the prefill workload (N = 16384
tokens, d = 4096, n = 4 branches, gate rank r = 64, bf16 state with fp32
accumulation): the write of sublayer l and the whole read of sublayer l+1
(Group RMSNorm, low-rank gate, gated combine, write strengths), i.e. every
step of the hot path.  Inputs are seeded synthetic tensors already resident in
HBM.  Prints one JSON line on stdout; progress goes to stderr.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --workload {prefill,prefill_fp8,prefill_r320,prefill_fp8_r320,decode,addnorm,
                                   chain,tiny,variants,all}
The default (prefill) line is the headline; the other workloads print their own
line (prefill_fp8: the same shape with an e4m3 branch state; prefill_r320: the
pages' model shape d = 2560 with gate rank r = d/8 = 320; prefill_fp8_r320:
that shape with an e4m3 state; variants: expand,
static read, round-robin write, per-channel write and collapse at the prefill
shape, one line each; decode: us per
call with the state warm in cache, back to back; addnorm:
the n = 1 fused residual add + RMSNorm; chain: 32 sublayers of read -> F ->
fused write+read -> ... -> write with the elementwise F stand-in).

Every timed region starts after about 100 ms of untimed streaming copies
(--no-burn-in skips them) so that the GPU's power management has settled; the
default line measures the copy probe and the other workloads first and times
the headline last.
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


def algorithmic_bytes(N, n, d, r, elt=2, has_write=True, state_elt=None):
    """Bytes the fused write+read must move: state in and out, y in, u out,
    s in and out (fp32), plus gamma and the gate/write weights once.  `elt` is
    the size of y, u and the weights; `state_elt` that of the branch state
    (default: the same; 1 for an e4m3 state)."""
    se = elt if state_elt is None else state_elt
    per_token = 2 * n * d * se + 2 * d * elt + 2 * n * 4
    weights = n * d * elt + 2 * r * n * d * elt + (n * n * d * elt if has_write else 0)
    return N * per_token + weights


def gate_flops(N, n, d, r, has_write=True):
    """Contraction flops of one read: down and up projections of the gate
    (2 r n d each) and the write projection (2 n n d), per token."""
    return N * (4 * r * n * d + (2 * n * n * d if has_write else 0))


# The files holding the kernels of gr_fused_write_read (the MFMA path and its
# device helpers); stored counters apply while these are unchanged.
FUSED_KERNEL_SOURCES = ("gr_device.h", "gr_fast_common.h", "gr_fast.hip", "gr_fast_k1.hip", "gr_fast_k2.hip")


def kernel_source_digest(files=FUSED_KERNEL_SOURCES):
    """Digest of a call's kernel sources, to tell whether stored counters
    still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "write_gr_read_amd", "csrc")
    for f in files:
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
    if not rec or rec.get("source_digest") != kernel_source_digest(tuple(rec.get("sources", FUSED_KERNEL_SOURCES))):
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(Xin, threads, n_tokens, single_tokens=1024):
    """The oracle (plain fp64 C) on a bounded sample of the same workload:
    `threads` threads over disjoint token ranges, and one thread on the first
    `single_tokens` tokens."""
    import numpy as np
    import oracle
    p0, p1 = Xin.params
    n_tokens = min(n_tokens, Xin.N)
    R = Xin.X[:n_tokens].double().numpy()
    y = Xin.y[:n_tokens].double().numpy()
    _, s0 = oracle.read(Xin.X[:1], p0.gamma, p0.w_down, p0.w_up, p0.w_write)
    s_in = np.repeat(s0, n_tokens, axis=0)
    w = [oracle._f64(t) for t in (p1.gamma, p1.w_down, p1.w_up, p1.w_write)]
    fn = lambda R_, y_, s_: oracle.fused(R_, y_, s_, *w)
    t0 = time.perf_counter()
    oracle.parallel_tokens(fn, [R, y, s_in], threads)
    dt = time.perf_counter() - t0
    m = min(single_tokens, n_tokens)
    t1 = time.perf_counter()
    fn(R[:m], y[:m], s_in[:m])
    dt1 = time.perf_counter() - t1
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fused write+read of the first {n_tokens} of {Xin.N} prefill tokens "
                      f"(fp64 C oracle, {threads} threads over disjoint token ranges, "
                      f"{dt:.2f} s wall, ~{dt * threads:.0f} thread-seconds)",
            "cpu_model": cpu_model(), "cores_in_affinity_mask": len(os.sched_getaffinity(0)),
            "single_thread": {"value": m / dt1, "unit": "tokens/s", "tokens": m, "seconds": dt1}}


def copy_probe(gr, torch, dev, stream):
    """What a plain 16-byte copy kernel moves on this GPU (read + write of
    1 GiB): context for the HBM fractions, and the known-size reference that
    scales the FETCH_SIZE / WRITE_SIZE counters of the traffic profiles."""
    nbytes = 1 << 30
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1)
    b = torch.empty_like(a)
    burn_in()
    for _ in range(3):
        gr.copy(a, b)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(10):
        gr.copy(a, b)
    stop.record(stream)
    torch.cuda.synchronize()
    return 2 * nbytes / (start.elapsed_time(stop) / 10 * 1e-3) / 1e9


BURN_IN_MS = 100.0   # 0 (--no-burn-in): measure without settling the GPU first
_burn_buf = {}


def burn_in():
    """Untimed streaming copies (256 MiB each way) for about BURN_IN_MS ms right
    before a timed region, so that the GPU's clocks have settled: a GPU that
    was idle (e.g. while inputs were generated on the host) boosts, then slows
    down for some tens of milliseconds while its power management settles
    (calls 6-25 of the prefill call take ~470 us from idle, ~430 us once
    settled).  Returns (copies, elapsed ms)."""
    if BURN_IN_MS <= 0:
        return 0, 0.0
    import torch
    import write_gr_read_amd as gr
    if "a" not in _burn_buf:
        _burn_buf["a"] = torch.empty(1 << 28, dtype=torch.uint8, device="cuda:0")
        _burn_buf["b"] = torch.empty_like(_burn_buf["a"])
    a, b = _burn_buf["a"], _burn_buf["b"]
    gr.copy(a, b)              # the library's first launch is not GPU time
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < BURN_IN_MS:
        for _ in range(20):
            gr.copy(a, b)
        torch.cuda.synchronize()
        n += 20
    return n, (time.perf_counter() - t0) * 1e3


def timed(fn, steps, warmup, stream):
    """Average ms per call of fn over `steps` calls after `warmup` calls (after
    the burn-in)."""
    import torch
    burn_in()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def per_call_ms(fn, reps, stream, between=None):
    """Duration of each of ``reps`` calls (HIP events around every call, on
    the call's stream); ``between`` runs untimed before each call."""
    import torch
    evs = []
    for _ in range(reps):
        if between is not None:
            between()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def percentiles(ms_list):
    import numpy as np
    q = np.percentile(np.asarray(ms_list), [10, 50, 90])
    return {"ms_p10": float(q[0]), "ms_p50": float(q[1]), "ms_p90": float(q[2])}


def graph_replay_ms(fn, steps, warmup, stream):
    """Average ms of ``fn`` captured once in a HIP graph and replayed."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()                      # eager calls on the capture stream first (workspace)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        fn()
    return timed(graph.replay, steps, warmup, stream)


def line(metric, value, unit, steps, warmup, ms, config, dtype="bf16", higher=True, **extra):
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": ms, "higher_is_better": higher, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config}
    out.update(extra)
    return out


def roofline(alg_bytes, ms, kernel, traffic=None):
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": gbps / PEAK_HBM_GBPS, "traffic": traffic, "kernel": kernel,
            "algorithmic_bytes_per_launch": alg_bytes}


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def mfma_roofline(flops, ms, kernel, traffic=None):
    """Roofline of a contraction-heavy call: algorithmic flops (the gate's
    down, up and write projections once each; the hi/lo operand split of the
    kernels doubles the MFMA work actually issued) over the bf16 MFMA peak."""
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": kernel,
            "algorithmic_flops_per_launch": flops}


def bench_other(which, args, dev):
    """Lines for the non-headline workloads."""
    import torch
    import write_gr_read_amd as gr
    from write_gr_read_amd import inputs
    stream = torch.cuda.current_stream(dev)
    if which in ("decode", "tiny"):
        k = 4 if which == "decode" else 1
        W = inputs.WORKLOADS[k]
        Xin = inputs.workload(k)
        N, n, d, r = Xin.N, Xin.n, Xin.d, Xin.r
        p0, p1 = Xin.params[0].to(dev), Xin.params[1].to(dev)
        X, y = Xin.X.to(dev), Xin.y.to(dev)
        u = torch.empty((N, d), dtype=X.dtype, device=dev)
        so = torch.empty((N, n), dtype=torch.float32, device=dev)
        _, s_in = gr.read(X, p0)
        steps = args.steps if args.steps_given else 2000
        call = lambda: gr.fused_write_read(X, y, s_in, p1, u=u, s=so)
        ms = timed(call, steps, args.warmup, stream)
        elt = 2 if Xin.dtype == "bf16" else 4
        alg = algorithmic_bytes(N, n, d, r, elt)
        extra = {}
        if which == "decode":
            # per call warm, cold (512 MiB written between calls so nothing of the
            # call's data is left in the caches), and replayed from a HIP graph
            flush = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
            extra["warm"] = percentiles(per_call_ms(call, 200, stream))
            extra["cold"] = percentiles(per_call_ms(call, 50, stream, between=lambda: flush.fill_(1)))
            extra["graph_replay_us_per_call"] = graph_replay_ms(call, steps, args.warmup, stream) * 1e3
            del flush
            log(f"decode: warm p50 {extra['warm']['ms_p50'] * 1e3:.1f} us, cold p50 "
                f"{extra['cold']['ms_p50'] * 1e3:.1f} us, graph replay {extra['graph_replay_us_per_call']:.1f} us")
        log(f"{which}: {ms * 1e3:.2f} us/call")
        return line(f"GR fused write+read us/call ({which}, N={N}, d={d}, n={n}, r={r})",
                    ms * 1e3, "us/call", steps, args.warmup, ms,
                    {"workload": W["name"], "N": N, "d": d, "n": n, "r": r, "cache": "warm, back-to-back"},
                    dtype=Xin.dtype, higher=False, tokens_per_s=N / (ms * 1e-3),
                    roofline=roofline(alg, ms, "gr_fused_write_read"), **extra)
    if which in ("prefill_fp8", "prefill_r320", "prefill_fp8_r320"):
        k = {"prefill_fp8": 6, "prefill_r320": 7, "prefill_fp8_r320": 8}[which]
        W = inputs.WORKLOADS[k]
        log(f"generating workload {W['name']} ...")
        Xin = inputs.workload(k)
        N, n, d, r = Xin.N, Xin.n, Xin.d, Xin.r
        p0, p1 = Xin.params[0].to(dev), Xin.params[1].to(dev)
        X, y = Xin.X.to(dev), Xin.y.to(dev)
        u = torch.empty((N, d), dtype=y.dtype, device=dev)
        so = torch.empty((N, n), dtype=torch.float32, device=dev)
        _, s_in = gr.read(X, p0)
        ms = timed(lambda: gr.fused_write_read(X, y, s_in, p1, u=u, s=so), args.steps, args.warmup, stream)
        f8 = Xin.dtype == "fp8"
        alg = algorithmic_bytes(N, n, d, r, 2, state_elt=1 if f8 else 2)
        log(f"{which}: {ms * 1e3:.1f} us/call, {N / (ms * 1e-3) / 1e6:.2f} M tok/s")
        sdt = "e4m3" if f8 else "bf16"
        return line(f"GR fused write+read tokens/s (prefill, d={d}, n={n}, r={r}, {sdt} state)",
                    N / (ms * 1e-3), "tokens/s", args.steps, args.warmup, ms,
                    {"workload": W["name"], "N": N, "d": d, "n": n, "r": r,
                     "state_dtype": sdt, "activation_dtype": "bf16", "accumulation": "fp32"},
                    dtype="bf16", gate_tflops=gate_flops(N, n, d, r) / (ms * 1e-3) / 1e12,
                    hbm_GBps_algorithmic=alg / (ms * 1e-3) / 1e9,
                    roofline=(roofline(alg, ms, "gr_fused_write_read", stored_traffic("gr_fused_write_read_fp8"))
                              if which == "prefill_fp8" else
                              mfma_roofline(gate_flops(N, n, d, r), ms, "gr_fused_write_read",
                                            stored_traffic("gr_fused_write_read_" + which[len("prefill_"):]))))
    if which == "variants":
        # the variants on the widened state at the prefill shape, bf16: one line each
        N, n, d = 16384, 4, 4096
        V = inputs.make_variant_inputs(N, n, d, "bf16", seed=8000, branch_scale=(1.0, 0.5, 2.0, 1.0))
        h, sc, w = V.h.to(dev), V.s.to(dev), V.w.to(dev)
        # three buffer sets rotate between calls, so a call's footprint (up to
        # 640 MiB) is not left in the 256 MB Infinity Cache by the previous call
        sets = [dict(X=V.X.to(dev), e=V.e.to(dev), y=V.y.to(dev),
                     u=torch.empty((N, d), dtype=torch.bfloat16, device=dev),
                     st=torch.empty((N, n, d), dtype=torch.bfloat16, device=dev)) for _ in range(3)]
        rot = {"i": 0}
        def rotating(f):
            def call():
                b = sets[rot["i"] % 3]
                rot["i"] += 1
                f(b)
            return call
        steps = args.steps if args.steps_given else 50
        ops = {
            "expand": (rotating(lambda b: gr.expand(b["e"], n, state=b["st"])), N * d * 2 + N * n * d * 2),
            "static_read": (rotating(lambda b: gr.static_read(b["X"], h, u=b["u"])), N * n * d * 2 + N * d * 2),
            "round_robin_write": (rotating(lambda b: gr.round_robin_write(b["X"], b["y"], 1)), 3 * N * d * 2),
            "write_per_channel": (rotating(lambda b: gr.write_per_channel(b["X"], b["y"], sc)),
                                  2 * N * n * d * 2 + N * d * 2 + n * d * 4),
            "collapse": (rotating(lambda b: gr.collapse(b["X"], w, out=b["u"])), N * n * d * 2 + N * d * 2 + d * 2),
        }
        lines = []
        for name, (fn, alg) in ops.items():
            ms = timed(fn, steps, args.warmup, stream)
            log(f"{name}: {ms * 1e3:.1f} us/call, {alg / (ms * 1e-3) / 1e9:.0f} GB/s")
            lines.append(line(f"GR variant {name} tokens/s (N={N}, d={d}, n={n}, bf16 state)",
                              N / (ms * 1e-3), "tokens/s", steps, args.warmup, ms,
                              {"workload": f"variant_{name}", "N": N, "d": d, "n": n,
                               "state_dtype": "bf16", "buffer_sets": 3},
                              roofline=roofline(alg, ms, f"gr_{name}")))
        return lines
    if which == "addnorm":
        W = inputs.WORKLOADS[2]
        A = inputs.workload(2)
        # three buffer sets rotate so the 192 MiB footprint does not sit in the 256 MB cache
        sets = [(A.x.to(dev), A.y.to(dev), torch.empty_like(A.x, device=dev)) for _ in range(3)]
        w = A.w.to(dev)
        state = {"i": 0}
        def step():
            x, yy, out = sets[state["i"] % 3]
            state["i"] += 1
            gr.residual_add_rmsnorm(x, yy, w, out=out)
        steps = args.steps if args.steps_given else 60
        ms = timed(step, steps, args.warmup, stream)
        alg = 4 * A.N * A.d * 2 + A.d * 2
        log(f"addnorm: {ms * 1e3:.1f} us/call, {alg / ms / 1e6:.0f} GB/s")
        return line(f"fused residual add + RMSNorm tokens/s (n=1, N={A.N}, d={A.d}, bf16)",
                    A.N / (ms * 1e-3), "tokens/s", steps, args.warmup, ms,
                    {"workload": W["name"], "N": A.N, "d": A.d, "buffer_sets": 3},
                    roofline=roofline(alg, ms, "residual_add_rmsnorm"))
    if which == "chain":
        W = inputs.WORKLOADS[5]
        Xin = inputs.workload(5)
        N, n, d, r = Xin.N, Xin.n, Xin.d, Xin.r
        ps = [p.to(dev) for p in Xin.params]
        X0 = Xin.X.to(dev)
        X = X0.clone()
        u = torch.empty((N, d), dtype=X.dtype, device=dev)
        yb = torch.empty_like(u)
        s_bufs = [torch.empty((N, n), dtype=torch.float32, device=dev) for _ in range(2)]
        def chain():
            s_cur = s_bufs[0]
            gr.read(X, ps[0], u=u, s=s_cur)
            gr.tanh_standin(u, yb)
            for k, p in enumerate(ps[1:]):
                s_nxt = s_bufs[(k + 1) % 2]
                gr.fused_write_read(X, yb, s_cur, p, u=u, s=s_nxt)
                gr.tanh_standin(u, yb)
                s_cur = s_nxt
            gr.write(X, yb, s_cur)
        steps = args.steps if args.steps_given else 5
        ms = timed(chain, steps, max(1, min(args.warmup, 2)), stream)
        ms_f = timed(lambda: gr.tanh_standin(u, yb), 20, 2, stream)
        gr_ms = ms - len(ps) * ms_f
        per_fused = algorithmic_bytes(N, n, d, r)
        weights = n * d * 2 + 2 * r * n * d * 2 + n * n * d * 2
        read_b = N * (n * d * 2 + d * 2 + n * 4) + weights
        write_b = N * (2 * n * d * 2 + d * 2 + n * 4)
        alg = (len(ps) - 1) * per_fused + read_b + write_b
        log(f"chain: {ms:.2f} ms per 32-sublayer pass (F stand-in {len(ps) * ms_f:.2f} ms of it)")
        return line(f"GR 32-sublayer chain tokens/s (N={N}, d={d}, n={n}, r={r}, bf16)",
                    N / (ms * 1e-3), "tokens/s", steps, 1, ms,
                    {"workload": W["name"], "N": N, "d": d, "n": n, "r": r, "sublayers": len(ps)},
                    gr_ms_per_pass=gr_ms, f_standin_ms_per_pass=len(ps) * ms_f,
                    roofline=roofline(alg, gr_ms, "GR calls of the chain (F excluded)"))
    if which in ("hc_mhc", "hc_tanh"):
        # Hyper-Connections (tanh) / mHC (sigmoid, Sinkhorn 20) on the prefill
        # shape: the fused write + read, one pass over the state
        mode = "mhc" if which == "hc_mhc" else "hc"
        N, n, d = 16384, 4, 4096
        Xin = inputs.make_hc_inputs(N, n, d, mode, "bf16", seed=11000 + (mode == "mhc"),
                                    branch_scale=(1.0, 0.5, 2.0, 1.0))
        X, y = Xin.X.to(dev), Xin.y.to(dev)
        p0, p1 = Xin.params[0].to(dev), Xin.params[1].to(dev)
        _, c_in = gr.hc_read(X, p0)                     # untimed: the write's coefficients
        u = torch.empty((N, d), dtype=X.dtype, device=dev)
        c_out = torch.empty_like(c_in)
        steps = args.steps if args.steps_given else 50
        ms = timed(lambda: gr.hc_fused_write_read(X, y, c_in, p1, u=u, coeff=c_out), steps, args.warmup, stream)
        # the same work as two calls (write, then read): two passes over the state
        ms_w = timed(lambda: gr.hc_write(X, y, c_in), steps, args.warmup, stream)
        ms_r = timed(lambda: gr.hc_read(X, p1, u=u, coeff=c_out), steps, args.warmup, stream)
        nc = n + n * n
        alg = N * (2 * n * d * 2 + 2 * d * 2 + 2 * nc * 4) + (n * d + d + (n + 2) * d) * 2 + (2 * n + n * n) * 4
        log(f"{which}: {ms * 1e3:.1f} us/call, {alg / ms / 1e6:.0f} GB/s algorithmic")
        name = "mHC" if mode == "mhc" else "HC"
        return line(f"{name} fused write+read tokens/s (N={N}, d={d}, n={n}, bf16 state)",
                    N / (ms * 1e-3), "tokens/s", steps, args.warmup, ms,
                    {"workload": f"hc_{mode}_prefill_bf16", "N": N, "d": d, "n": n, "mode": mode,
                     "sinkhorn_iters": Xin.params[1].iters if mode == "mhc" else 0},
                    roofline=roofline(alg, ms, f"gr_hc_fused_write_read ({name})", stored_traffic(which)),
                    write_only_ms=ms_w, read_only_ms=ms_r, unfused_ms=ms_w + ms_r)
    raise ValueError(which)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU baseline (default: the host's, at most 16)")
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens of the workload the CPU baseline runs (about 20 thread-seconds at 16384)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time the copy probe (always beside the headline; with --workload, before it)")
    ap.add_argument("--no-copy-probe", action="store_true", help="skip the copy probe")
    ap.add_argument("--no-burn-in", action="store_true",
                    help="skip the untimed burn-in copies at the start (profiling runs, whose "
                         "summaries separate the call's kernels from the copy probe's)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the tiny / decode / add+RMSNorm / chain / HC / single-pass keys of the default line")
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "prefill_fp8", "prefill_r320", "prefill_fp8_r320", "decode", "addnorm",
                             "chain", "tiny", "variants", "hc_mhc", "hc_tanh", "all"])
    args = ap.parse_args()
    args.steps_given = "--steps" in sys.argv

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GR path is per-token and is sharded over "
              "tokens with no communication; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import write_gr_read_amd as gr
    from write_gr_read_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    global BURN_IN_MS
    if args.no_burn_in:
        BURN_IN_MS = 0.0
    if args.workload != "prefill":
        names = (["prefill_fp8", "prefill_r320", "prefill_fp8_r320", "decode", "addnorm", "chain", "tiny",
                  "variants", "hc_mhc", "hc_tanh"]
                 if args.workload == "all" else [args.workload])
        if args.copy_probe:
            log(f"copy probe: {copy_probe(gr, torch, dev, torch.cuda.current_stream(dev)):.0f} GB/s")
        for w in names:
            res = bench_other(w, args, dev)
            for one in (res if isinstance(res, list) else [res]):
                print(json.dumps(one), flush=True)
        if args.workload != "all":
            return
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
    stream = torch.cuda.current_stream(dev)
    alg = algorithmic_bytes(N, n, d, r)

    # The copy probe and the other workloads' lines run before the headline is
    # timed, and every timed region starts after a burn-in (see burn_in), so
    # the headline is measured at the GPU's steady state.  The timed region is
    # the warmup calls, then exactly the timed steps.
    copy_gbps = None
    if not args.no_copy_probe:
        copy_gbps = copy_probe(gr, torch, dev, stream)
        log(f"copy probe: {copy_gbps:.0f} GB/s (read + write of 1 GiB)")
    others = None
    if not args.no_others:
        # the other configurations of the workload set, one key each with its
        # own roofline: the tiny fp32 call and decode (us/call), the n = 1 fused
        # add + RMSNorm, the 32-sublayer chain, mHC and HC on the prefill shape,
        # and the single-pass kernel on this same prefill call
        others = {}
        for w in ("tiny", "decode", "addnorm", "chain", "hc_mhc", "hc_tanh"):
            log(f"workload {w} ...")
            res = bench_other(w, args, dev)
            keep = ("metric", "value", "unit", "ms_per_step", "steps", "config", "roofline", "tokens_per_s",
                    "warm", "cold", "graph_replay_us_per_call", "gr_ms_per_pass", "f_standin_ms_per_pass",
                    "write_only_ms", "read_only_ms", "unfused_ms")
            others[w] = {k: res[k] for k in keep if k in res}
        os.environ["GR_KERNEL_VARIANT"] = "single"
        try:
            ms1 = timed(lambda: gr.fused_write_read(X, y, s_in, p1, u=u, s=s_next), args.steps, args.warmup, stream)
        finally:
            del os.environ["GR_KERNEL_VARIANT"]
        others["prefill_single_pass"] = {"value": N / (ms1 * 1e-3), "unit": "tokens/s", "ms_per_step": ms1,
                                         "roofline": roofline(alg, ms1, "gr_fused_write_read (GR_KERNEL_VARIANT=single)")}
        log(f"single-pass kernel on the prefill call: {ms1 * 1e3:.1f} us/call")

    nb, msb = burn_in()
    log(f"burn-in: {nb} untimed 256 MiB copies over {msb:.0f} ms (GPU clocks settle)")
    log(f"warmup {args.warmup} ...")
    for _ in range(args.warmup):
        gr.fused_write_read(X, y, s_in, p1, u=u, s=s_next)
    torch.cuda.synchronize()
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

    # spread of single calls (HIP events around each; not part of the timed region)
    out.update(percentiles(per_call_ms(lambda: gr.fused_write_read(X, y, s_in, p1, u=u, s=s_next),
                                       args.steps, stream)))

    if copy_gbps is not None:
        out["copy_probe_GBps"] = copy_gbps
    if others is not None:
        out["other_workloads"] = others

    if not args.no_cpu:
        # 16 threads: the host CPU share of one GPU on the measurement machines
        threads = args.cpu_threads or max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"CPU baseline: oracle on {args.cpu_tokens} tokens, {threads} threads ...")
        out["cpu_baseline"] = cpu_baseline(Xin, threads, args.cpu_tokens)
        log(f"CPU baseline: {out['cpu_baseline']['value']:.0f} tokens/s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
