"""GPU parity of the single-pass cluster kernel (GR_KERNEL_VARIANT=single):
one persistent launch in which the 32 workgroups of an XCD split the channels
of each token tile and exchange partial sums through that XCD's L2, so the
state is read once and written once ("Paper reading: Qwen3.8 Flash Next",
part 2 Residual, sec. 4 eq:rms .. eq:write; sec. 7: one traversal per
direction).  Same bar as the default path (tests/parity.py): the written state
bit for bit, u and s at the stated tolerances; and the state equal to the
default two-pass kernels' bit for bit.  Every test also checks that no bounded
wait of the kernel timed out (the device error word stays 0).
"""
import numpy as np
import pytest
import torch

import oracle
import write_gr_read_amd as gr
from write_gr_read_amd import inputs
from parity import check, check_exact, sample_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def single_pass(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gr.lib()
    gr.device_error_word(reset=True)
    monkeypatch.setenv("GR_KERNEL_VARIANT", "single")
    yield
    torch.cuda.synchronize()
    assert gr.device_error_word() == 0, "a wait of the single-pass kernel timed out"


def orc_read(X, p, dt):
    return oracle.read(X, p.gamma, p.w_down, p.w_up, p.w_write, 1e-6, dt)


def run_case(Xin, label, monkeypatch):
    dt = Xin.dtype
    p0, p1 = Xin.params
    X, y = Xin.X.to(DEV), Xin.y.to(DEV)
    u0, s0 = gr.read(X, p0.to(DEV))
    ou0, os0 = orc_read(Xin.X, p0, dt)
    check(f"{label} read u", u0, ou0, dt)
    check(f"{label} read s", s0, os0, dt)
    s_in = torch.from_numpy(os0).float().to(DEV)
    Xf = X.clone()
    u1, s1 = gr.fused_write_read(Xf, y, s_in, p1.to(DEV))
    oR, ou1, os1 = oracle.fused(Xin.X, Xin.y, os0, p1.gamma, p1.w_down, p1.w_up, p1.w_write, 1e-6, dt)
    check_exact(f"{label} fused state", Xf, oR)
    check(f"{label} fused u", u1, ou1, dt)
    check(f"{label} fused s", s1, os1, dt)
    # the default two-pass kernels on the same inputs: the same stored state
    monkeypatch.delenv("GR_KERNEL_VARIANT")
    Xg = X.clone()
    u2, _ = gr.fused_write_read(Xg, y, s_in, p1.to(DEV))
    monkeypatch.setenv("GR_KERNEL_VARIANT", "single")
    torch.cuda.synchronize()
    assert torch.equal(Xg, Xf), f"{label}: state differs from the two-pass kernels'"
    check(f"{label} u vs two-pass", u1, u2.double().cpu().numpy(), dt)


@pytest.mark.parametrize("N,d,r,w_std,with_write", [
    (1, 4096, 64, 0.02, True), (31, 4096, 64, 0.02, True), (100, 4096, 32, 0.02, True),
    (257, 4096, 48, 0.05, True), (130, 4096, 64, 0.02, False), (300, 4096, 16, 0.3, True),
    (65, 2048, 32, 0.02, True), (700, 2048, 16, 0.05, True), (300, 2048, 64, 0.05, True),
    (2049, 2048, 32, 0.02, True),
])
def test_single_pass_shapes(N, d, r, w_std, with_write, monkeypatch):
    """Several tiles per cluster plus ragged tails (tiles of 32 tokens, 8
    clusters), clusters with no tile, with and without W_write, both slice
    widths (128 and 64 channels per workgroup), gate ranks 16..64."""
    X = inputs.make_gr_inputs(N, 4, d, r, "bf16", seed=N + d + r, w_std=w_std,
                              branch_scale=(1.0, 0.5, 2.0, 1.0), with_write=with_write)
    run_case(X, f"single-N{N}-d{d}-r{r}", monkeypatch)


def test_single_pass_prefill_subset(monkeypatch):
    """The prefill workload's first 1024 tokens, every token compared."""
    run_case(inputs.workload(3, N=1024), "single-prefill-1024", monkeypatch)


def test_single_pass_prefill_full_sampled():
    """The prefill workload at full size (N = 16384), 96 sampled tokens."""
    Xin = inputs.workload(3)
    idx = sample_tokens(Xin.N, 96, seed=13)
    p1 = Xin.params[1]
    X = Xin.X.to(DEV)
    s_in = torch.full((Xin.N, 4), 0.875, device=DEV)
    u, s = gr.fused_write_read(X, Xin.y.to(DEV), s_in, p1.to(DEV))
    oR, ou, os_ = oracle.fused(Xin.X[idx], Xin.y[idx], np.full((len(idx), 4), 0.875), p1.gamma,
                               p1.w_down, p1.w_up, p1.w_write, 1e-6, "bf16")
    check_exact("single-prefill state (sampled)", X.cpu()[idx], oR)
    check("single-prefill u (sampled)", u.cpu()[idx], ou, "bf16")
    check("single-prefill s (sampled)", s.cpu()[idx], os_, "bf16")


def test_single_pass_deterministic():
    X = inputs.make_gr_inputs(1500, 4, 4096, 64, "bf16", seed=71)
    p = X.params[1].to(DEV)
    outs = []
    for _ in range(2):
        R = X.X.to(DEV)
        u, s = gr.fused_write_read(R, X.y.to(DEV), torch.ones(1500, 4, device=DEV), p)
        outs.append((R.cpu(), u.cpu(), s.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_single_pass_graph_replay():
    """Captured once, replayed three times with eager work in between: the
    exchange tags advance on the device, so every replay equals the eager call."""
    X = inputs.make_gr_inputs(600, 4, 4096, 64, "bf16", seed=72)
    p = X.params[1].to(DEV)
    R0, y = X.X.to(DEV), X.y.to(DEV)
    s_in = torch.rand(600, 4, device=DEV) * 2
    Re = R0.clone()
    ue, se = gr.fused_write_read(Re, y, s_in, p)
    Rg, ug, sg = R0.clone(), torch.empty_like(ue), torch.empty_like(se)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gr.fused_write_read(Rg, y, s_in, p, u=ug, s=sg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gr.fused_write_read(Rg, y, s_in, p, u=ug, s=sg)
    for k in range(3):
        Rg.copy_(R0)
        ug.zero_(); sg.zero_()
        gr.fused_write_read(R0.clone(), y, s_in, p)     # an eager call between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Rg, Re) and torch.equal(ug, ue) and torch.equal(sg, se), f"replay {k}"


def test_single_pass_two_streams():
    """Calls queued on two streams at once are ordered by the library (they
    share its device array and each needs every CU): every result equals the
    same call made alone."""
    A = inputs.make_gr_inputs(900, 4, 4096, 64, "bf16", seed=73)
    B = inputs.make_gr_inputs(400, 4, 2048, 32, "bf16", seed=74)
    alone = []
    for Xin in (A, B):
        R = Xin.X.to(DEV)
        u, s = gr.fused_write_read(R, Xin.y.to(DEV), torch.full((Xin.N, 4), 0.9, device=DEV),
                                   Xin.params[1].to(DEV))
        torch.cuda.synchronize()
        alone.append((R, u, s))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for Xin, st in zip((A, B), streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            p = Xin.params[1].to(DEV)
            y = Xin.y.to(DEV)
            s_in = torch.full((Xin.N, 4), 0.9, device=DEV)
            for _ in range(3):
                R = Xin.X.to(DEV)
                u, s = gr.fused_write_read(R, y, s_in, p)
            outs.append((R, u, s))
    torch.cuda.synchronize()
    for (R1, u1, s1), (R2, u2, s2) in zip(alone, outs):
        assert torch.equal(R1, R2) and torch.equal(u1, u2) and torch.equal(s1, s2)
