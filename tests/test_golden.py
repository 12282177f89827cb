"""Checks against numbers the pages print (tests/golden/model_shape.json, each
value cited there): the GR module of the described model has n = 4 branches of
width d = 2560 and a gate of rank r = 320 = d/8 ("Qwen3.8-Flash-Next
architecture notes, 06 Residual", sec. 2 and 5; "Paper reading: Qwen3.8 Flash
Next", part 2 Residual, sec. 4), and an FP8 branch state halves the state bytes
of a BF16 one (same notes, sec. 5; same paper reading, sec. 7).  CPU only."""
import ctypes
import json
import os

import pytest

import bench
from write_gr_read_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "model_shape.json")))


def test_the_printed_numbers_agree_with_each_other():
    n, d, r = GOLD["n"], GOLD["d"], GOLD["r"]
    num, den = GOLD["rank_fraction"]
    assert r * den == d * num                      # r = d/8
    assert GOLD["state_width"] == n * d            # 4 x 2560


@pytest.mark.parametrize("k,state", [(7, "bf16"), (8, "fp8")])
def test_model_shape_workloads_use_the_printed_shape(k, state):
    W = inputs.WORKLOADS[k]
    assert (W["n"], W["d"], W["r"]) == (GOLD["n"], GOLD["d"], GOLD["r"])
    assert W["dtype"] == state


def test_fp8_state_halves_the_counted_state_bytes():
    """The roofline's numerator counts the state read and written once per
    token; with one-byte e4m3 words that term is half the bf16 one."""
    n, d, r, N = GOLD["n"], GOLD["d"], GOLD["r"], 1000
    state = {se: bench.algorithmic_bytes(N, n, d, r, 2, True, se) - bench.algorithmic_bytes(N, n, d, r, 2, True, 0)
             for se in (1, 2)}
    assert state[2] == N * 2 * GOLD["state_width"] * 2     # read + write of 2-byte words
    num, den = GOLD["fp8_over_bf16_state_bytes"]
    assert state[1] * den == state[2] * num


@pytest.mark.parametrize("dt", [1, 2])   # GR_BF16, GR_FP8_E4M3
def test_library_takes_the_printed_shape(dt):
    """The workspace query for a fused call at the printed shape succeeds (host
    side only, no kernel runs; the fast path's wide-gate form covers
    r + n = 324)."""
    import write_gr_read_amd as gr
    if not os.path.exists(gr.library_path()):
        pytest.skip("libgr.so not built")
    fake = 1 << 20                                  # non-null, never dereferenced
    lay = gr._Layer(GOLD["n"], GOLD["d"], GOLD["r"], 1e-6, fake, fake, fake, fake)
    nbytes = ctypes.c_size_t(0)
    assert gr.lib().gr_workspace_size(1, dt, 4096, ctypes.byref(lay), ctypes.byref(nbytes)) == 0
    assert nbytes.value > 0
