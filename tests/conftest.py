"""Shared pytest set-up: the ``gpu`` marker and import paths.

Tests marked ``gpu`` call the HIP library through its C ABI and need an MI355X;
everything else (the oracle's pins, input generation, host-side argument
checks, symbol export) runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Margins of the GPU parity checks run in this session (tests/parity.py):
    the worst max|g-o|/RMS(o) and relative L2 error per dtype, and the checks
    with elements past the A13 bound when the combine scale A is left out."""
    try:
        from parity import RECORDS
    except ImportError:
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("parity margins")
    for dt in sorted({r[1] for r in RECORDS}):
        rs = [r for r in RECORDS if r[1] == dt]
        worst_rms = max(rs, key=lambda r: r[2])
        worst_l2 = max(rs, key=lambda r: r[3])
        tr.write_line(f"{dt}: {len(rs)} checks; worst max|g-o|/RMS {worst_rms[2]:.3e} ({worst_rms[0]}); "
                      f"worst relative L2 {worst_l2[3]:.3e} ({worst_l2[0]})")
    strict = [r for r in RECORDS if r[4] > 0]
    tr.write_line(f"checks with elements past 2e-2*max(|o|, RMS/16) (no combine scale): {len(strict)}")
    for r in strict[:40]:
        tr.write_line(f"  {r[0]}: {r[4]} of {r[5]}")
