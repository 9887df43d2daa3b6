"""GPU check of the clock probe (a measurement utility of the library, used
by the benchmark to report the shader clock under load)."""
import pytest
import torch

import combine_router_gating_amd as moe
from gpu_helpers import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_clock_probe_reports_a_plausible_clock():
    log("clock probe: 2 ms")
    out = torch.zeros(2, dtype=torch.int64, device=DEV)
    moe.moe_clock_probe(out, 2000)
    torch.cuda.synchronize()
    cycles, ticks = out.cpu().tolist()
    assert ticks >= 200000  # at least the requested 2 ms of the 100 MHz counter
    assert ticks < 100 * 1000 * 1000  # and far less than a second
    mhz = 100.0 * cycles / ticks
    assert 100.0 < mhz < 3000.0, mhz
