"""GPU check of the shader-clock probe (sage_sclk_probe), the measurement aid the benchmark reports
next to its timings: every workgroup reports increasing counters and the clock lies within the
part's DPM range (500 - 2400 MHz on MI355X, with some margin)."""

import pytest
import torch

import quantized_attention_quantize_amd as sage
from quantized_attention_quantize_amd import api

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def test_sclk_probe_reports_a_plausible_clock():
    assert torch.cuda.is_available()
    sage.load_library()
    r = api.sclk_probe("cuda", nblocks=256, iters=4000)
    say(f"sclk probe: {r}")
    assert r["workgroups"] == 256
    assert 300.0 <= r["min_mhz"] <= r["median_mhz"] <= r["max_mhz"] <= 3000.0
    assert r["probe_ms"] > 0


def test_idle_sclk_probe_beside_a_kernel():
    """The idle form on a second stream, beside a busy matrix product on the default stream, reports
    a clock in range and covers its sleep window."""
    sage.load_library()
    side = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda")
    out = api.sclk_probe("cuda", nblocks=8, iters=200, load=False, stream=side)
    for _ in range(20):
        a = (a @ a).clamp_(-1, 1)
    torch.cuda.synchronize()
    r = api.sclk_result(out)
    say(f"idle sclk probe: {r}")
    assert r["workgroups"] == 8 and 300.0 <= r["min_mhz"] <= r["max_mhz"] <= 3000.0 and r["probe_ms"] > 0.1
