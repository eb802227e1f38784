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
