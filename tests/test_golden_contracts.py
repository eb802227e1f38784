"""The pages' stated contracts (tests/golden/page_contracts.json) checked on the oracle."""

import json
import os

import numpy as np

from quantized_attention_quantize_amd.synthetic import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_contracts.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_sm_scale_default(orc):
    g = load()["sm_scale_default"]["values_fp32"]
    for d, v in g.items():
        assert orc.default_sm_scale(int(d)) == np.float32(v)


def test_oracle_shapes_follow_page_contracts(orc):
    # the same ranks and the LSE-drops-the-head-dim rule on a reduced token count
    for case in load()["shapes"]:
        B, H, _, d = case["q"]
        N = 64
        inp = make_inputs(B, H, N, N, d, seed=0)
        rows = np.arange(0, B * H * N, 97, dtype=np.int64)
        r = orc.run_qe(inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v), rows=rows)
        assert r.o16.shape == (rows.size, d) and r.lse.shape == (rows.size,)
        if "lse" in case:
            assert case["lse"] == case["q"][:3]
        assert case["out"] == case["q"]


def test_mask_semantics_false_is_masked(orc):
    inp = make_inputs(1, 1, 64, 128, 64, seed=1, mask="half_keys")
    m = inp.mask_u8
    assert m[0, 0, 0, 63] == 1 and m[0, 0, 0, 64] == 0
    o_mask, _ = orc.attn_ex(inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v), mask=m)
    o_half, _ = orc.attn_ex(inp.bits(inp.q), inp.bits(inp.k)[:, :, :64].copy(), inp.bits(inp.v)[:, :, :64].copy())
    np.testing.assert_allclose(o_mask, o_half, atol=1e-13)
