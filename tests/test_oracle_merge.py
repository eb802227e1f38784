"""Pins for the oracle's merge of partial attention results (the LSE output's purpose on the
SageAttention docs digest, "Utilize SageAttention for Distributed Inference").

Merging exact attention over disjoint key sets gives exact attention over their union (causal
splits included, where whole parts are invisible to some rows); one part is the identity; parts
with equal LSEs average; the order of the parts does not matter; a split of smoothed, quantized
attention over key slices (each slice with its own K mean) stays within the quantization budget of
exact attention.
"""

import numpy as np
import pytest

from quantized_attention_quantize_amd.synthetic import make_inputs


def _keys_mask(B, Nq, Nk, lo, hi, causal):
    m = np.zeros((B, 1, Nq, Nk), np.uint8)
    m[..., lo:hi] = 1
    if causal:
        m &= np.tril(np.ones((Nq, Nk), np.uint8))[None, None]
    return m


@pytest.mark.parametrize("cuts,causal", [((0, 100, 230), False), ((0, 64, 128, 230), True), ((0, 1, 230), False)])
def test_merge_of_exact_parts_is_exact(orc, cuts, causal):
    B, H, Nq, Nk, d = 2, 2, 150, 230, 64
    inp = make_inputs(B, H, Nq, Nk, d, seed=21)
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    full_o, full_l = orc.attn_ex(Qb, Kb, Vb, causal=causal)
    parts = [orc.attn_ex(Qb, Kb, Vb, mask=_keys_mask(B, Nq, Nk, lo, hi, causal))
             for lo, hi in zip(cuts[:-1], cuts[1:])]
    o, l = orc.merge_lse(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    if causal:  # rows before a part's first key see nothing of it
        assert np.isneginf(parts[-1][1]).any()
    np.testing.assert_allclose(o, full_o, rtol=0, atol=2e-6)  # the parts travel as fp32
    np.testing.assert_allclose(l, full_l, rtol=0, atol=1e-6)


def test_merge_single_part_and_empty_rows(orc):
    rng = np.random.default_rng(0)
    o = rng.standard_normal((1, 50, 64)).astype(np.float32)
    lse = rng.standard_normal((1, 50)).astype(np.float32)
    lse[0, 7] = -np.inf
    o[0, 7] = 0
    mo, ml = orc.merge_lse(o, lse)
    np.testing.assert_allclose(mo, o[0], rtol=0, atol=1e-12)
    assert np.isneginf(ml[7]) and (mo[7] == 0).all()
    np.testing.assert_allclose(ml[np.isfinite(ml)], lse[0][np.isfinite(lse[0])], atol=1e-12)


def test_merge_equal_lse_averages_and_is_order_free(orc):
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 40, 128)).astype(np.float32)
    lse = np.full((3, 40), 2.5, np.float32)
    mo, ml = orc.merge_lse(o, lse)
    np.testing.assert_allclose(mo, o.astype(np.float64).mean(0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, 2.5 + np.log(3.0), rtol=0, atol=1e-12)
    lse2 = rng.standard_normal((3, 40)).astype(np.float32) * 4
    a = orc.merge_lse(o, lse2)
    perm = [2, 0, 1]
    b = orc.merge_lse(o[perm], lse2[perm])
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("pv", ["fp16", "fp8"])
def test_split_kv_quantized_parts_within_budget(orc, pv):
    """Key slices run the whole quantized method on their own (own K mean, own blocks); merged, they
    stay within the quantization budget of exact attention over all keys."""
    B, H, N, d = 1, 2, 512, 128
    inp = make_inputs(B, H, N, N, d, sigma=4.0 if pv == "fp16" else 8.0, seed=22)
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    cut = 320
    parts = [orc.run_qe(Qb, np.ascontiguousarray(Kb[:, :, lo:hi]), np.ascontiguousarray(Vb[:, :, lo:hi]), pv=pv)
             for lo, hi in ((0, cut), (cut, N))]
    o, l = orc.merge_lse(np.stack([p.o32 for p in parts]), np.stack([p.lse for p in parts]))
    eo, el = orc.attn_ex(Qb, Kb, Vb)
    rel = np.abs(o - eo).sum() / np.abs(eo).sum()
    assert rel < (2.5e-2 if pv == "fp16" else 5e-2), rel
    assert np.abs(l - el).max() < 2e-2
