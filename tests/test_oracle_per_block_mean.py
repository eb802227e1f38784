"""Pins for the oracle's per_block_mean (docs digest, "sageattn3_blackwell" usage: K smoothed by
per-block means instead of the global mean, described there as slightly more accurate).

A block's mean of constant keys is that constant; a constant added to one block's keys leaves its
codes and scales alone and moves only that block's score term; with unit-vector queries the score
terms are the block means themselves; group-query heads equal repeated key/value heads; against
exact attention the emulation stays in budget and, on keys whose channel offsets drift from block
to block, beats smoothing by the global mean.
"""

import numpy as np
import pytest
import torch

from quantized_attention_quantize_amd.synthetic import make_inputs


def _bits(x, dtype=torch.bfloat16):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_block_means_of_constant_blocks(orc):
    d, N = 64, 150  # blocks of 64, 64 and 22 tokens
    K = np.zeros((1, 1, N, d), np.float32)
    vals = [3.25, -7.5, 0.125]
    for u, v in enumerate(vals):
        K[0, 0, 64 * u:64 * u + 64] = v + np.arange(d) / 8.0
    Kb = _bits(K)
    m = orc.block_mean(Kb)
    assert m.shape == (1, 1, 3, d)
    for u, v in enumerate(vals):
        np.testing.assert_array_equal(m[0, 0, u], _f32(Kb[0, 0, 64 * u]))


def test_block_shift_moves_only_that_blocks_term(orc):
    inp = make_inputs(1, 2, 70, 200, 64, seed=80)
    Qb = inp.bits(inp.q)
    rng = np.random.default_rng(8)
    K = (rng.integers(-64, 65, size=(1, 2, 200, 64)) / 8.0).astype(np.float32)  # exact in bf16, also +4
    Kb = _bits(K)
    a = orc.quant_qk(Qb, Kb, per_block_mean=True)
    K2 = K.copy()
    K2[:, :, 64:128] += 4.0
    K2b = _bits(K2)
    assert np.array_equal(_f32(K2b), K2)  # the shifted keys are representable: block 1's mean moves by 4
    b = orc.quant_qk(Qb, K2b, per_block_mean=True)
    assert np.array_equal(a.k8, b.k8) and np.array_equal(a.ks, b.ks) and np.array_equal(a.q8, b.q8)
    assert np.array_equal(a.corr_blk[:, :, [0, 2, 3]], b.corr_blk[:, :, [0, 2, 3]])
    qsum = _f32(Qb).astype(np.float64).sum(-1)  # q . (4, 4, ..., 4) / 4
    np.testing.assert_allclose(b.corr_blk[:, :, 1] - a.corr_blk[:, :, 1], 4.0 * qsum, rtol=0, atol=1e-4)
    assert (a.corr == 0).all()  # the block terms replace the LSE shift


def test_unit_queries_read_the_block_means(orc):
    d, N = 64, 256
    inp = make_inputs(1, 1, d, N, d, seed=81)
    Q = np.eye(d, dtype=np.float32)[None, None]  # query i = e_i
    r = orc.quant_qk(_bits(Q), inp.bits(inp.k), per_block_mean=True)
    m = r.kmean  # [1,1,4,d] block means
    np.testing.assert_array_equal(r.corr_blk[0, 0], m[0, 0])  # corr_blk[u][i] = m_u[i]


def test_gqa_equals_repeated_heads(orc):
    inp = make_inputs(1, 4, 90, 130, 64, seed=82, Hkv=2)
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    g = orc.run_qe(Qb, Kb, Vb, per_block_mean=True, causal=True)
    rep = lambda X: np.ascontiguousarray(np.repeat(X, 2, axis=1))
    r = orc.run_qe(Qb, rep(Kb), rep(Vb), per_block_mean=True, causal=True)
    assert np.array_equal(g.o16, r.o16) and np.array_equal(g.lse, r.lse)


@pytest.mark.parametrize("pv", ["fp16", "fp8"])
def test_per_block_mean_within_budget_and_better_on_drifting_keys(orc, pv):
    N, d = 512, 128
    inp = make_inputs(1, 2, N, N, d, sigma=2.0, seed=83)
    Qb = inp.bits(inp.q)
    rng = np.random.default_rng(5)
    drift = 6.0 * rng.standard_normal((1, 2, N // 64, d)).astype(np.float32)  # a new offset every 64 keys
    K = inp.k.float().numpy() + np.repeat(drift, 64, axis=2)
    Kb, Vb = _bits(K), inp.bits(inp.v)
    eo, el = orc.attn_ex(Qb, Kb, Vb)
    glob = orc.run_qe(Qb, Kb, Vb, pv=pv)
    blk = orc.run_qe(Qb, Kb, Vb, pv=pv, per_block_mean=True)
    e_g = np.abs(glob.o32 - eo).sum() / np.abs(eo).sum()
    e_b = np.abs(blk.o32 - eo).sum() / np.abs(eo).sum()
    assert e_b < (2.5e-2 if pv == "fp16" else 5e-2)
    assert e_b < e_g, (e_b, e_g)
    assert np.abs(blk.lse - el).max() < 2e-2
