"""Pins for the oracle's handling of non-finite inputs (NaN, and infinities that turn into NaN):
each planted value must reach exactly the outputs that the policy's reach sets (tests/nonfinite.py)
name, and every other output must equal the result without it, bit for bit.  The sets are written
from the policy's statement, not from the oracle, so a NaN the oracle drops (a skipped tile, a
maximum that ignores NaN, a zero scale) or spreads too far fails here."""

import numpy as np
import pytest
import torch

from quantized_attention_quantize_amd.synthetic import make_inputs, random_mask

import nonfinite as nf

N, H, D = 300, 2, 64  # five 64-token blocks with a ragged tail of 44; two 256-row blocks
NAN16 = {"bf16": np.uint16(0x7FC0), "fp16": np.uint16(0x7E00)}
INF16 = {"bf16": np.uint16(0x7F80), "fp16": np.uint16(0x7C00)}


def _inputs(dtype="bf16", seed=90):
    inp = make_inputs(1, H, N, N, D, sigma=4.0, seed=seed, dtype=torch.float16 if dtype == "fp16" else torch.bfloat16)
    return inp.bits(inp.q).copy(), inp.bits(inp.k).copy(), inp.bits(inp.v).copy()


def _plant(X, h, i, c, val):
    Y = X.copy()
    Y[0, h, i, c] = val
    return Y


def _o(r, dtype="bf16"):
    """o32 [H, N, d] and lse [H, N] of a run_qe result over all rows."""
    return r.o32.reshape(H, N, D), r.lse.reshape(H, N)


def _same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def _check_rows(o1, l1, o0, l0, nan_rows):
    """Rows nan_rows (bool [H, N]) are NaN in O and LSE; all others equal the clean run exactly."""
    assert np.isnan(o1[nan_rows]).all() and np.isnan(l1[nan_rows]).all()
    keep = ~nan_rows
    assert _same_bits(o1[keep], o0[keep]) and _same_bits(l1[keep], l0[keep])


def _check_channel(o1, l1, o0, l0, c, nan_rows):
    """Channel c of rows nan_rows (bool [H, N]) is NaN; every other element of O and all of the LSE
    equal the clean run exactly."""
    assert np.isnan(o1[..., c][nan_rows]).all()
    want = np.isnan(o0).copy()
    want[..., c] |= nan_rows
    assert np.array_equal(np.isnan(o1), want)
    assert _same_bits(o1[~want], o0[~want]) and _same_bits(l1, l0)


# ---- quantization ----------------------------------------------------------------------------
@pytest.mark.parametrize("val", ["nan", "inf"])
def test_quant_q_nonfinite_poisons_its_block(orc, val):
    Q, K, _ = _inputs()
    i0 = 130  # block 2
    Q1 = _plant(Q, 1, i0, 7, NAN16["bf16"] if val == "nan" else INF16["bf16"])
    a, b = orc.quant_qk(Q, K), orc.quant_qk(Q1, K)
    u = i0 // 64
    assert (np.isnan(b.qs[0, 1, u]) if val == "nan" else np.isposinf(b.qs[0, 1, u]))
    assert not b.q8[0, 1, u * 64:(u + 1) * 64].any()  # every code of the block is 0
    blk = np.zeros(b.qs.shape, bool)
    blk[0, 1, u] = True
    assert _same_bits(b.qs[~blk], a.qs[~blk])
    rows = np.ones(b.q8.shape[:3], bool)
    rows[0, 1, u * 64:(u + 1) * 64] = False
    assert np.array_equal(b.q8[rows], a.q8[rows])
    assert np.array_equal(b.k8, a.k8) and _same_bits(b.ks, a.ks)


def test_quant_k_nan_poisons_the_head_mean(orc):
    Q, K, _ = _inputs()
    K1 = _plant(K, 0, 77, 5, NAN16["bf16"])
    a, b = orc.quant_qk(Q, K), orc.quant_qk(Q, K1)
    assert np.isnan(b.kmean[0, 0, 5]) and np.isnan(b.kmean[0, 0]).sum() == 1
    assert np.isnan(b.ks[0, 0]).all() and not b.k8[0, 0].any()
    assert np.isnan(b.corr[0, 0]).all()  # the LSE shift q . kmean of every row of head 0
    assert _same_bits(b.ks[0, 1], a.ks[0, 1]) and np.array_equal(b.k8[0, 1], a.k8[0, 1])
    assert np.array_equal(b.q8, a.q8) and _same_bits(b.corr[0, 1], a.corr[0, 1])


def test_quant_k_nan_per_block_mean_poisons_its_block(orc):
    Q, K, _ = _inputs()
    j0 = 200  # block 3
    K1 = _plant(K, 1, j0, 9, NAN16["bf16"])
    a, b = orc.quant_qk(Q, K, per_block_mean=True), orc.quant_qk(Q, K1, per_block_mean=True)
    u = j0 // 64
    assert np.isnan(b.kmean[0, 1, u, 9]) and np.isnan(b.kmean).sum() == 1
    assert np.isnan(b.ks[0, 1, u]) and np.isnan(b.ks).sum() == 1
    assert not b.k8[0, 1, u * 64:(u + 1) * 64].any()
    assert np.isnan(b.corr_blk[0, 1, u]).all() and np.isnan(b.corr_blk).sum() == N
    other = np.ones(b.k8.shape[:3], bool)
    other[0, 1, u * 64:(u + 1) * 64] = False
    assert np.array_equal(b.k8[other], a.k8[other])


def test_prep_v_nan(orc):
    _, _, V = _inputs()
    V1 = _plant(V, 0, 33, 11, NAN16["bf16"])
    h16, _ = orc.prep_v(V1, "fp16")
    c16, _ = orc.prep_v(V, "fp16")
    assert np.isnan(orc.f16_to_f32(h16[0, 0, 33, 11])).all()
    diff = h16 != c16
    assert diff.sum() == 1 and diff[0, 0, 33, 11]
    h8, s8 = orc.prep_v(V1, "fp8")
    c8, cs8 = orc.prep_v(V, "fp8")
    assert np.isnan(s8[0, 0, 11]) and np.isnan(s8).sum() == 1
    assert not h8[0, 0, :, 11].any()  # every code of the NaN channel is 0
    other = np.ones(h8.shape, bool)
    other[0, 0, :, 11] = False
    assert np.array_equal(h8[other], c8[other])
    # smooth_v: the channel mean is NaN
    vm = orc.kmean(V1)
    assert np.isnan(vm[0, 0, 11]) and np.isnan(vm).sum() == 1


# ---- the quantized emulation ---------------------------------------------------------------
def _vis(causal, mask):
    return nf.visible(N, N, causal, None if mask is None else mask[0, 0])


CASES = [(False, None), (True, None), (False, "mask"), (True, "mask")]


def _mask(kind):
    if kind is None:
        return None
    m = random_mask(1, 1, N, N, p_keep=0.5, seed=91).numpy()
    m[0, 0, 5] = False  # a row without any visible key
    m[0, 0, :, 64:128] = False  # a key tile masked for every row
    return m.astype(np.uint8)


@pytest.mark.parametrize("causal,mk", CASES)
@pytest.mark.parametrize("val", ["nan", "inf"])
def test_qe_q_nonfinite(orc, causal, mk, val):
    Q, K, V = _inputs()
    m = _mask(mk)
    i0 = 70
    Q1 = _plant(Q, 0, i0, 3, NAN16["bf16"] if val == "nan" else INF16["bf16"])
    o0, l0 = _o(orc.run_qe(Q, K, V, causal=causal, mask=m, tau=8.0))
    o1, l1 = _o(orc.run_qe(Q1, K, V, causal=causal, mask=m, tau=8.0))
    rows = np.zeros((H, N), bool)
    rows[0] = nf.reach_q(_vis(causal, m), i0)
    _check_rows(o1, l1, o0, l0, rows)
    if mk is not None:  # the row without keys stays O = 0, LSE = -inf
        assert (o1[0, 5] == 0).all() and np.isneginf(l1[0, 5])


@pytest.mark.parametrize("causal,mk", CASES)
@pytest.mark.parametrize("pbm", [False, True])
def test_qe_k_nan(orc, causal, mk, pbm):
    Q, K, V = _inputs()
    m = _mask(mk)
    j0 = 150
    K1 = _plant(K, 1, j0, 6, NAN16["bf16"])
    o0, l0 = _o(orc.run_qe(Q, K, V, causal=causal, mask=m, per_block_mean=pbm))
    o1, l1 = _o(orc.run_qe(Q, K1, V, causal=causal, mask=m, per_block_mean=pbm))
    vis = _vis(causal, m)
    rows = np.zeros((H, N), bool)
    rows[1] = nf.reach_k_block(vis, j0) if pbm else nf.reach_k_head(vis)
    _check_rows(o1, l1, o0, l0, rows)


@pytest.mark.parametrize("causal,mk", CASES)
@pytest.mark.parametrize("pv,smooth_v", [("fp16", False), ("fp8", False), ("fp16", True)])
def test_qe_v_nan(orc, causal, mk, pv, smooth_v):
    Q, K, V = _inputs()
    m = _mask(mk)
    j0, c0 = 140, 21
    V1 = _plant(V, 0, j0, c0, NAN16["bf16"])
    kw = dict(causal=causal, mask=m, pv=pv, smooth_v=smooth_v, tau=0.0 if pv == "fp8" else 8.0)
    o0, l0 = _o(orc.run_qe(Q, K, V, **kw))
    o1, l1 = _o(orc.run_qe(Q, K, V1, **kw))
    vis = _vis(causal, m)
    rows = np.zeros((H, N), bool)
    if pv == "fp16" and not smooth_v:
        rows[0] = nf.reach_v16(vis, j0, causal, "oracle", None if m is None else m[0, 0])
        assert (rows[0] >= nf.must_v(vis, j0)).all()
    else:  # the channel's scale or mean
        rows[0] = nf.live_rows(vis)
    _check_channel(o1, l1, o0, l0, c0, rows)


def test_qe_all_rows_keyless_ignore_nan_v(orc):
    """With every key masked, O = 0 and LSE = -inf even though V holds a NaN in every tile."""
    Q, K, V = _inputs()
    V1 = V.copy()
    V1[0, 0, ::64, 0] = NAN16["bf16"]
    m = np.zeros((1, 1, N, N), np.uint8)
    r = orc.run_qe(Q, K, V1, mask=m)
    assert (r.o32 == 0).all() and np.isneginf(r.lse).all()


# ---- exact attention and the merge --------------------------------------------------------------
@pytest.mark.parametrize("where", ["q", "k", "v"])
def test_exact_nan_reaches_what_depends_on_it(orc, where):
    Q, K, V = _inputs()
    n = 96
    Q, K, V = Q[:, :, :n].copy(), K[:, :, :n].copy(), V[:, :, :n].copy()
    i0 = 40
    X = {"q": Q, "k": K, "v": V}[where]
    X1 = _plant(X, 0, i0, 2, NAN16["bf16"])
    args = {"q": (X1, K, V), "k": (Q, X1, V), "v": (Q, K, X1)}[where]
    o0, l0 = orc.attn_ex(Q, K, V, causal=True)
    o1, l1 = orc.attn_ex(*args, causal=True)
    o0, o1 = o0.reshape(H, n, D), o1.reshape(H, n, D)
    l0, l1 = l0.reshape(H, n), l1.reshape(H, n)
    rows = np.zeros((H, n), bool)
    if where == "q":
        rows[0, i0] = True
    else:
        rows[0, i0:] = True  # the rows that see key i0
    if where == "v":
        assert np.isnan(o1[..., 2][rows]).all()
        want = np.zeros(o1.shape, bool)
        want[..., 2] = rows
        assert np.array_equal(np.isnan(o1), want) and np.array_equal(l1, l0)
        assert np.array_equal(o1[~want], o0[~want])
    else:
        assert np.isnan(o1[rows]).all() and np.isnan(l1[rows]).all()
        assert np.array_equal(o1[~rows], o0[~rows]) and np.array_equal(l1[~rows], l0[~rows])


def test_merge_nan_and_empty_parts(orc):
    rng = np.random.default_rng(92)
    S, R, d = 3, 6, 8
    o = rng.standard_normal((S, R, d)).astype(np.float32)
    lse = rng.standard_normal((S, R)).astype(np.float32)
    lse[1, 0] = np.nan  # a NaN part poisons its row
    lse[:, 1] = -np.inf  # no part sees a key
    o[:, 1] = np.nan  # ... and the parts' O are never read
    lse[2, 2] = -np.inf  # an empty part among live ones
    o[2, 2] = np.nan
    o[0, 3, 4] = np.nan  # a NaN in one live part's O reaches that element
    out, L = orc.merge_lse(o, lse)
    assert np.isnan(out[0]).all() and np.isnan(L[0])
    assert (out[1] == 0).all() and np.isneginf(L[1])
    assert np.isfinite(out[2]).all() and np.isfinite(L[2])
    want2, wl2 = orc.merge_lse(o[:2, 2:3], lse[:2, 2:3])  # the same as merging the live parts alone
    assert np.allclose(out[2], want2[0], rtol=1e-12, atol=0) and np.isclose(L[2], wl2[0], rtol=1e-12)
    assert np.isnan(out[3, 4]) and np.isfinite(np.delete(out[3], 4)).all() and np.isfinite(L[3])
