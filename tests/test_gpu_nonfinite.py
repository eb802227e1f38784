"""GPU test of the library's rule for non-finite inputs: a NaN (or an infinity) planted in one Q
row, one K row or one V element reaches exactly the outputs that the rule's reach sets
(tests/nonfinite.py, the GPU key loop) name, and every other element of O and the LSE is bit for bit
what the same call gives without it.  The quantization of the planted inputs is compared with the
oracle's: codes and finite scales bit-exact, NaN scales in the same places.  The merge kernel keeps
a NaN LSE and ignores the O of a part without keys."""

import numpy as np
import pytest
import torch

import quantized_attention_quantize_amd as sage
from quantized_attention_quantize_amd.synthetic import additive_mask, make_inputs, random_mask

import nonfinite as nf
from gpu_helpers import DEV, say, unpermute_vt

pytestmark = pytest.mark.gpu

N, H, D = 300, 2, 128  # five key tiles (ragged tail of 44) and two 256-row query blocks


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sage.load_library()


def _inputs(seed=95):
    return make_inputs(1, H, N, N, D, sigma=4.0, seed=seed)


def _plant(t, h, i, c, val):
    u = t.clone()
    u[0, h, i, c] = val
    return u


def _mask(kind):
    if kind is None:
        return None
    m = random_mask(1, 1, N, N, p_keep=0.5, seed=96)
    m[0, 0, 5] = False  # a row without a visible key
    m[0, 0, :, 64:128] = False  # a tile hidden from every row
    m[0, 0, :256, 256:] = False  # the last tile hidden from the first query block only
    return additive_mask(m) if kind == "f32" else m


def _bool(mask):
    if mask is None:
        return None
    m = mask[0, 0].numpy()
    return m != -np.inf if m.dtype == np.float32 else m.astype(bool)


def _run(q, k, v, causal, mask, **kw):
    o, lse = sage.sageattn(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=causal,
                           attn_mask=None if mask is None else mask.to(DEV), return_lse=True, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()[0], lse.cpu().numpy()[0]


def _bits32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _check_rows(o1, l1, o0, l0, rows):
    assert np.isnan(o1[rows]).all() and np.isnan(l1[rows]).all(), "planted NaN missing from a reached row"
    keep = ~rows
    assert not np.isnan(o1[keep]).any() and not np.isnan(l1[keep]).any(), "NaN outside the reached rows"
    assert np.array_equal(_bits32(o1[keep]), _bits32(o0[keep])) and np.array_equal(_bits32(l1[keep]), _bits32(l0[keep]))


def _check_channel(o1, l1, o0, l0, c, rows):
    want = np.zeros(o1.shape, bool)
    want[..., c] = rows
    assert np.array_equal(np.isnan(o1), want), "NaN set differs from the reach set"
    assert np.array_equal(_bits32(o1[~want]), _bits32(o0[~want])) and np.array_equal(_bits32(l1), _bits32(l0))


MASKS = [(False, None), (True, None), (False, "bool"), (True, "bool"), (False, "f32")]
MASK_IDS = ["plain", "causal", "mask", "causal_mask", "fmask"]


@pytest.mark.parametrize("causal,mk", MASKS, ids=MASK_IDS)
@pytest.mark.parametrize("val", ["nan", "inf"])
def test_q_nonfinite(causal, mk, val):
    say(f"non-finite Q {val} causal={causal} mask={mk}")
    inp, m = _inputs(), _mask(mk)
    i0 = 70
    q1 = _plant(inp.q, 0, i0, 3, float(val))
    o0, l0 = _run(inp.q, inp.k, inp.v, causal, m)
    o1, l1 = _run(q1, inp.k, inp.v, causal, m)
    rows = np.zeros((H, N), bool)
    rows[0] = nf.reach_q(nf.visible(N, N, causal, _bool(m)), i0)
    _check_rows(o1, l1, o0, l0, rows)
    if mk is not None:
        assert (o1[0, 5] == 0).all() and np.isneginf(l1[0, 5])


@pytest.mark.parametrize("causal,mk", MASKS, ids=MASK_IDS)
@pytest.mark.parametrize("pbm", [False, True], ids=["head_mean", "block_mean"])
def test_k_nan(causal, mk, pbm):
    if pbm and mk == "f32":
        pytest.skip("the float mask and per_block_mean are not combined")
    say(f"non-finite K causal={causal} mask={mk} per_block_mean={pbm}")
    inp, m = _inputs(), _mask(mk)
    j0 = 150
    k1 = _plant(inp.k, 1, j0, 6, float("nan"))
    o0, l0 = _run(inp.q, inp.k, inp.v, causal, m, per_block_mean=pbm)
    o1, l1 = _run(inp.q, k1, inp.v, causal, m, per_block_mean=pbm)
    vis = nf.visible(N, N, causal, _bool(m))
    rows = np.zeros((H, N), bool)
    rows[1] = nf.reach_k_block(vis, j0) if pbm else nf.reach_k_head(vis)
    _check_rows(o1, l1, o0, l0, rows)


@pytest.mark.parametrize("causal,mk", MASKS, ids=MASK_IDS)
@pytest.mark.parametrize("pv,smooth_v", [("fp16", False), ("fp8", False), ("fp16", True)],
                         ids=["fp16", "fp8", "smooth_v"])
@pytest.mark.parametrize("j0", [140, 270])
def test_v_nan(causal, mk, pv, smooth_v, j0):
    say(f"non-finite V key {j0} {pv} smooth_v={smooth_v} causal={causal} mask={mk}")
    inp, m = _inputs(), _mask(mk)
    c0 = 21
    v1 = _plant(inp.v, 0, j0, c0, float("nan"))
    o0, l0 = _run(inp.q, inp.k, inp.v, causal, m, pv_dtype=pv, smooth_v=smooth_v)
    o1, l1 = _run(inp.q, inp.k, v1, causal, m, pv_dtype=pv, smooth_v=smooth_v)
    bm = _bool(m)
    vis = nf.visible(N, N, causal, bm)
    rows = np.zeros((H, N), bool)
    if pv == "fp16" and not smooth_v:
        rows[0] = nf.reach_v16(vis, j0, causal, "kernel", bm)
        assert (rows[0] >= nf.must_v(vis, j0)).all()
    else:
        rows[0] = nf.live_rows(vis)
    _check_channel(o1, l1, o0, l0, c0, rows)


def test_quantization_of_nonfinite_inputs_vs_oracle(orc):
    """NaN in a Q row, +inf in another Q block, NaN in a K row: codes bit-exact with the oracle,
    scales equal where finite and NaN / inf in the same places; the K mean likewise."""
    inp = _inputs()
    q = _plant(_plant(inp.q, 0, 70, 3, float("nan")), 1, 200, 9, float("inf"))
    k = _plant(inp.k, 1, 150, 6, float("nan"))
    for pbm in (False, True):
        say(f"non-finite quantization per_block_mean={pbm}")
        g = sage.quantize_qk(q.to(DEV), k.to(DEV), per_block_mean=pbm)
        torch.cuda.synchronize()
        c = orc.quant_qk(inp.bits(q), inp.bits(k), per_block_mean=pbm)
        assert np.array_equal(g.q8.cpu().numpy(), c.q8) and np.array_equal(g.k8.cpu().numpy(), c.k8)
        for got, want in ((g.q_scale, c.qs), (g.k_scale, c.ks), (g.k_block_mean if pbm else g.k_mean, c.kmean)):
            got = got.cpu().numpy()
            got = got[:, :, :want.shape[2]] if got.ndim == 4 else got  # block means past the last block
            assert np.array_equal(np.isnan(got), np.isnan(want))
            fin = ~np.isnan(want)
            assert np.array_equal(_bits32(got[fin]), _bits32(want[fin]))
        assert np.isnan(c.qs[0, 0, 1]) and np.isposinf(c.qs[0, 1, 3])


@pytest.mark.parametrize("pv", ["fp16", "fp8"])
def test_prepare_v_of_nan_vs_oracle(orc, pv):
    say(f"non-finite prepare_v {pv}")
    inp = _inputs()
    v = _plant(inp.v, 0, 140, 21, float("nan"))
    vt, vs = sage.prepare_v(v.to(DEV), pv)
    torch.cuda.synchronize()
    want, want_s = orc.prep_v(inp.bits(v), pv)
    got = vt.cpu().numpy()
    nat = unpermute_vt(got.view(np.uint16) if pv == "fp16" else got, pv)[:, :, :N]
    if pv == "fp16":  # one NaN element; its payload is not part of the rule
        gf = nat.view(np.float16)
        wf = want.view(np.float16)
        assert np.array_equal(np.isnan(gf), np.isnan(wf)) and np.isnan(wf).sum() == 1
        assert np.array_equal(nat[~np.isnan(wf)], want[~np.isnan(wf)])
    else:
        assert np.array_equal(nat, want) and not nat[0, 0, :, 21].any()
        s = vs.cpu().numpy()
        assert np.array_equal(np.isnan(s), np.isnan(want_s)) and np.isnan(s[0, 0, 21])
        fin = ~np.isnan(want_s)
        assert np.array_equal(_bits32(s[fin]), _bits32(want_s[fin]))


def test_merge_nan_and_empty_parts(orc):
    say("non-finite merge")
    g = torch.Generator().manual_seed(97)
    S, B, Hh, Nq, d = 3, 1, 2, 5, 64
    o = torch.randn(S, B, Hh, Nq, d, generator=g)
    lse = torch.randn(S, B, Hh, Nq, generator=g)
    lse[1, 0, 0, 0] = float("nan")  # a NaN part poisons its row
    lse[:, 0, 0, 1] = -float("inf")  # no part saw a key ...
    o[:, 0, 0, 1] = float("nan")  # ... and their O is never read
    lse[2, 0, 0, 2] = -float("inf")  # an empty part among live ones
    o[2, 0, 0, 2] = float("nan")
    o[0, 0, 0, 3, 4] = float("nan")  # a NaN in one part's O reaches that element
    out, ml = sage.merge_lse(o.to(DEV), lse.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, ml = out.cpu().numpy()[0, 0], ml.cpu().numpy()[0, 0]
    wo, wl = orc.merge_lse(o.numpy().reshape(S, -1, d), lse.numpy().reshape(S, -1))
    wo, wl = wo.reshape(Hh, Nq, d)[0], wl.reshape(Hh, Nq)[0]
    assert np.array_equal(np.isnan(out), np.isnan(wo)) and np.array_equal(np.isnan(ml), np.isnan(wl))
    assert np.isnan(out[0]).all() and np.isnan(ml[0])
    assert (out[1] == 0).all() and np.isneginf(ml[1])
    assert np.isnan(out[3, 4]) and np.isnan(out).sum() == d + 1
    fin = ~np.isnan(wo)
    np.testing.assert_allclose(out[fin], wo[fin], rtol=1e-5, atol=1e-6)
