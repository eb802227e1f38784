"""GPU parity on small and ragged shapes: the HIP path through the C ABI against the CPU oracle.

Bit-exact: K mean, int8 Q/K codes, their scales, the prepared V (fp16 / e4m3 bytes and the e4m3
per-channel scale) and the int32 Q8.K8^T scores, from bf16 and from fp16 inputs.  Tolerance: O
within relative L1 1e-3 of the oracle's quantized emulation (both rounded to the output dtype) and
LSE within 1e-3; against fp64 exact attention, cosine >= 0.999 and relative L1 <= 3e-2 for FP16
PV.  Masks: boolean and float32 additive.
"""

import dataclasses

import numpy as np
import pytest
import torch

import quantized_attention_quantize_amd as sage
from quantized_attention_quantize_amd import api
from quantized_attention_quantize_amd.synthetic import (additive_mask, make_inputs, random_additive_mask,
                                                        random_mask)

from gpu_helpers import (DEV, TAU, assert_lse_close, bits, check_o, cosine, f32_of_bf16_bits, lse_rows, qe_schedule,
                         rel_l1, rows_of, say, to_dev, unpermute_vt)

pytestmark = pytest.mark.gpu

QE_REL_L1 = 1e-3  # output vs quantized emulation: the relative-L1 parity bar
QE_LSE = 1e-3
EX_COS = 0.999
EX_REL_L1 = 3e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sage.load_library()  # raises loudly if the HIP library is missing


SHAPES = [(1, 2, 256, 256, 64), (1, 1, 1, 1, 64), (1, 2, 63, 63, 128), (2, 1, 65, 65, 128), (1, 2, 129, 300, 64),
          (1, 3, 300, 129, 128), (2, 2, 64, 64, 64), (1, 1, 700, 1000, 128)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("B,H,Nq,Nk,d", SHAPES)
def test_quantize_bitexact(orc, B, H, Nq, Nk, d, dtype):
    say(f"quantize B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dtype}")
    inp = make_inputs(B, H, Nq, Nk, d, sigma=4.0, seed=3, dtype=dtype)
    q, k, v = to_dev(inp)
    g = sage.quantize_qk(q, k)
    torch.cuda.synchronize()
    c = orc.quant_qk(inp.bits(inp.q), inp.bits(inp.k), dtype=inp.dtype)
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), c.kmean.view(np.uint32))
    assert np.array_equal(g.q8.cpu().numpy(), c.q8)
    assert np.array_equal(g.k8.cpu().numpy(), c.k8)
    assert np.array_equal(g.q_scale.cpu().numpy().view(np.uint32), c.qs.view(np.uint32))
    assert np.array_equal(g.k_scale.cpu().numpy().view(np.uint32), c.ks.view(np.uint32))
    np.testing.assert_allclose(g.lse_corr.cpu().numpy(), c.corr, rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", [(1, 4, 2, 300, 417, 128), (2, 6, 1, 129, 65, 64)])
def test_quantize_bitexact_gqa(orc, B, H, Hkv, Nq, Nk, d):
    """Group-query attention: K has Hkv heads; each query head's LSE shift uses its key head's mean."""
    say(f"quantize gqa B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d}")
    inp = gqa_inputs(make_inputs(B, H, Nq, Nk, d, sigma=4.0, seed=5), Hkv)
    q, k, v = to_dev(inp)
    g = sage.quantize_qk(q, k)
    torch.cuda.synchronize()
    c = orc.quant_qk(inp.bits(inp.q), inp.bits(inp.k))
    assert g.k8.shape[1] == Hkv and g.Hkv == Hkv
    assert np.array_equal(g.k_mean.cpu().numpy().view(np.uint32), c.kmean.view(np.uint32))
    assert np.array_equal(g.q8.cpu().numpy(), c.q8) and np.array_equal(g.k8.cpu().numpy(), c.k8)
    assert np.array_equal(g.q_scale.cpu().numpy().view(np.uint32), c.qs.view(np.uint32))
    assert np.array_equal(g.k_scale.cpu().numpy().view(np.uint32), c.ks.view(np.uint32))
    np.testing.assert_allclose(g.lse_corr.cpu().numpy(), c.corr, rtol=2e-6, atol=2e-6)
    # the debug scores of the last query head come from its own key head
    got = sage.debug_qk_int32(g, B - 1, H - 1, 0, min(Nq, 64), 0, min(Nk, 64)).cpu().numpy()
    hk = (H - 1) // (H // Hkv)
    want = orc.scores(c.q8[:, H - 1:H], c.k8[:, hk:hk + 1], B - 1, 0, 0, min(Nq, 64), 0, min(Nk, 64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", [(1, 2, 2, 300, 417, 128), (2, 4, 2, 129, 65, 64), (1, 1, 1, 700, 1000, 128),
                                             (1, 2, 2, 1100, 2500, 128), (1, 4, 2, 8192, 2500, 64)])
def test_quantize_per_block_mean(orc, B, H, Hkv, Nq, Nk, d, dtype):
    """per_block_mean: block means, codes and scales bit-exact; the score terms within fp32
    accumulation of the oracle's fp64 dot products; the global mean and the LSE shift zero.  The
    last two shapes have 40 key blocks (a second, partial group of 32 for the score kernel), the
    last one two 32-row blocks per wave."""
    say(f"quantize per_block_mean B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype}")
    inp = make_inputs(B, H, Nq, Nk, d, sigma=4.0, seed=9, dtype=dtype)
    if Hkv != H:
        inp = gqa_inputs(inp, Hkv)
    q, k, v = to_dev(inp)
    g = sage.quantize_qk(q, k, per_block_mean=True)
    torch.cuda.synchronize()
    c = orc.quant_qk(inp.bits(inp.q), inp.bits(inp.k), dtype=inp.dtype, per_block_mean=True)
    assert np.array_equal(g.k_block_mean.cpu().numpy().view(np.uint32), c.kmean.view(np.uint32))
    assert np.array_equal(g.q8.cpu().numpy(), c.q8) and np.array_equal(g.k8.cpu().numpy(), c.k8)
    assert np.array_equal(g.q_scale.cpu().numpy(), c.qs) and np.array_equal(g.k_scale.cpu().numpy(), c.ks)
    assert not g.k_mean.any() and not g.lse_corr.any()
    gc = g.blk_corr.cpu().numpy()
    scale = np.abs(c.corr_blk).max() + 1e-30
    assert np.abs(gc - c.corr_blk).max() <= 2e-6 * scale * d ** 0.5


def test_per_block_mean_beats_global_mean_on_drifting_keys(orc):
    """Keys whose channel offsets change every 64 tokens: per-block smoothing is closer to exact
    attention than smoothing by the global mean (the GPU path against the oracle's exact path)."""
    B, H, N, d = 1, 2, 512, 128
    inp = make_inputs(B, H, N, N, d, sigma=2.0, seed=19)
    g = torch.Generator().manual_seed(4)
    drift = 6.0 * torch.randn(B, H, N // 64, 1, d, generator=g)
    k = (inp.k.float().reshape(B, H, N // 64, 64, d) + drift).reshape(B, H, N, d).to(torch.bfloat16)
    inp = dataclasses.replace(inp, k=k)
    q, kk, v = to_dev(inp)
    eo, _ = orc.attn_ex(inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v))
    og = sage.sageattn(q, kk, v).float().cpu().numpy().reshape(-1, d)
    ob = sage.sageattn(q, kk, v, per_block_mean=True).float().cpu().numpy().reshape(-1, d)
    eg, eb = rel_l1(og, eo), rel_l1(ob, eo)
    say(f"  rel-L1 vs exact: global mean {eg:.3e}, per-block mean {eb:.3e}")
    assert eb < eg and eb < 3e-2


def gqa_inputs(inp, Hkv):
    """The same inputs with K and V cut to Hkv heads (every (H/Hkv)-th head)."""
    g = inp.q.shape[1] // Hkv
    return dataclasses.replace(inp, k=inp.k[:, ::g].contiguous(), v=inp.v[:, ::g].contiguous())


def test_quantize_nhd_layout_and_zero_blocks(orc):
    inp = make_inputs(2, 3, 130, 200, 128, sigma=4.0, seed=4)
    qb = inp.q.clone()
    qb[0, 1, 64:128] = 0  # an all-zero Q block: scale 0, codes 0
    kb = inp.k.clone()
    kb[1, 2] = kb[1, 2, :1]  # constant keys: smoothed K exactly zero
    q = qb.permute(0, 2, 1, 3).contiguous().to(DEV)  # NHD
    k = kb.permute(0, 2, 1, 3).contiguous().to(DEV)
    g = sage.quantize_qk(q, k, tensor_layout="NHD")
    torch.cuda.synchronize()
    c = orc.quant_qk(bits(qb), bits(kb))
    assert np.array_equal(g.q8.cpu().numpy(), c.q8) and np.array_equal(g.k8.cpu().numpy(), c.k8)
    assert np.array_equal(g.q_scale.cpu().numpy(), c.qs) and np.array_equal(g.k_scale.cpu().numpy(), c.ks)
    assert g.q_scale[0, 1, 1].item() == 0.0 and (g.k_scale[1, 2] == 0).all()


@pytest.mark.parametrize("B,H,Nq,Nk,d", SHAPES[:6])
def test_debug_scores_bitexact(orc, B, H, Nq, Nk, d):
    inp = make_inputs(B, H, Nq, Nk, d, sigma=4.0, seed=5)
    q, k, v = to_dev(inp)
    g = sage.quantize_qk(q, k)
    c = orc.quant_qk(inp.bits(inp.q), inp.bits(inp.k))
    nqp, nkp = c.q8.shape[2], c.k8.shape[2]
    for b in range(B):
        for h in range(H):
            say(f"scores b={b} h={h} window full")
            got = sage.debug_qk_int32(g, b, h, 0, nqp, 0, nkp).cpu().numpy()
            want = orc.scores(c.q8, c.k8, b, h, 0, nqp, 0, nkp)
            assert np.array_equal(got, want)
    # an unaligned window
    r0, nr, c0, nc = 5, min(70, nqp - 5), 3, min(100, nkp - 3)
    got = sage.debug_qk_int32(g, B - 1, H - 1, r0, nr, c0, nc).cpu().numpy()
    assert np.array_equal(got, orc.scores(c.q8, c.k8, B - 1, H - 1, r0, nr, c0, nc))


def test_debug_scores_extremes(orc):
    """Codes at +-127 everywhere reach the largest |int32| the path produces (127^2 * d)."""
    d = 128
    Q = torch.full((1, 1, 64, d), 3.0, dtype=torch.bfloat16)
    K = torch.zeros(1, 1, 128, d, dtype=torch.bfloat16)
    K[0, 0, :64] = -2.0
    K[0, 0, 64:] = 2.0  # smoothed: +-2 -> codes -127 / 127
    g = sage.quantize_qk(Q.to(DEV), K.to(DEV))
    got = sage.debug_qk_int32(g, 0, 0, 0, 64, 0, 128).cpu().numpy()
    assert (got[:, :64] == -127 * 127 * d).all() and (got[:, 64:] == 127 * 127 * d).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 256, 64), (2, 1, 65, 128), (1, 3, 300, 128), (1, 1, 1, 64)])
def test_prep_v_smooth_v_bitexact(orc, B, H, N, d, dtype):
    """smooth_v: V's channel means and the fp16 codes of V - mean, bit for bit."""
    say(f"prep_v smooth_v B={B} H={H} N={N} d={d} {dtype}")
    inp = make_inputs(B, H, N, N, d, seed=6, dtype=dtype)
    v = (inp.v.float() + 37.0).to(dtype)
    vm = torch.empty(B, H, d, dtype=torch.float32, device=DEV)
    vt, vs = sage.prepare_v(v.to(DEV), "fp16", v_mean=vm)
    torch.cuda.synchronize()
    vb = bits(v)
    want_m = orc.kmean(vb, inp.dtype)
    want, _ = orc.prep_v(vb, "fp16", dtype=inp.dtype, vmean=want_m)
    assert np.array_equal(vm.cpu().numpy().view(np.uint32), want_m.view(np.uint32))
    nat = unpermute_vt(vt.cpu().numpy().view(np.uint16), "fp16")
    assert np.array_equal(nat[:, :, :N, :], want)
    assert not nat[:, :, N:, :].any()  # pad keys stay zero


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("pv", ["fp16", "fp8"])
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 256, 64), (2, 1, 65, 128), (1, 3, 300, 128), (1, 1, 1, 64)])
def test_prep_v_bitexact(orc, pv, B, H, N, d, dtype):
    say(f"prep_v {pv} B={B} H={H} N={N} d={d} {dtype}")
    inp = make_inputs(B, H, N, N, d, seed=6, dtype=dtype)
    vt, vs = sage.prepare_v(inp.v.to(DEV), pv)
    torch.cuda.synchronize()
    want, want_s = orc.prep_v(inp.bits(inp.v), pv, dtype=inp.dtype)
    got = vt.cpu().numpy()
    got = got.view(np.uint16) if pv == "fp16" else got
    nat = unpermute_vt(got, pv)
    assert np.array_equal(nat[:, :, :N, :], want)
    assert not nat[:, :, N:, :].any()  # pad keys are zero
    if pv == "fp8":
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


def test_prep_v_fp8_extremes(orc):
    """Ties, subnormals, saturation edge and a zero channel through the e4m3 preparation."""
    N, d = 64, 64
    V = torch.randn(1, 1, N, d).to(torch.bfloat16)
    V[0, 0, :, 0] = 0  # all-zero channel: scale 0, codes 0
    V[0, 0, 0, 1] = 448.0
    V[0, 0, 1:, 1] = torch.tensor([2.0 ** -e for e in range(3, 3 + N - 1)], dtype=torch.float32).to(torch.bfloat16)
    vt, vs = sage.prepare_v(V.to(DEV), "fp8")
    want, want_s = orc.prep_v(bits(V), "fp8")
    nat = unpermute_vt(vt.cpu().numpy(), "fp8")
    assert np.array_equal(nat[:, :, :N], want) and np.array_equal(vs.cpu().numpy(), want_s)


def oracle_mask(mask, Nq=None):
    """A bool mask as uint8, a float32 mask as it is; a mask broadcast over the queries ([B,1,1,Nk])
    is written out to Nq rows for the oracle."""
    if mask is None:
        return None
    if Nq is not None and mask.shape[-2] == 1:
        mask = mask.expand(*mask.shape[:-2], Nq, mask.shape[-1]).contiguous()
    return mask.numpy() if mask.dtype == torch.float32 else mask.numpy().astype(np.uint8)


def run_both(orc, inp, *, pv="fp16", causal=False, mask=None, sm_scale=None, layout="HND", rows=None, smooth_v=False,
             per_block_mean=False):
    q, k, v = to_dev(inp)
    if layout == "NHD":
        q, k, v = (t.permute(0, 2, 1, 3).contiguous() for t in (q, k, v))
    mask_dev = None if mask is None else mask.to(DEV)
    out, lse = sage.sageattn(q, k, v, tensor_layout=layout, is_causal=causal, attn_mask=mask_dev, sm_scale=sm_scale,
                             return_lse=True, pv_dtype=pv, smooth_v=smooth_v, per_block_mean=per_block_mean)
    torch.cuda.synchronize()
    assert out.dtype == inp.q.dtype  # the output takes the input dtype
    B, H, Nq, d = inp.q.shape
    if rows is None:
        rows = np.arange(B * H * Nq, dtype=np.int64)
    m = oracle_mask(mask, inp.q.shape[2])
    r = orc.run_qe(inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v), pv=pv, causal=causal, mask=m,
                   sm_scale=sm_scale, rows=rows, dtype=inp.dtype, smooth_v=smooth_v, per_block_mean=per_block_mean,
                   **qe_schedule(pv))
    # the plain reading (exact running maximum); for e4m3 P that is the kernels' schedule itself
    r.plain = r if TAU[pv] == 0 else orc.run_qe(
        inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v), pv=pv, causal=causal, mask=m, sm_scale=sm_scale,
        rows=rows, dtype=inp.dtype, smooth_v=smooth_v, per_block_mean=per_block_mean, tau=0.0)
    ex_o, ex_l = orc.attn_ex(inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v), causal=causal, mask=m,
                             sm_scale=sm_scale, rows=rows, dtype=inp.dtype)
    got_o = rows_of(out, rows, layout)
    got_l = lse_rows(lse, rows)
    return got_o, got_l, r, ex_o, ex_l


def check(got_o, got_l, r, ex_o, ex_l, *, pv="fp16", out_dtype="bf16", ex_cos=EX_COS, tag=""):
    dec = f32_of_bf16_bits if out_dtype == "bf16" else (lambda b: b.view(np.float16).astype(np.float32))
    e1 = check_o(got_o, dec(r.o16), pv, tag, plain=dec(r.plain.o16))
    assert_lse_close(got_l, r.lse, QE_LSE)
    assert_lse_close(got_l, r.plain.lse, QE_LSE)
    live = np.abs(ex_o).sum(axis=1) > 0
    if live.any():
        cos = cosine(got_o[live], ex_o[live])
        ex1 = rel_l1(got_o[live], ex_o[live])
        assert cos >= ex_cos, f"cosine vs exact {cos}"
        assert ex1 <= (EX_REL_L1 if pv == "fp16" else 5e-2), f"rel-L1 vs exact {ex1}"
    return e1


CASES = [
    dict(name="tiny", B=1, H=2, Nq=256, Nk=256, d=64),
    dict(name="d128", B=1, H=2, Nq=512, Nk=512, d=128),
    dict(name="ragged", B=2, H=1, Nq=300, Nk=417, d=128),
    dict(name="one_key", B=1, H=2, Nq=77, Nk=1, d=64),
    dict(name="one_query", B=1, H=2, Nq=1, Nk=333, d=128),
    dict(name="causal", B=1, H=2, Nq=600, Nk=600, d=128, causal=True),
    dict(name="causal_rect", B=1, H=1, Nq=300, Nk=520, d=64, causal=True),
    dict(name="mask_half", B=2, H=2, Nq=320, Nk=640, d=128, mask="half"),
    dict(name="mask_rand_per_head", B=1, H=3, Nq=257, Nk=200, d=64, mask="rand_h"),
    dict(name="mask_rand_bcast_causal", B=2, H=2, Nq=200, Nk=200, d=128, mask="rand_1", causal=True),
    dict(name="fp8", B=1, H=2, Nq=400, Nk=777, d=128, pv="fp8", sigma=8.0),
    dict(name="fp8_d64_causal", B=1, H=2, Nq=300, Nk=300, d=64, pv="fp8", causal=True),
    dict(name="fp8_mask", B=1, H=2, Nq=256, Nk=320, d=128, pv="fp8", mask="half"),
    # key-padding masks [B, 1, 1, Nk], broadcast over the queries (mask_stride_q = 0)
    dict(name="mask_keypad", B=2, H=2, Nq=300, Nk=417, d=128, mask="keypad"),
    dict(name="fmask_keypad_fp8_causal", B=2, H=2, Nq=260, Nk=260, d=64, pv="fp8", causal=True, mask="f_keypad"),
    dict(name="sm_scale", B=1, H=2, Nq=256, Nk=256, d=128, sm_scale=0.05),
    # short key ranges at d = 128 (the phase-split step, whose second wave group takes the softmax
    # of the tile after the current one: here past the last tile from the first step on)
    dict(name="one_tile", B=1, H=2, Nq=300, Nk=40, d=128),
    dict(name="one_key_d128_fp8", B=1, H=2, Nq=200, Nk=1, d=128, pv="fp8", sigma=8.0),
    dict(name="two_tiles_ragged", B=1, H=2, Nq=257, Nk=65, d=128),
    dict(name="causal_short", B=1, H=2, Nq=70, Nk=70, d=128, causal=True),
    dict(name="fp8_causal_one_block", B=1, H=2, Nq=256, Nk=256, d=128, pv="fp8", causal=True),
    # peaked rows: most of a row's weight sits on a few keys, where e4m3 P = 448 * p reaches 448 and
    # FP16 P (under its lazy maximum) reaches 2^8 (e4m3 P and V on rows this peaked are at cosine
    # 0.9989 from exact attention in the emulation itself)
    dict(name="fp8_peaked", B=1, H=2, Nq=300, Nk=900, d=128, pv="fp8", sm_scale=0.6, ex_cos=0.998),
    dict(name="fp16_peaked_causal", B=1, H=2, Nq=400, Nk=400, d=128, sm_scale=0.6, causal=True),
    dict(name="nhd", B=2, H=3, Nq=200, Nk=260, d=64, layout="NHD"),
    dict(name="gqa", B=1, H=4, Hkv=2, Nq=300, Nk=417, d=128),
    dict(name="gqa_fp8_causal", B=2, H=6, Hkv=2, Nq=257, Nk=257, d=64, pv="fp8", causal=True),
    dict(name="mqa_nhd_mask_per_head", B=1, H=4, Hkv=1, Nq=200, Nk=333, d=128, layout="NHD", mask="rand_h"),
    # fp16 inputs (and outputs)
    dict(name="fp16_in", B=1, H=2, Nq=300, Nk=417, d=128, dtype="fp16"),
    dict(name="fp16_in_d64_causal", B=2, H=2, Nq=257, Nk=257, d=64, dtype="fp16", causal=True),
    dict(name="fp16_in_fp8_pv", B=1, H=2, Nq=400, Nk=333, d=128, dtype="fp16", pv="fp8", sigma=8.0),
    dict(name="fp16_in_gqa_nhd_mask", B=1, H=4, Hkv=2, Nq=200, Nk=260, d=128, dtype="fp16", layout="NHD",
         mask="rand_h"),
    # float32 additive masks
    dict(name="fmask_bcast", B=2, H=2, Nq=300, Nk=417, d=128, mask="f_rand_1"),
    dict(name="fmask_per_head_d64", B=1, H=3, Nq=257, Nk=200, d=64, mask="f_rand_h"),
    dict(name="fmask_causal", B=1, H=2, Nq=600, Nk=600, d=128, mask="f_rand_1", causal=True),
    dict(name="fmask_fp8", B=1, H=2, Nq=300, Nk=450, d=128, pv="fp8", sigma=8.0, mask="f_rand_h"),
    dict(name="fmask_fp8_d64_causal", B=1, H=2, Nq=200, Nk=333, d=64, pv="fp8", causal=True, mask="f_rand_1"),
    dict(name="fmask_zero_inf_tiles", B=1, H=2, Nq=520, Nk=700, d=128, mask="f_tiles"),
    # the skipped-tile walk: leading, alternating and trailing dropped key tiles per 256-row block
    dict(name="mask_tile_walk", B=1, H=2, Nq=520, Nk=1000, d=128, mask="walk"),
    dict(name="mask_tile_walk_fp8_d64", B=1, H=2, Nq=520, Nk=1000, d=64, pv="fp8", mask="walk"),
    dict(name="mask_tile_walk_causal", B=1, H=2, Nq=1000, Nk=1000, d=128, causal=True, mask="walk"),
    dict(name="fmask_tile_walk", B=1, H=2, Nq=520, Nk=1000, d=128, mask="f_walk"),
    dict(name="fmask_tile_walk_fp8", B=1, H=2, Nq=520, Nk=1000, d=128, pv="fp8", mask="f_walk"),
    dict(name="fmask_gqa_fp16_in_nhd", B=1, H=4, Hkv=1, Nq=130, Nk=260, d=128, dtype="fp16", layout="NHD",
         mask="f_rand_h"),
    # smooth_v on values with a large channel bias
    dict(name="smooth_v", B=1, H=2, Nq=300, Nk=417, d=128, smooth_v=True, v_bias=60.0),
    dict(name="smooth_v_causal_gqa_mask_d64", B=2, H=4, Hkv=2, Nq=257, Nk=257, d=64, smooth_v=True, v_bias=20.0,
         causal=True, mask="rand_1"),
    dict(name="smooth_v_fp16_in_nhd", B=1, H=3, Nq=200, Nk=129, d=128, dtype="fp16", layout="NHD", smooth_v=True,
         v_bias=100.0),
    # per_block_mean: K smoothed by each 64-token block's own mean, block score terms added back
    dict(name="pbm", B=1, H=2, Nq=300, Nk=417, d=128, per_block_mean=True),
    dict(name="pbm_causal_mask_gqa_d64", B=2, H=4, Hkv=2, Nq=257, Nk=257, d=64, per_block_mean=True, causal=True,
         mask="rand_1"),
    dict(name="pbm_fp8_fp16_in", B=1, H=2, Nq=333, Nk=700, d=128, pv="fp8", sigma=8.0, dtype="fp16",
         per_block_mean=True),
    dict(name="pbm_smooth_v_nhd", B=1, H=3, Nq=200, Nk=129, d=128, layout="NHD", per_block_mean=True, smooth_v=True,
         v_bias=30.0),
]


def case_mask(c, B, H, Nq, Nk):
    kind = c.get("mask")
    if kind == "half":
        mask = torch.ones(B, 1, Nq, Nk, dtype=torch.bool)
        mask[..., Nk // 2:] = False
        return mask
    if kind == "rand_h":
        return random_mask(B, H, Nq, Nk, 0.6, seed=3)
    if kind == "rand_1":
        return random_mask(B, 1, Nq, Nk, 0.5, seed=4)
    if kind == "f_rand_1":
        return random_additive_mask(B, 1, Nq, Nk, p_drop=0.25, scale=2.0, seed=5)
    if kind == "f_rand_h":
        return random_additive_mask(B, H, Nq, Nk, p_drop=0.3, scale=3.0, seed=6)
    if kind == "keypad":  # a key-padding mask [B, 1, 1, Nk]: each batch entry drops its own keys
        m = torch.ones(B, 1, 1, Nk, dtype=torch.bool)
        for b in range(B):
            m[b, 0, 0, Nk - 37 * (b + 1):] = False
        m[0, 0, 0, 5:70] = False  # and a run crossing a key tile
        return m
    if kind == "f_keypad":  # the same as an fp32 additive mask [B, 1, 1, Nk], broadcast over the queries
        m = torch.zeros(B, 1, 1, Nk, dtype=torch.float32)
        m[..., Nk // 3:] = float("-inf")
        m[..., :40] = 0.7
        return m
    if kind in ("walk", "f_walk"):
        # Per 256-row block, which 64-key tiles any of its rows sees: rows 0-255 every third tile
        # from tile 2 (tiles 0-1 dropped, one of them partly masked), rows 256-511 tile 7 (partly)
        # and the ragged last tile only, rows 512+ the first four tiles only.
        vis = torch.zeros(Nq, Nk, dtype=torch.bool)
        for t in range(2, (Nk + 63) // 64, 3):
            vis[:256, 64 * t:64 * t + 64] = True
        vis[:256, 64 * 8 + 10:64 * 8 + 30] = False
        vis[256:512, 64 * 7:64 * 7 + 33] = True
        vis[256:512, 64 * ((Nk - 1) // 64):] = True
        vis[512:, :256] = True
        vis[600:, 900:] = True  # later blocks (causal case): a visible run across the ragged tail
        vis = vis[:Nq, :Nk].expand(B, 1, Nq, Nk)
        if kind == "walk":
            return vis.clone()
        m = torch.where(vis, 0.0, float("-inf")).to(torch.float32)
        m[..., :256, 64 * 5:64 * 6] += 0.5 * torch.randn(B, 1, min(Nq, 256), 64,
                                                        generator=torch.Generator().manual_seed(8))
        return m
    if kind == "f_tiles":
        # whole 256 x 64 tiles that are all 0 (read no mask), all -inf (skipped) or mixed
        m = torch.zeros(B, 1, Nq, Nk, dtype=torch.float32)
        m[..., 64:128] = float("-inf")  # a dropped key tile
        m[..., 256:512, 192:256] = float("-inf")
        m[..., 300:, 320:384] = 0.5 * torch.randn(B, 1, Nq - 300, 64, generator=torch.Generator().manual_seed(7))
        m[..., 9, :] = float("-inf")  # a row that sees nothing
        return m
    assert kind is None, kind
    return None


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_attention_parity(orc, case):
    c = dict(case)
    say(f"attention case {c}")
    B, H, Nq, Nk, d = c["B"], c["H"], c["Nq"], c["Nk"], c["d"]
    dtype = torch.float16 if c.get("dtype") == "fp16" else torch.bfloat16
    inp = make_inputs(B, H, Nq, Nk, d, sigma=c.get("sigma", 4.0), seed=11, dtype=dtype)
    if "Hkv" in c:
        inp = gqa_inputs(inp, c["Hkv"])
    if "v_bias" in c:  # a per-channel offset of +-v_bias on V (what smooth_v is for)
        sign = torch.where(torch.arange(d) % 3 == 0, -1.0, 1.0)
        inp = dataclasses.replace(inp, v=(inp.v.float() + c["v_bias"] * sign).to(dtype))
    mask = case_mask(c, B, H, Nq, Nk)
    got_o, got_l, r, ex_o, ex_l = run_both(orc, inp, pv=c.get("pv", "fp16"), causal=c.get("causal", False), mask=mask,
                                           sm_scale=c.get("sm_scale"), layout=c.get("layout", "HND"),
                                           smooth_v=c.get("smooth_v", False),
                                           per_block_mean=c.get("per_block_mean", False))
    check(got_o, got_l, r, ex_o, ex_l, pv=c.get("pv", "fp16"), out_dtype=inp.dtype, ex_cos=c.get("ex_cos", EX_COS),
          tag=c["name"])


def test_fully_masked_rows_and_tiles(orc):
    B, H, Nq, Nk, d = 1, 2, 300, 300, 64
    inp = make_inputs(B, H, Nq, Nk, d, seed=12)
    mask = torch.ones(B, 1, Nq, Nk, dtype=torch.bool)
    mask[0, 0, 7, :] = False  # one row sees nothing
    mask[0, 0, 256:, :] = False  # a whole 256-row tile sees nothing
    mask[0, 0, :, 64:128] = False  # a whole key tile is dropped
    got_o, got_l, r, ex_o, ex_l = run_both(orc, inp, mask=mask)
    check(got_o, got_l, r, ex_o, ex_l)
    dead = np.array([h * Nq + i for h in range(H) for i in [7] + list(range(256, 300))])
    assert (got_o[dead] == 0).all() and np.isneginf(got_l[dead]).all()


def test_zero_query_closed_form(orc):
    """Q = 0: every score is 0, so O is the mean of the prepared values and LSE = ln(Nk)."""
    B, H, N, d = 1, 2, 200, 128
    inp = make_inputs(B, H, N, N, d, seed=13)
    inp.q.zero_()
    out, lse = sage.sageattn(*to_dev(inp), return_lse=True)
    vhat = torch.from_numpy(inp.v.float().numpy()).to(torch.float16).double()
    want = vhat.mean(dim=2, keepdim=True).expand(B, H, N, d)
    np.testing.assert_allclose(out.float().cpu().numpy(), want.numpy(), rtol=1e-2, atol=1e-3)
    np.testing.assert_allclose(lse.cpu().numpy(), np.log(N), atol=1e-5)


def test_outputs_leave_neighbours_untouched():
    """Canary: the output and LSE buffers live inside larger buffers; nothing outside changes."""
    B, H, Nq, Nk, d = 1, 2, 131, 131, 128
    inp = make_inputs(B, H, Nq, Nk, d, seed=14)
    q, k, v = to_dev(inp)
    qk = sage.quantize_qk(q, k)
    big = torch.full((B * H * Nq * d + 4096,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = big[2048:2048 + B * H * Nq * d].view(B, H, Nq, d)
    lbig = torch.full((B * H * Nq + 128,), 3.25, dtype=torch.float32, device=DEV)
    lse = lbig[64:64 + B * H * Nq].view(B, H, Nq)
    sage.attn_fwd(qk, v, out=out, lse=lse, return_lse=True)
    torch.cuda.synchronize()
    assert (big[:2048] == -7.0).all() and (big[2048 + B * H * Nq * d:] == -7.0).all()
    assert (lbig[:64] == 3.25).all() and (lbig[64 + B * H * Nq:] == 3.25).all()
    assert torch.isfinite(out.float()).all()


def test_repeatable_bitwise():
    inp = make_inputs(1, 2, 700, 700, 128, seed=15)
    q, k, v = to_dev(inp)
    ref = sage.sageattn(q, k, v, return_lse=True)
    for _ in range(5):
        o, l = sage.sageattn(q, k, v, return_lse=True)
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])


def test_errors_raise():
    inp = make_inputs(1, 1, 64, 64, 64, seed=16)
    q, k, v = to_dev(inp)
    with pytest.raises(ValueError):
        sage.sageattn(q[..., :32].contiguous(), k[..., :32].contiguous(), v[..., :32].contiguous())
    with pytest.raises(ValueError):  # mixed input dtypes
        sage.sageattn(q.half(), k, v)
    with pytest.raises(ValueError):  # a float mask must be float32
        sage.sageattn(q, k, v, attn_mask=torch.zeros(1, 1, 64, 64, dtype=torch.float16, device=DEV))
    with pytest.raises(api.SageError) as ei:  # fp16 Q with bf16 K, past the Python checks
        sage.quantize_qk(q.half(), k)
    assert ei.value.status == 1
    with pytest.raises(api.SageError) as ei:  # smooth_v belongs to the FP16 PV path
        sage.sageattn(q, k, v, pv_dtype="fp8", smooth_v=True)
    assert ei.value.status == 2
    with pytest.raises(api.SageError) as ei:  # per_block_mean is not combined with a float mask
        sage.sageattn(q, k, v, per_block_mean=True, attn_mask=torch.zeros(1, 1, 64, 64, device=DEV))
    assert ei.value.status == 2


@pytest.mark.parametrize("pv", ["fp16", "fp8"])
def test_zero_inf_float_mask_equals_boolean_mask(pv):
    """A float32 mask of 0 / -inf gives what the boolean mask gives, up to the float path's
    rounding (the float-mask kernel converts every score to fp32 before its maximum)."""
    B, H, Nq, Nk, d = 1, 2, 300, 400, 128
    inp = make_inputs(B, H, Nq, Nk, d, seed=17, sigma=4.0 if pv == "fp16" else 8.0)
    q, k, v = to_dev(inp)
    bm = random_mask(B, 1, Nq, Nk, 0.5, seed=8)
    ob, lb = sage.sageattn(q, k, v, attn_mask=bm.to(DEV), return_lse=True, pv_dtype=pv)
    of, lf = sage.sageattn(q, k, v, attn_mask=additive_mask(bm).to(DEV), return_lse=True, pv_dtype=pv)
    torch.cuda.synchronize()
    assert rel_l1(of.float().cpu().numpy(), ob.float().cpu().numpy()) < 2e-3
    assert_lse_close(lf.cpu().numpy(), lb.cpu().numpy(), 1e-4)


def test_output_dtype_is_a_choice(orc):
    """bf16 inputs with an fp16 output buffer (and the reverse) through the C ABI."""
    B, H, N, d = 1, 2, 200, 128
    for dt_in, dt_out in ((torch.bfloat16, torch.float16), (torch.float16, torch.bfloat16)):
        say(f"output dtype {dt_in} -> {dt_out}")
        inp = make_inputs(B, H, N, N, d, seed=18, dtype=dt_in)
        q, k, v = to_dev(inp)
        qk = sage.quantize_qk(q, k)
        out = torch.empty(B, H, N, d, dtype=dt_out, device=DEV)
        sage.attn_fwd(qk, v, out=out)
        torch.cuda.synchronize()
        name = "fp16" if dt_out == torch.float16 else "bf16"
        r = orc.run_qe(inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v), dtype=inp.dtype, out_dtype=name,
                       **qe_schedule("fp16"))
        want = f32_of_bf16_bits(r.o16) if name == "bf16" else r.o16.view(np.float16).astype(np.float32)
        assert rel_l1(out.float().cpu().numpy().reshape(-1, d), want) <= QE_REL_L1
