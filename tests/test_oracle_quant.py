"""Pins for the oracle's K mean, smoothing, per-block INT8 quantization and int32 scores.

Each check comes from mathematics rather than from the oracle itself: exact means of dyadic data,
shift invariance of the smoothed quantization, the round-trip error bound of a symmetric
quantizer, hand-built blocks with known codes (including exact .5 ties), and brute-force integer
dot products.
"""

import numpy as np
import pytest
import torch

from quantized_attention_quantize_amd.synthetic import make_inputs


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _dyadic(rng, shape, denom=4, lim=16):
    """Values k/denom with |k| < lim: exactly representable in bf16 and in every sum below."""
    return rng.integers(-lim, lim, size=shape).astype(np.float32) / denom


def test_kmean_exact_on_dyadic_data(orc):
    rng = np.random.default_rng(0)
    K = _dyadic(rng, (2, 3, 128, 64))
    km = orc.kmean(_bf16_bits(K))
    want = K.astype(np.float64).mean(axis=2)  # exact: sums of quarters over a power-of-two count
    assert np.array_equal(km.astype(np.float64), want)


def test_kmean_fp64_accumulation_matches_fsum(orc):
    import math
    inp = make_inputs(1, 2, 64, 777, 64, sigma=4.0, seed=5)
    kb = inp.bits(inp.k)
    km = orc.kmean(kb)
    kf = _f32(kb).astype(np.float64)
    for h in range(2):
        for c in range(0, 64, 7):
            exact = math.fsum(kf[0, h, :, c].tolist()) / 777.0
            assert km[0, h, c] == np.float32(exact)


def test_shift_invariance_of_smoothed_k(orc):
    """K' = K + 1 c^T (per-channel integer shift): kmean' = kmean + c exactly, so the smoothed K, its
    int8 codes and scales are bitwise identical, and the LSE shift is carried by corr alone."""
    rng = np.random.default_rng(1)
    B, H, N, d = 1, 2, 128, 64
    K = _dyadic(rng, (B, H, N, d))
    c = (rng.integers(-4, 5, size=(B, H, 1, d)) * 4).astype(np.float32)
    Q = _dyadic(rng, (B, H, N, d), denom=8)
    V = _dyadic(rng, (B, H, N, d), denom=8)
    Kb, Ks, Qb, Vb = _bf16_bits(K), _bf16_bits(K + c), _bf16_bits(Q), _bf16_bits(V)
    assert np.array_equal(_f32(Ks), K + c)  # the shifted keys are exact in bf16
    a = orc.quant_qk(Qb, Kb)
    b = orc.quant_qk(Qb, Ks)
    assert np.array_equal(b.kmean, a.kmean + c[:, :, 0, :])
    assert np.array_equal(a.k8, b.k8) and np.array_equal(a.ks, b.ks)
    assert np.array_equal(a.q8, b.q8) and np.array_equal(a.qs, b.qs)
    vh, vs = orc.prep_v(Vb, "fp16")
    oa = orc.attn_qe(a, vh, vs, "fp16", N, N)
    ob = orc.attn_qe(b, vh, vs, "fp16", N, N)
    assert np.array_equal(oa[0], ob[0])
    # LSE moves by sm_scale * (q . c); in EX exactly that, in QE through corr
    sm = orc.default_sm_scale(d)
    shift = sm * np.einsum("bhnd,bhd->bhn", Q.astype(np.float64), c[:, :, 0, :].astype(np.float64)).reshape(-1)
    np.testing.assert_allclose(ob[2] - oa[2], shift, atol=2e-5 * (1 + np.abs(shift)).max())
    ea = orc.attn_ex(Qb, Kb, Vb)
    eb = orc.attn_ex(Qb, Ks, Vb)
    np.testing.assert_allclose(eb[0], ea[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(eb[1] - ea[1], shift, atol=1e-9)


def test_quant_roundtrip_bound_and_code_range(orc):
    inp = make_inputs(1, 3, 200, 200, 64, sigma=4.0, seed=2)
    Qb, Kb = inp.bits(inp.q), inp.bits(inp.k)
    qk = orc.quant_qk(Qb, Kb)
    Q = _f32(Qb)
    Ks = (_f32(Kb) - qk.kmean[:, :, None, :]).astype(np.float32)  # one fp32 rounding per element
    for x, x8, sc in ((Q, qk.q8, qk.qs), (Ks, qk.k8, qk.ks)):
        N = x.shape[2]
        assert x8.shape[2] == 256 and not x8[:, :, N:].any()  # zero pad rows
        assert np.abs(x8.astype(np.int32)).max() <= 127
        for u in range(sc.shape[2]):
            r0, r1 = 64 * u, min(64 * u + 64, N)
            blk = x[:, :, r0:r1].astype(np.float64)
            codes = x8[:, :, r0:r1].astype(np.float64)
            s = sc[:, :, u].astype(np.float64)[:, :, None, None]
            err = np.abs(blk - s * codes)
            # half a code, plus the binary32 error of x * fl(127/amax) against x / fl(amax/127):
            # three roundings of relative size 2^-24 on a value of at most 127 codes
            assert (err <= s * (0.5 + 127 * 3 * 2.0 ** -24) + 1e-30).all()
            # each nonzero block reaches the end of the code range exactly once at its max
            assert (np.abs(codes).max(axis=(2, 3)) == 127).all()
            amax = np.abs(blk).max(axis=(2, 3))
            assert np.array_equal(sc[:, :, u], (amax.astype(np.float32) / np.float32(127)))


def test_hand_built_block_known_codes_and_ties(orc):
    """amax = 127 makes scale = inv = 1, so codes are RNE of the values themselves."""
    d = 64
    Q = np.zeros((1, 1, 64, d), np.float32)
    vals = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -126.5, 0.25, 7.75, -100.0]
    want = [127, 2, 4, -2, -4, 0, 2, 0, 126, -126, 0, 8, -100]
    Q[0, 0, 0, :len(vals)] = vals
    qk = orc.quant_qk(_bf16_bits(Q), _bf16_bits(np.ones_like(Q)))
    assert qk.qs[0, 0, 0] == 1.0
    assert list(qk.q8[0, 0, 0, :len(vals)]) == want
    # a block whose max is 254 has scale 2 and halves every value before rounding
    Q2 = Q * 2
    qk2 = orc.quant_qk(_bf16_bits(Q2), _bf16_bits(np.ones_like(Q)))
    assert qk2.qs[0, 0, 0] == 2.0
    assert list(qk2.q8[0, 0, 0, :len(vals)]) == want


def test_zero_block_and_tail_block(orc):
    d = 64
    Q = np.zeros((1, 1, 65, d), np.float32)
    Q[0, 0, 64, 3] = -0.75  # the tail block holds one row
    K = np.ones((1, 1, 65, d), np.float32)  # constant keys: smoothed K is exactly zero
    qk = orc.quant_qk(_bf16_bits(Q), _bf16_bits(K))
    assert qk.qs.shape == (1, 1, 2) and qk.qs[0, 0, 0] == 0.0 and not qk.q8[0, 0, :64].any()
    assert qk.qs[0, 0, 1] == np.float32(0.75) / np.float32(127) and qk.q8[0, 0, 64, 3] == -127
    assert (qk.ks == 0).all() and not qk.k8.any()
    assert qk.q8.shape[2] == 128 and not qk.q8[0, 0, 65:].any()


def test_corr_is_q_dot_kmean(orc):
    inp = make_inputs(1, 2, 100, 300, 128, sigma=4.0, seed=3)
    Qb, Kb = inp.bits(inp.q), inp.bits(inp.k)
    qk = orc.quant_qk(Qb, Kb)
    want = np.einsum("bhnd,bhd->bhn", _f32(Qb).astype(np.float64), qk.kmean.astype(np.float64))
    np.testing.assert_allclose(qk.corr, want, rtol=1e-6, atol=1e-6)


def test_scores_brute_force(orc):
    rng = np.random.default_rng(4)
    q8 = rng.integers(-127, 128, size=(1, 2, 256, 128)).astype(np.int8)
    k8 = rng.integers(-127, 128, size=(1, 2, 256, 128)).astype(np.int8)
    q8[0, 1, 0, :] = 127
    k8[0, 1, 0, :] = -127  # the extreme product sum -127^2 * 128
    for h in range(2):
        got = orc.scores(q8, k8, 0, h, 0, 200, 10, 190)
        want = q8[0, h, :200].astype(np.int64) @ k8[0, h, 10:200].astype(np.int64).T
        assert np.array_equal(got.astype(np.int64), want)
    assert orc.scores(q8, k8, 0, 1, 0, 1, 0, 1)[0, 0] == -127 * 127 * 128


def test_prep_v_fp8_per_channel(orc):
    inp = make_inputs(1, 2, 64, 300, 64, sigma=4.0, seed=6)
    Vb = inp.bits(inp.v)
    v8, vs = orc.prep_v(Vb, "fp8")
    V = _f32(Vb)
    vmax = np.abs(V).max(axis=2)
    assert np.array_equal(vs, vmax / np.float32(448))
    dec = orc.e4m3_to_f32(v8)
    # the per-channel max maps to +-448 exactly, everything else within half an e4m3 step
    assert (np.abs(dec).max(axis=2) == 448.0).all()
    scaled = V * (np.float32(448) / vmax)[:, :, None, :]
    rel = np.abs(dec - scaled) / np.maximum(np.abs(scaled), 2.0 ** -6)
    assert rel.max() <= 2.0 ** -4 + 1e-7
    v16, none = orc.prep_v(Vb, "fp16")
    assert none is None
    assert np.array_equal(orc.f16_to_f32(v16), V)  # bf16 values in fp16 normal range are exact
