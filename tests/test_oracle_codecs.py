"""Pins for the oracle's number-format codecs against independent library routines.

fp16: numpy's float16 cast (IEEE binary16, round to nearest even).
bf16: torch's bfloat16 cast (round to nearest even).
e4m3: torch's float8_e4m3fn cast (OCP E4M3, round to nearest even) and a brute-force
nearest-code search over the 254 finite codes, plus the saturation rule as a closed form.
"""

import numpy as np
import pytest
import torch


def _nan_eq(a_bits, b_bits, to_float):
    a = to_float(a_bits)
    b = to_float(b_bits)
    both_nan = np.isnan(a) & np.isnan(b)
    return (a_bits == b_bits) | both_nan


def test_f16_exhaustive_over_bf16_inputs(orc):
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    got = orc.f32_to_f16(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    ok = _nan_eq(got, want, lambda b: b.view(np.float16).astype(np.float32))
    assert ok.all(), np.nonzero(~ok)[0][:10]


def test_f16_random_and_edge_fp32(orc):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    # ties and boundaries around the fp16 grid
    edges = np.array([65504.0, 65519.99, 65520.0, 65535.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
                      2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -0.0, 0.0, np.inf, -np.inf],
                     np.float32)
    # every fp16 value +- half an ulp (exact ties) via fp64 midpoints
    h = np.arange(0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[1:] + h[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, edges, mids, -mids])
    got = orc.f32_to_f16(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    ok = _nan_eq(got, want, lambda b: b.view(np.float16).astype(np.float32))
    assert ok.all(), x[~ok][:10]


def test_f16_decode_all_codes(orc):
    codes = np.arange(1 << 16, dtype=np.uint16)
    got = orc.f16_to_f32(codes)
    want = codes.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_bf16_random_vs_torch(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    # exact ties: bf16 values +- half a bf16 ulp
    b = (np.arange(0x7f80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    mids = ((b[1:] + b[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.array([3.4e38, 3.39e38, -0.0, np.inf], np.float32)])
    got = orc.f32_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    to_f = lambda v: (v.astype(np.uint32) << 16).view(np.float32)
    ok = _nan_eq(got, want, to_f)
    assert ok.all(), x[~ok][:10]


def test_e4m3_decode_all_codes_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_to_f32(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    # the format's landmarks
    assert got[0x7E] == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def _e4m3_structured_inputs():
    """Every exponent in and around the e4m3 range x every 12-bit leading-fraction pattern, with the
    trailing fraction bits all-zero, lowest-bit-only and all-ones (so ties and sticky bits occur)."""
    out = []
    for e in range(-13, 10):
        lead = np.arange(1 << 12, dtype=np.uint32) << 11
        for tail in (0, 1, (1 << 11) - 1):
            frac = lead | tail
            bits = (np.uint32(e + 127) << 23) | frac
            out.append(bits.view(np.float32))
    x = np.concatenate(out)
    return np.concatenate([x, -x])


def test_e4m3_encode_vs_torch(orc):
    rng = np.random.default_rng(2)
    rnd = (rng.standard_normal(3_000_000) * np.exp2(rng.integers(-12, 9, 3_000_000))).astype(np.float32)
    x = np.concatenate([_e4m3_structured_inputs(), rnd, np.array([0.0, -0.0], np.float32)])
    x = x[np.abs(x) < 464.0]  # beyond the midpoint to 480 torch returns NaN; saturation is tested below
    got = orc.f32_to_e4m3(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = got != want
    assert not bad.any(), (x[bad][:8], got[bad][:8], want[bad][:8])


def test_e4m3_encode_vs_nearest_code_search(orc):
    """Brute force: the nearest finite code, ties to the code with an even last bit."""
    finite = np.array([c for c in range(0x7F)], np.uint8)
    vals = orc.e4m3_to_f32(finite).astype(np.float64)  # 0 .. 448, increasing
    rng = np.random.default_rng(3)
    x = np.concatenate([
        (rng.random(200_000) * 470).astype(np.float32),
        (rng.random(100_000) * 0.02).astype(np.float32),
        ((vals[1:] + vals[:-1]) / 2).astype(np.float32),  # exact ties
    ])
    got = orc.f32_to_e4m3(x)
    dist = np.abs(x.astype(np.float64)[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among equally near codes take the even one
    even = cand & ((finite[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)
    assert (got == pick).all(), x[got != pick][:8]


def test_e4m3_saturation_and_specials(orc):
    x = np.array([464.0, 465.0, 480.0, 1e4, 3e38, np.inf, -464.0, -1e30, -np.inf, np.nan], np.float32)
    got = orc.f32_to_e4m3(x)
    assert list(got[:6]) == [0x7E] * 6
    assert list(got[6:9]) == [0xFE] * 3
    assert got[9] & 0x7F == 0x7F
    # 448 itself and values just above it round to 448
    assert list(orc.f32_to_e4m3(np.array([448.0, 448.04, 463.99], np.float32))) == [0x7E] * 3
