"""GPU parity of the FP4 microscaling method (sage_fp4_quantize_qkv / sage_fp4_attn_fwd, through
the C ABI) against the oracle (sage_fp4_oracle.c).

Bit-exact: K mean and Q means, the e2m1 codes and E8M0 scales of Q, K and V (after undoing the
documented packing and lane order).  Tolerance: lse_corr and the correction rows within fp32
accumulation error; raw scores of a window (debug entry) within fp32 accumulation error of the
oracle's exact sums; O within rel-L1 1e-3 of the oracle's emulation (both rounded to the output
dtype), LSE within 1e-3; against exact attention the measured MX-FP4 budget (cosine >= 0.97,
rel-L1 <= 0.25).  Cases: ragged tails (Nq, Nk not multiples of 128 or 64), causal with Nq != Nk,
GQA, per-block and global Q means, fp16 inputs, fp32 output, one key, one query, Q = 0, a K whose
channel means are large against its spread.
"""

import numpy as np
import pytest
import torch

import quantized_attention_quantize_amd as sage
from quantized_attention_quantize_amd.synthetic import make_inputs

from gpu_helpers import (DEV, TAU_FP4, check_o, assert_lse_close, cosine, f32_of_bf16_bits, fp4_check_quant, rel_l1, say,
                         to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sage.load_library()


def _dec(bits, dtype):
    return f32_of_bf16_bits(bits) if dtype == "bf16" else bits.view(np.float16).astype(np.float32)


def _out_f32(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy()


CASES = [
    dict(name="tiny", B=1, H=2, Nq=256, Nk=256),
    dict(name="ragged", B=2, H=2, Nq=300, Nk=200),
    dict(name="causal_rect", B=1, H=2, Nq=333, Nk=520, causal=True),
    dict(name="causal_square", B=1, H=3, Nq=700, Nk=700, causal=True),
    dict(name="gqa_global_mean", B=1, H=4, Hkv=2, Nq=250, Nk=390, pbm=False),
    dict(name="gqa_causal", B=2, H=4, Hkv=1, Nq=260, Nk=260, causal=True),
    dict(name="fp16", B=1, H=2, Nq=321, Nk=333, dtype=torch.float16),
    dict(name="fp32_out_global", B=1, H=2, Nq=128, Nk=700, pbm=False, out=torch.float32),
    dict(name="one_key", B=1, H=2, Nq=70, Nk=1),
    dict(name="one_query", B=1, H=2, Nq=1, Nk=300, causal=True),
    dict(name="large_k_mean", B=1, H=2, Nq=400, Nk=450, sigma=96.0),
    dict(name="large_k_mean_fp16", B=1, H=2, Nq=200, Nk=333, sigma=96.0, dtype=torch.float16),
    # peaked rows: p reaches 2^tau under the lazy maximum (P = 448 * 2^-tau * p nears 448); FP4's
    # distance to exact attention grows with the peak, so only parity with the emulation is checked
    dict(name="peaked_causal", B=1, H=2, Nq=300, Nk=500, causal=True, sm_scale=0.3, budget=False),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_fp4_parity(orc, case):
    c = dict(case)
    say(f"fp4 case {c}")
    B, H, Hkv, Nq, Nk, d = c["B"], c["H"], c.get("Hkv", c["H"]), c["Nq"], c["Nk"], 128
    causal, pbm = c.get("causal", False), c.get("pbm", True)
    tdt = c.get("dtype", torch.bfloat16)
    dts = "fp16" if tdt == torch.float16 else "bf16"
    inp = make_inputs(B, H, Nq, Nk, d, sigma=c.get("sigma", 4.0), seed=90, Hkv=Hkv, dtype=tdt)
    q, k, v = to_dev(inp)
    g = sage.quantize_qkv_fp4(q, k, v, per_block_mean=pbm)
    sm = c.get("sm_scale")
    out, lse = sage.attn_fwd_fp4(g, is_causal=causal, sm_scale=sm, return_lse=True, out_dtype=c.get("out"))
    torch.cuda.synchronize()
    Q, K, V = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    r = orc.fp4_quant_qk(Q, K, dtype=dts, per_block_mean=pbm)
    v4, ve = orc.fp4_prep_v(V, dts)
    Kf = _dec(K, dts)
    k_max = max(float(np.abs(Kf).max()), float(np.abs(Kf - r.kmean[:, :, None, :]).max()))
    fp4_check_quant(g, r, Nq, Nk, (v4, ve), k_max)
    say("  quantization bit-exact")
    out_dt = c.get("out") or tdt
    ods = {torch.float32: "bf16", torch.bfloat16: "bf16", torch.float16: "fp16"}[out_dt]
    o32, o16, qlse = orc.fp4_attn_qe(r, v4, ve, causal=causal, sm_scale=sm, tau=TAU_FP4, out_dtype=ods)
    got = _out_f32(out).reshape(-1, d)
    want = o32 if out_dt == torch.float32 else _dec(o16, ods)
    check_o(got, want, "fp8", c["name"])  # e4m3 P under the exact running maximum: the plain reading
    assert_lse_close(lse.cpu().numpy().reshape(-1), qlse, 1e-3)
    eo, el = orc.attn_ex(Q, K, V, causal=causal, sm_scale=sm, dtype=dts)
    cs, rl = cosine(got, eo), rel_l1(got, eo)
    say(f"  vs exact: cosine {cs:.5f} rel-L1 {rl:.3e}")
    if Nk > 1 and Nq > 1 and c.get("budget", True):
        assert cs >= 0.97 and rl <= 0.25


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,pbm", [(1, 2, 2, 4500, 1100, True), (1, 8, 4, 4500, 4000, True),
                                              (2, 4, 4, 3000, 2600, False)])
def test_fp4_quantize_groups_of_q_blocks(orc, B, H, Hkv, Nq, Nk, pbm):
    """Quantization bit-exact and correction rows within fp32 accumulation error where the
    correction kernel takes more than one group of 32 Q blocks (36 blocks: a partial second group)
    and, for 8 heads x 4000 keys, two key blocks per wave; and with the global Q mean."""
    say(f"fp4 quantize B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} per_block_mean={pbm}")
    inp = make_inputs(B, H, Nq, Nk, 128, sigma=4.0, seed=95, Hkv=Hkv)
    q, k, v = to_dev(inp)
    g = sage.quantize_qkv_fp4(q, k, v, per_block_mean=pbm)
    torch.cuda.synchronize()
    Q, K, V = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    r = orc.fp4_quant_qk(Q, K, per_block_mean=pbm)
    v4, ve = orc.fp4_prep_v(V)
    Kf = f32_of_bf16_bits(K)
    k_max = max(float(np.abs(Kf).max()), float(np.abs(Kf - r.kmean[:, :, None, :]).max()))
    fp4_check_quant(g, r, Nq, Nk, (v4, ve), k_max)


def test_fp4_debug_scores_window(orc):
    B, H, Nq, Nk, d = 1, 2, 300, 200, 128
    inp = make_inputs(B, H, Nq, Nk, d, seed=91)
    q, k, v = to_dev(inp)
    g = sage.quantize_qkv_fp4(q, k, v)
    r = orc.fp4_quant_qk(inp.bits(inp.q), inp.bits(inp.k))
    for (b, h, r0, nr, c0, nc) in [(0, 1, 0, 300, 0, 200), (0, 0, 96, 64, 64, 130)]:
        got = sage.debug_scores_fp4(g, b, h, r0, nr, c0, nc).cpu().numpy()
        want = orc.fp4_scores(r, b, h, r0, nr, c0, nc)
        tol = 1e-6 * np.abs(want).max() + 1e-6
        assert np.abs(got - want).max() <= 64 * tol, np.abs(got - want).max()


def test_fp4_zero_q_closed_form(orc):
    """Q = 0: every score is the correction term of a zero mean, i.e. 0; O = mean of the dequantized V."""
    B, H, N, d = 1, 2, 200, 128
    inp = make_inputs(B, H, N, N, d, seed=92)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    _, k, v = to_dev(inp)
    out, lse = sage.sageattn_fp4(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    v4, ve = orc.fp4_prep_v(inp.bits(inp.v))
    vmean = orc.mx_dequant(v4, ve, 2).mean(2)  # [B, H, d]
    np.testing.assert_allclose(_out_f32(out), np.broadcast_to(vmean[:, :, None, :], (B, H, N, d)), rtol=8e-3, atol=2e-3)
    np.testing.assert_allclose(lse.cpu().numpy(), np.log(N), rtol=0, atol=1e-5)


def test_fp4_repeatable_and_errors():
    inp = make_inputs(1, 2, 200, 200, 128, seed=93)
    q, k, v = to_dev(inp)
    a = sage.sageattn_fp4(q, k, v, is_causal=True)
    b = sage.sageattn_fp4(q, k, v, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(ValueError):
        sage.sageattn_fp4(q[..., :64].contiguous(), k[..., :64].contiguous(), v[..., :64].contiguous())
    g = sage.quantize_qkv_fp4(q, k, v)
    bad = torch.empty(1, 2, 200, 128, dtype=torch.bfloat16, device=DEV)[..., 1:]
    with pytest.raises(Exception):
        sage.attn_fwd_fp4(g, out=bad)
