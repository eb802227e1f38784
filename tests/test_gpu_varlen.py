"""GPU parity of packed variable-length batches (sage_quantize_qk_varlen / sage_attn_fwd_varlen)
against the oracle's per-sequence emulation.

Bit-exact: each sequence's K mean, int8 codes and scales equal the dense oracle quantization of that
sequence alone.  Tolerance: O within relative L1 1e-3 of the emulation (both rounded to the
output dtype), LSE within 1e-3; against exact attention, cosine >= 0.999 and relative L1 <= 3e-2
(FP16 PV; 5e-2 for FP8).  Cases: the docs digest's example lengths (512, 1024, 768; 16 heads,
d = 128, fp16), ragged lengths with a one-token sequence, a sequence without queries and one
without keys, Nq != Nk per sequence, causal, GQA, FP8 PV and d = 64.
"""

import numpy as np
import pytest
import torch

import quantized_attention_quantize_amd as sage
from quantized_attention_quantize_amd.synthetic import make_varlen_inputs

from gpu_helpers import DEV, TAU, assert_lse_close, check_o, cosine, f32_of_bf16_bits, qe_schedule, rel_l1, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sage.load_library()


def _dec(bits, dtype):
    return f32_of_bf16_bits(bits) if dtype == "bf16" else bits.view(np.float16).astype(np.float32)


CASES = [
    dict(name="pages_example", sq=[512, 1024, 768], sk=[512, 1024, 768], H=16, d=128, dtype=torch.float16),
    dict(name="pages_example_causal", sq=[512, 1024, 768], sk=[512, 1024, 768], H=16, d=128, dtype=torch.float16,
         causal=True),
    dict(name="ragged", sq=[70, 1, 130, 300], sk=[90, 5, 130, 257], H=2, d=128),
    dict(name="empty_and_keyless", sq=[50, 0, 40, 30], sk=[60, 20, 45, 0], H=2, d=64),
    dict(name="causal_rect", sq=[100, 257, 64], sk=[300, 257, 130], H=3, d=64, causal=True),
    dict(name="gqa_fp8", sq=[333, 129], sk=[333, 500], H=4, Hkv=2, d=128, pv="fp8", sigma=8.0),
    dict(name="gqa_fp8_causal_d64", sq=[200, 65, 256], sk=[200, 65, 256], H=4, Hkv=1, d=64, pv="fp8", sigma=8.0,
         causal=True),
    dict(name="smooth_v_ragged", sq=[70, 1, 130, 300], sk=[90, 5, 130, 0], H=2, d=128, smooth_v=True, v_bias=40.0),
    dict(name="per_block_mean_ragged_causal", sq=[70, 1, 130, 300], sk=[90, 5, 200, 0], H=4, Hkv=2, d=128,
         per_block_mean=True, causal=True),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_varlen_parity(orc, case):
    c = dict(case)
    say(f"varlen case {c}")
    pv, causal = c.get("pv", "fp16"), c.get("causal", False)
    inp = make_varlen_inputs(c["sq"], c["sk"], c["H"], c["d"], sigma=c.get("sigma", 4.0), seed=60,
                             Hkv=c.get("Hkv", 0), dtype=c.get("dtype", torch.bfloat16))
    if "v_bias" in c:
        inp.v = (inp.v.float() + c["v_bias"]).to(inp.v.dtype)
    sv = c.get("smooth_v", False)
    pbm = c.get("per_block_mean", False)
    q, k, v = inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    cq, ck = inp.cu_q.to(DEV), inp.cu_k.to(DEV)
    mq, mk = max(c["sq"]), max(c["sk"])
    out, lse = sage.sageattn_varlen(q, k, v, cq, ck, mq, mk, is_causal=causal, return_lse=True, pv_dtype=pv,
                                    smooth_v=sv, per_block_mean=pbm)
    g = sage.quantize_qk_varlen(q, k, cq, ck, mq, mk, per_block_mean=pbm)
    torch.cuda.synchronize()
    assert out.shape == q.shape and out.dtype == q.dtype and lse.shape == (c["H"], q.shape[0])
    Q, K, V = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    cuq, cuk = inp.cu_q.tolist(), inp.cu_k.tolist()

    # quantization of each sequence, bit for bit against the dense oracle on that sequence alone
    for b in range(len(c["sq"])):
        q0, q1, k0, k1 = cuq[b], cuq[b + 1], cuk[b], cuk[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        cq_ = orc.quant_qk(np.ascontiguousarray(Q[q0:q1].transpose(1, 0, 2)[None]),
                           np.ascontiguousarray(K[k0:k1].transpose(1, 0, 2)[None]), dtype=inp.dtype,
                           per_block_mean=pbm)
        nqp, nkp = cq_.q8.shape[2], cq_.k8.shape[2]
        assert np.array_equal(g.q8[b, :, :nqp].cpu().numpy(), cq_.q8[0]), ("q8", b)
        assert np.array_equal(g.k8[b, :, :nkp].cpu().numpy(), cq_.k8[0]), ("k8", b)
        assert not g.q8[b, :, nqp:].any() and not g.k8[b, :, nkp:].any()
        assert np.array_equal(g.q_scale[b, :, :cq_.qs.shape[2]].cpu().numpy(), cq_.qs[0])
        assert np.array_equal(g.k_scale[b, :, :cq_.ks.shape[2]].cpu().numpy(), cq_.ks[0])
        if pbm:
            nb = cq_.kmean.shape[2]
            assert np.array_equal(g.k_block_mean[b, :, :nb].cpu().numpy(), cq_.kmean[0])
            assert np.allclose(g.blk_corr[b, :, :nb, :q1 - q0].cpu().numpy(), cq_.corr_blk[0], rtol=1e-5, atol=1e-4)
        else:
            assert np.array_equal(g.k_mean[b].cpu().numpy(), cq_.kmean[0])
    say("  per-sequence quantization bit-exact")

    o32, o16, qlse = orc.run_qe_varlen(Q, K, V, cuq, cuk, pv=pv, causal=causal, dtype=inp.dtype, smooth_v=sv,
                                       per_block_mean=pbm, **qe_schedule(pv))
    plain = o16 if TAU[pv] == 0 else orc.run_qe_varlen(Q, K, V, cuq, cuk, pv=pv, causal=causal, dtype=inp.dtype,
                                                       smooth_v=sv, per_block_mean=pbm, tau=0.0)[1]
    got = out.float().cpu().numpy()
    check_o(got, _dec(o16, inp.dtype), pv, "varlen", plain=_dec(plain, inp.dtype))
    assert_lse_close(lse.cpu().numpy(), qlse, 1e-3)
    eo, el = orc.attn_ex_varlen(Q, K, V, cuq, cuk, causal=causal, dtype=inp.dtype)
    live = np.abs(eo).sum(-1) > 0
    if live.any():
        assert cosine(got[live], eo[live]) >= 0.999
        assert rel_l1(got[live], eo[live]) <= (3e-2 if pv == "fp16" else 5e-2)
    # rows of a sequence without keys: O = 0, LSE = -inf
    for b in range(len(c["sq"])):
        if cuk[b + 1] == cuk[b] and cuq[b + 1] > cuq[b]:
            assert (got[cuq[b]:cuq[b + 1]] == 0).all() and torch.isneginf(lse[:, cuq[b]:cuq[b + 1]]).all()


def test_varlen_one_sequence_equals_dense():
    """One packed sequence gives what the dense path gives for B = 1 (same kernels, other addressing)."""
    inp = make_varlen_inputs([777], [777], 4, 128, seed=61)
    q, k, v = inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    o, l = sage.sageattn_varlen(q, k, v, inp.cu_q.to(DEV), inp.cu_k.to(DEV), 777, 777, is_causal=True,
                                return_lse=True)
    od, ld = sage.sageattn(q[None], k[None], v[None], tensor_layout="NHD", is_causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, od[0]) and torch.equal(l, ld[0])


def test_varlen_errors():
    inp = make_varlen_inputs([64, 64], [64, 64], 2, 64, seed=62)
    q, k, v = inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    with pytest.raises(ValueError):  # cu_seqlens on the host
        sage.sageattn_varlen(q, k, v, inp.cu_q, inp.cu_k.to(DEV), 64, 64)
    with pytest.raises(ValueError):  # int64 cu_seqlens
        sage.sageattn_varlen(q, k, v, inp.cu_q.to(DEV).long(), inp.cu_k.to(DEV), 64, 64)
    with pytest.raises(ValueError):
        sage.sageattn_varlen(q, k, v, inp.cu_q.to(DEV), inp.cu_k.to(DEV), 64, 64, smooth_k=False)
