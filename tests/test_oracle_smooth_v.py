"""Pins for the oracle's smooth_v (docs digest, "SageAttention CUDA INT8/FP16 Kernel (Ampere sm80)":
per-channel V mean subtracted for biased value tensors, FP16 PV).

The probabilities of a row sum to one, so subtracting a per-channel constant from V and adding it
back to the output is exact in real arithmetic: values constant over tokens come out exactly, the
LSE does not move, and on V with a large channel bias smoothing removes the FP16 rounding error
that the bias causes, measured against fp64 exact attention.
"""

import numpy as np
import pytest
import torch

from quantized_attention_quantize_amd.synthetic import make_inputs


def _bits(x, dtype=torch.bfloat16):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_constant_values_come_out_exactly(orc, H, Hkv):
    inp = make_inputs(1, H, 100, 150, 64, seed=70, Hkv=Hkv)
    Qb, Kb = inp.bits(inp.q), inp.bits(inp.k)
    c = np.linspace(-50, 50, 64).astype(np.float32)
    V = np.stack([np.broadcast_to(c + 10 * hk, (150, 64)) for hk in range(Hkv)])[None]  # per key/value head
    Vb = _bits(V)
    cv = (Vb[0, :, 0].astype(np.uint32) << 16).view(np.float32)  # [Hkv, d]: the bf16 values
    r = orc.run_qe(Qb, Kb, Vb, smooth_v=True, causal=True)
    want = np.repeat(cv, H // Hkv, axis=0)[:, None, :]  # query head h reads key/value head h // (H / Hkv)
    assert np.array_equal(r.o32.reshape(H, 100, 64), np.broadcast_to(want, (H, 100, 64)))
    r0 = orc.run_qe(Qb, Kb, Vb, causal=True)
    assert np.array_equal(r.lse, r0.lse)  # V does not enter the LSE


def test_smooth_v_keeps_empty_rows_empty(orc):
    inp = make_inputs(1, 1, 40, 64, 64, seed=71)
    mask = np.ones((1, 1, 40, 64), np.uint8)
    mask[0, 0, 5] = 0
    r = orc.run_qe(inp.bits(inp.q), inp.bits(inp.k), _bits(inp.v.float().numpy() + 30.0), smooth_v=True, mask=mask)
    assert (r.o32[5] == 0).all() and np.isneginf(r.lse[5])


@pytest.mark.parametrize("bias,gain", [(30.0, 1.0), (200.0, 2.5)])
def test_smooth_v_is_what_buys_accuracy_on_biased_values(orc, bias, gain):
    N, d = 512, 128
    inp = make_inputs(1, 2, N, N, d, sigma=4.0, seed=72)
    Qb, Kb = inp.bits(inp.q), inp.bits(inp.k)
    rng = np.random.default_rng(3)
    V = inp.v.float().numpy() + bias * rng.choice([-1.0, 1.0], size=(1, 2, 1, d)).astype(np.float32)
    Vb = _bits(V)
    eo, _ = orc.attn_ex(Qb, Kb, Vb)
    plain = orc.run_qe(Qb, Kb, Vb)
    smooth = orc.run_qe(Qb, Kb, Vb, smooth_v=True)
    err_plain = np.abs(plain.o32 - eo).mean()
    err_smooth = np.abs(smooth.o32 - eo).mean()
    assert err_smooth * gain < err_plain, (err_smooth, err_plain)
    # smoothing V leaves the attention weights alone: the error is that of the unbiased problem
    unb = orc.run_qe(Qb, Kb, _bits(inp.v.float().numpy()))
    eo_unb, _ = orc.attn_ex(Qb, Kb, inp.bits(inp.v))
    assert err_smooth < 3 * np.abs(unb.o32 - eo_unb).mean() + 1e-4
    np.testing.assert_array_equal(smooth.lse, plain.lse)


def test_smooth_v_rejects_fp8(orc):
    inp = make_inputs(1, 1, 64, 64, 64, seed=73)
    with pytest.raises(ValueError):
        orc.prep_v(inp.bits(inp.v), "fp8", vmean=np.zeros((1, 1, 64), np.float32))
