"""GPU parity of the LSE merge (sage_merge_lse) and a split-KV run on one GPU.

Merge kernel: random partial results (fp32, bf16, fp16 parts; rows where some or all parts saw no
key) against the oracle's merge, rel-L1 <= 1e-6 for fp32 output (1e-3 for 16-bit output) and LSE
within 1e-5.  Split-KV: the keys are cut into slices, the whole quantized method runs on each slice
(own K mean and blocks) with fp32 partial outputs, and the merge gives the result over all keys;
this is compared with the oracle's merge of its own per-slice emulations (rel-L1 <= 1e-3, LSE
1e-3) and with exact attention over all keys (the usual accuracy bars).  A split by boolean masks
over the full key range checks parts that are empty for some rows.
"""

import numpy as np
import pytest
import torch

import quantized_attention_quantize_amd as sage
from quantized_attention_quantize_amd.synthetic import make_inputs

from gpu_helpers import DEV, assert_lse_close, check_o, cosine, f32_of_bf16_bits, qe_schedule, rel_l1, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sage.load_library()


def _as_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


@pytest.mark.parametrize("S", [1, 2, 3])
@pytest.mark.parametrize("part_dtype,out_dtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16),
                                                  (torch.float16, torch.float32), (torch.float32, torch.float16)])
def test_merge_kernel_vs_oracle(orc, S, part_dtype, out_dtype):
    say(f"merge S={S} parts {part_dtype} out {out_dtype}")
    B, H, Nq, d = 2, 3, 77, 128
    g = torch.Generator().manual_seed(30 + S)
    parts = torch.randn(S, B, H, Nq, d, generator=g).to(part_dtype)
    lse = (4 * torch.randn(S, B, H, Nq, generator=g)).float()
    lse[0, 0, 0, 5] = float("-inf")  # a part that saw no key of this row
    parts[0, 0, 0, 5] = 0
    lse[:, 1, 2, 9] = float("-inf")  # a row no part saw
    parts[:, 1, 2, 9] = 0
    out, ml = sage.merge_lse(parts.to(DEV), lse.to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    R = B * H * Nq
    wo, wl = orc.merge_lse(parts.float().numpy().reshape(S, R, d), lse.numpy().reshape(S, R))
    got = _as_f32(out).reshape(R, d)
    tol = 1e-6 if out_dtype == torch.float32 else 2e-3
    assert rel_l1(got, wo) <= tol
    assert_lse_close(ml.cpu().numpy().reshape(R), wl, 1e-5)
    dead = (1 * H + 2) * Nq + 9
    assert (got[dead] == 0).all() and np.isneginf(ml.reshape(R)[dead].item())


def test_merge_into_strided_output():
    """The merged output may be written through strides (here into an NHD buffer)."""
    S, B, H, Nq, d = 2, 1, 4, 50, 64
    g = torch.Generator().manual_seed(40)
    parts = torch.randn(S, B, H, Nq, d, generator=g).to(DEV)
    lse = torch.randn(S, B, H, Nq, generator=g).to(DEV)
    ref, _ = sage.merge_lse(parts, lse)
    nhd = torch.full((B, Nq, H, d), 7.0, device=DEV)
    sage.merge_lse(parts, lse, out=nhd.permute(0, 2, 1, 3), return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(nhd.permute(0, 2, 1, 3), ref)


@pytest.mark.parametrize("pv,cuts", [("fp16", (0, 320, 700)), ("fp16", (0, 64, 129, 700)), ("fp8", (0, 448, 700))])
def test_split_kv_slices(orc, pv, cuts):
    B, H, N, d = 1, 2, 700, 128
    say(f"split-kv {pv} cuts={cuts}")
    inp = make_inputs(B, H, N, N, d, sigma=4.0 if pv == "fp16" else 8.0, seed=41)
    q, k, v = to_dev(inp)
    S = len(cuts) - 1
    o_parts = torch.empty(S, B, H, N, d, dtype=torch.float32, device=DEV)
    l_parts = torch.empty(S, B, H, N, dtype=torch.float32, device=DEV)
    for s, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        qk = sage.quantize_qk(q, k[:, :, lo:hi].contiguous())
        sage.attn_fwd(qk, v[:, :, lo:hi].contiguous(), pv_dtype=pv, return_lse=True, out=o_parts[s], lse=l_parts[s])
    out, lse = sage.merge_lse(o_parts, l_parts, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    R = B * H * N
    qe = [orc.run_qe(Qb, np.ascontiguousarray(Kb[:, :, lo:hi]), np.ascontiguousarray(Vb[:, :, lo:hi]), pv=pv,
                     **qe_schedule(pv))
          for lo, hi in zip(cuts[:-1], cuts[1:])]
    # each part against its own emulation first (fp32 outputs: the kernel's unrounded O)
    for s, r in enumerate(qe):
        check_o(o_parts[s].cpu().numpy().reshape(R, d), r.o32, pv, f"part {s} (fp32 O)")
    wo, wl = orc.merge_lse(np.stack([r.o32 for r in qe]), np.stack([r.lse for r in qe]))
    got = _as_f32(out).reshape(R, d)
    e1 = rel_l1(got, f32_of_bf16_bits(orc.f32_to_bf16(wo.astype(np.float32))))  # both rounded to bf16
    say(f"  merged vs merged emulation rel-L1 {e1:.3e}")
    assert e1 <= 1e-3
    assert_lse_close(lse.cpu().numpy().reshape(R), wl, 1e-3)
    eo, el = orc.attn_ex(Qb, Kb, Vb)
    assert cosine(got, eo) >= 0.999
    assert rel_l1(got, eo) <= (3e-2 if pv == "fp16" else 5e-2)
    assert np.abs(lse.cpu().numpy().reshape(R) - el).max() < 2e-2


def test_split_by_masks_with_empty_parts(orc):
    """Parts defined by boolean masks over the full key range, causal within: early rows see none
    of the later parts (LSE -inf there), which the merge must ignore."""
    B, H, N, d = 1, 2, 520, 64
    inp = make_inputs(B, H, N, N, d, seed=42)
    q, k, v = to_dev(inp)
    cuts = (0, 200, 520)
    qk = sage.quantize_qk(q, k)  # one quantization over all keys
    o_parts, l_parts, masks = [], [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        m = torch.zeros(B, 1, N, N, dtype=torch.bool)
        m[..., lo:hi] = True
        masks.append(m)
        o, l = sage.attn_fwd(qk, v, is_causal=True, attn_mask=m.to(DEV), return_lse=True,
                             out=torch.empty(B, H, N, d, dtype=torch.float32, device=DEV))
        o_parts.append(o)
        l_parts.append(l)
    out, lse = sage.merge_lse(torch.stack(o_parts), torch.stack(l_parts), out_dtype=torch.bfloat16)
    full_o, full_l = sage.sageattn(q, k, v, is_causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isneginf(l_parts[1][0, 0, :200]).all()
    R = B * H * N
    # the same quantization and the same keys: the merge reproduces the single pass up to rounding
    assert rel_l1(_as_f32(out).reshape(R, d), _as_f32(full_o).reshape(R, d)) <= 2e-3
    assert_lse_close(lse.cpu().numpy().reshape(R), full_l.cpu().numpy().reshape(R), 1e-4)
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    r = orc.run_qe(Qb, Kb, Vb, causal=True, **qe_schedule("fp16"))
    assert rel_l1(_as_f32(out).reshape(R, d), f32_of_bf16_bits(r.o16)) <= 2e-3
