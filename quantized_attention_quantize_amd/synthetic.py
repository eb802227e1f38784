"""Seeded synthetic inputs for the quantized-attention workloads.

This module holds the workload shapes and the random-input recipe and nothing of the method's
arithmetic; both the HIP path's tests/benchmark and the CPU oracle consume what it produces.

The recipe follows the examples on the SageAttention docs digest (context7 llms.txt), sections
"SageAttention Triton INT8/FP16 Kernel Examples" and "sageattn -- Auto-selecting attention kernel":
plain ``torch.randn`` bf16 tensors in HND layout, and a boolean mask that keeps the first half of
the keys.  Keys additionally carry a per-(batch, head, channel) bias of standard deviation sigma, the
channel-wise offset that key smoothing exists to remove.

Draw order (fp32, one CPU generator seeded with ``seed``; Hk = H, or the key/value head count of a
group-query workload):
    Q  = randn(B, H, Nq, d)
    Kn = randn(B, Hk, Nk, d)
    Kb = sigma * randn(B, Hk, 1, d)
    V  = randn(B, Hk, Nk, d)
then K = bf16(Kn + Kb), Q = bf16(Q), V = bf16(V) (or fp16 of the same draws for fp16 inputs).

``additive_mask`` turns a boolean mask into the equivalent float32 additive mask (0 to attend, -inf
to drop) and ``random_additive_mask`` draws a float32 mask with finite biases and -inf holes.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    sigma: float
    causal: bool = False
    # None, "half_keys" ([B,1,Nq,Nk] bool, True for keys < Nk/2) or "half_keys_f32" (the same as a
    # float32 additive mask: 0 for keys < Nk/2, -inf beyond)
    mask: str | None = None
    pv: str = "fp16"  # "fp16" or "fp8"
    lse: bool = True
    note: str = field(default="", compare=False)
    Hkv: int = 0  # key/value heads (group-query attention); 0 = H
    dtype: str = "bf16"  # element type of q, k, v and the output: "bf16" or "fp16"
    kv_splits: int = 1  # > 1: the keys run as this many slices with fp32 partial results, then merged
    seqlens: tuple = ()  # a packed variable-length batch of these sequence lengths (B, Nq, Nk: count, longest)
    smooth_v: bool = False  # V's channel means subtracted before its FP16 rounding, added back to O
    per_block_mean: bool = False  # INT8: K smoothed by each 64-token block's own mean; FP4: Q by its 128-token blocks'
    method: str = "int8"  # "int8" (INT8 QK, FP16/FP8 PV) or "fp4" (MX FP4 Q/K/V, e4m3 P)

    @property
    def ops(self) -> float:
        """Throughput numerator 4*B*H*Nq*Nk*d (summed over the sequences of a packed batch), halved
        for causal."""
        if self.seqlens:
            o = 4.0 * self.H * self.d * float(sum(n * n for n in self.seqlens))
        else:
            o = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return o / 2 if self.causal else o


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 256, 64, 4.0, pv="fp16",
                     note="B=1 H=2 N=256 d=64, INT8 QK (64-token blocks) + FP16 PV, seed 0"),
    "n8k": Workload("n8k", 2, 32, 8192, 8192, 128, 4.0, pv="fp16",
                    note="B=2 H=32 N=8192 d=128 bf16, non-causal, INT8 QK + FP16 PV, bf16 out + fp32 LSE"),
    "n8k_causal": Workload("n8k_causal", 2, 32, 8192, 8192, 128, 4.0, causal=True, pv="fp16",
                           note="B=2 H=32 N=8192 d=128 bf16, causal, INT8 QK + FP16 PV"),
    "n8k_mask": Workload("n8k_mask", 2, 32, 8192, 8192, 128, 4.0, mask="half_keys", pv="fp16",
                         note="B=2 H=32 N=8192 d=128 bf16, bool mask [B,1,N,N] keeping keys < N/2, LSE"),
    "n17776_fp8": Workload("n17776_fp8", 1, 24, 17776, 17776, 128, 8.0, pv="fp8",
                           note="B=1 H=24 N=17776 d=128 bf16, non-causal, INT8 QK + FP8 e4m3 PV"),
    "n8k_gqa": Workload("n8k_gqa", 2, 32, 8192, 8192, 128, 4.0, pv="fp16", Hkv=8,
                        note="B=2 H=32 over 8 K/V heads, N=8192 d=128 bf16, non-causal, INT8 QK + FP16 PV, LSE"),
    "n8k_fp16": Workload("n8k_fp16", 2, 32, 8192, 8192, 128, 4.0, pv="fp16", dtype="fp16",
                         note="B=2 H=32 N=8192 d=128 fp16 in and out, non-causal, INT8 QK + FP16 PV, LSE"),
    "n8k_split2": Workload("n8k_split2", 2, 32, 8192, 8192, 128, 4.0, pv="fp16", kv_splits=2,
                           note="B=2 H=32 N=8192 d=128 bf16, keys in 2 slices of 4096 (each quantized with its own K "
                                "mean), fp32 partial O + LSE, merged to bf16 O + LSE"),
    "varlen_mix": Workload("varlen_mix", 8, 32, 8192, 8192, 128, 4.0, pv="fp16", dtype="fp16",
                           seqlens=(8192, 4096, 2048, 6144, 1024, 3072, 512, 7680),
                           note="packed batch of 8 sequences (8192, 4096, 2048, 6144, 1024, 3072, 512, 7680 tokens; "
                                "32768 in all), H=32 d=128 fp16, non-causal, INT8 QK + FP16 PV, LSE"),
    "n8k_smoothv_pbm": Workload("n8k_smoothv_pbm", 2, 32, 8192, 8192, 128, 4.0, pv="fp16", smooth_v=True,
                                per_block_mean=True,
                                note="B=2 H=32 N=8192 d=128 bf16, non-causal, INT8 QK with per-block K means + FP16 PV "
                                     "with smooth_v, LSE"),
    "fp4_b1h24n4096": Workload("fp4_b1h24n4096", 1, 24, 4096, 4096, 128, 4.0, lse=False, per_block_mean=True,
                               method="fp4",
                               note="B=1 H=24 N=4096 d=128 bf16, non-causal, MX FP4 Q/K/V (Q smoothed by 128-token "
                                    "block means) + e4m3 P, bf16 out"),
    "n8k_fp4": Workload("n8k_fp4", 2, 32, 8192, 8192, 128, 4.0, per_block_mean=True, method="fp4",
                        note="B=2 H=32 N=8192 d=128 bf16, non-causal, MX FP4 Q/K/V (Q smoothed by 128-token block "
                             "means) + e4m3 P, bf16 out + fp32 LSE"),
    "n8k_fmask": Workload("n8k_fmask", 2, 32, 8192, 8192, 128, 4.0, mask="half_keys_f32", pv="fp16",
                          note="B=2 H=32 N=8192 d=128 bf16, float32 additive mask [B,1,N,N]: 0 for keys < N/2, "
                               "-inf beyond, LSE"),
}


@dataclass
class Inputs:
    q: torch.Tensor  # bf16 or fp16 [B,H,Nq,d] (CPU)
    k: torch.Tensor
    v: torch.Tensor
    mask: torch.Tensor | None  # bool or float32 [B,1,Nq,Nk] (CPU) or None

    def bits(self, t: torch.Tensor) -> np.ndarray:
        """bf16 / fp16 tensor -> numpy uint16 bit patterns (what the oracle consumes)."""
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    @property
    def dtype(self) -> str:
        """"bf16" or "fp16": the element type of q, k and v."""
        return "fp16" if self.q.dtype == torch.float16 else "bf16"

    @property
    def mask_u8(self):
        """The mask as the oracle takes it: uint8 for a boolean mask, float32 as it is."""
        if self.mask is None:
            return None
        return self.mask.numpy() if self.mask.dtype == torch.float32 else self.mask.numpy().astype(np.uint8)


def make_inputs(B, H, Nq, Nk, d, sigma=4.0, seed=0, mask=None, Hkv=0, dtype=torch.bfloat16) -> Inputs:
    """Hkv > 0 draws K and V with Hkv heads (group-query attention), in the same order.  dtype is
    torch.bfloat16 or torch.float16."""
    assert dtype in (torch.bfloat16, torch.float16)
    Hk = Hkv if Hkv > 0 else H
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float32)
    kn = torch.randn(B, Hk, Nk, d, generator=g, dtype=torch.float32)
    kb = sigma * torch.randn(B, Hk, 1, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hk, Nk, d, generator=g, dtype=torch.float32)
    k = (kn + kb).to(dtype)
    del kn
    m = None
    if mask in ("half_keys", "half_keys_f32"):
        m = torch.ones(B, 1, Nq, Nk, dtype=torch.bool)
        m[:, :, :, Nk // 2:] = False
        if mask == "half_keys_f32":
            m = additive_mask(m)
    elif mask is not None:
        raise ValueError(mask)
    return Inputs(q.to(dtype), k, v.to(dtype), m)


def workload_inputs(w: Workload, seed: int = 0) -> Inputs:
    return make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.sigma, seed, w.mask, w.Hkv,
                       torch.float16 if w.dtype == "fp16" else torch.bfloat16)


def random_mask(B, Hm, Nq, Nk, p_keep=0.7, seed=1) -> torch.Tensor:
    """Element-wise random boolean mask (True = attend) for edge-case tests."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.rand(B, Hm, Nq, Nk, generator=g) < p_keep


def additive_mask(mask: torch.Tensor) -> torch.Tensor:
    """Boolean mask (True = attend) -> float32 additive mask: 0 where True, -inf where False."""
    return torch.zeros(mask.shape, dtype=torch.float32).masked_fill(~mask, float("-inf"))


def random_additive_mask(B, Hm, Nq, Nk, p_drop=0.2, scale=2.0, seed=3) -> torch.Tensor:
    """float32 additive mask: biases scale * randn, with a fraction p_drop of entries at -inf."""
    g = torch.Generator("cpu").manual_seed(seed)
    m = scale * torch.randn(B, Hm, Nq, Nk, generator=g, dtype=torch.float32)
    drop = torch.rand(B, Hm, Nq, Nk, generator=g) < p_drop
    return m.masked_fill(drop, float("-inf"))


@dataclass
class VarlenInputs:
    q: torch.Tensor  # [total_q, H, d] (CPU), packed
    k: torch.Tensor  # [total_k, Hkv, d]
    v: torch.Tensor
    cu_q: torch.Tensor  # int32 [nseq + 1], starts at 0
    cu_k: torch.Tensor

    def bits(self, t: torch.Tensor) -> np.ndarray:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    @property
    def dtype(self) -> str:
        return "fp16" if self.q.dtype == torch.float16 else "bf16"


def make_varlen_inputs(seqlens_q, seqlens_k, H, d, sigma=4.0, seed=0, Hkv=0, dtype=torch.bfloat16) -> VarlenInputs:
    """Packed variable-length batch, as in the docs digest's ``sageattn_varlen`` example: sequence b
    has seqlens_q[b] query and seqlens_k[b] key rows.  Draws (fp32, one generator): Q = randn(Tq,H,d),
    Kn = randn(Tk,Hk,d), Kb = sigma * randn(nseq,Hk,d) (each sequence's key-channel offset, added to
    its rows), V = randn(Tk,Hk,d)."""
    Hk = Hkv if Hkv > 0 else H
    Tq, Tk = int(sum(seqlens_q)), int(sum(seqlens_k))
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(Tq, H, d, generator=g, dtype=torch.float32)
    k = torch.randn(Tk, Hk, d, generator=g, dtype=torch.float32)
    kb = sigma * torch.randn(len(seqlens_k), Hk, d, generator=g, dtype=torch.float32)
    v = torch.randn(Tk, Hk, d, generator=g, dtype=torch.float32)
    cu_q = torch.tensor([0] + list(np.cumsum(seqlens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(seqlens_k)), dtype=torch.int32)
    for b in range(len(seqlens_k)):
        k[cu_k[b]:cu_k[b + 1]] += kb[b]
    return VarlenInputs(q.to(dtype), k.to(dtype), v.to(dtype), cu_q, cu_k)
