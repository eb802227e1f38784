"""ctypes binding of the FP4 microscaling attention (include/sage_fp4.h).

Argument marshalling only; every step runs in the library's gfx950 kernels.  Shaped like the
pages' ``sageattn3_blackwell(q, k, v, is_causal, per_block_mean)`` (SageAttention docs digest,
"FP4 Attention for Blackwell GPUs") with the quantize -> attention split and the out / lse /
sm_scale / return_lse parameters of the FlashInfer API doc (flashinfer.nvfp4_attention_sm120_fwd)::

    out = sageattn_fp4(q, k, v, is_causal=False, per_block_mean=True, sm_scale=None, return_lse=False)

FP4 is OCP MX FP4 (e2m1 elements, one E8M0 scale per 32 elements), the block-scale format of
gfx950's scaled MFMA.  q, k, v: bf16 or fp16 [B, H, N, 128] (HND), k and v with Hkv heads.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from .api import FP4QKV, _check, _desc, _dtype_code, _stream, load_library, pad_tokens, sm_scale_arg


@dataclass
class QuantizedFP4:
    """Device buffers of sage_fp4_qkv (layouts in include/sage_fp4.h)."""
    q4: torch.Tensor        # uint8 [B, H, Nq_pad, d/2]
    q_scale: torch.Tensor   # uint8 [B, H, Nq_pad, d/32]
    k4: torch.Tensor        # uint8 [B, Hkv, Nk_pad, d/2]
    k_scale: torch.Tensor   # uint8 [B, Hkv, Nk_pad, d/32]
    v4t: torch.Tensor       # uint8 [B, Hkv, d, Nk_pad/2]
    v_scale: torch.Tensor   # uint8 [B, Hkv, Nk_pad/32, d]
    k_mean: torch.Tensor    # fp32 [B, Hkv, d]
    q_mean: torch.Tensor    # fp32 [B, H, nqm, d]
    qk_corr: torch.Tensor   # fp32 [B, H, nqm, Nk_pad]
    lse_corr: torch.Tensor  # fp32 [B, H, Nq]
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    per_block_mean: bool
    dtype: torch.dtype = torch.bfloat16

    def cstruct(self) -> FP4QKV:
        return FP4QKV(self.q4.data_ptr(), self.q_scale.data_ptr(), self.k4.data_ptr(), self.k_scale.data_ptr(),
                      self.v4t.data_ptr(), self.v_scale.data_ptr(), self.k_mean.data_ptr(), self.q_mean.data_ptr(),
                      self.qk_corr.data_ptr(), self.lse_corr.data_ptr(), self.B, self.H, self.Hkv, self.Nq, self.Nk,
                      self.d, self.q4.shape[2], self.k4.shape[2], 1 if self.per_block_mean else 0)


def softmax_tau_fp4() -> int:
    """Lazy-maximum threshold (whole log2 units) of the FP4 attention kernel's online softmax."""
    return int(load_library().sage_fp4_softmax_tau())


def q_blocks(Nq: int, per_block_mean: bool) -> int:
    return int(load_library().sage_fp4_q_blocks(Nq, 1 if per_block_mean else 0))


def alloc_fp4(B, H, Hkv, Nq, Nk, d, device, per_block_mean=True, dtype=torch.bfloat16) -> QuantizedFP4:
    nq, nk, nqm = pad_tokens(Nq), pad_tokens(Nk), q_blocks(Nq, per_block_mean)
    u8, f32 = torch.uint8, torch.float32
    e = lambda *s, dt=u8: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
    return QuantizedFP4(e(B, H, nq, d // 2), e(B, H, nq, d // 32), e(B, Hkv, nk, d // 2), e(B, Hkv, nk, d // 32),
                        e(B, Hkv, d, nk // 2), e(B, Hkv, nk // 32, d), e(B, Hkv, d, dt=f32), e(B, H, nqm, d, dt=f32),
                        e(B, H, nqm, nk, dt=f32), e(B, H, Nq, dt=f32), B, H, Hkv, Nq, Nk, d, bool(per_block_mean),
                        dtype)


def fp4_workspace(B, H, Hkv, Nq, Nk, d, device) -> torch.Tensor:
    n = int(load_library().sage_fp4_workspace_bytes(B, H, Hkv, Nq, Nk, d))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def quantize_qkv_fp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, per_block_mean: bool = True,
                     out: QuantizedFP4 | None = None, workspace: torch.Tensor | None = None) -> QuantizedFP4:
    """Smoothing (K by its global mean; Q by its 128-token block means or global mean), MX FP4
    codes and scales of Q, K (per 32 channels) and V (per 32 tokens), the correction rows."""
    L = load_library()
    dq, dk, dv = _desc(q, "HND"), _desc(k, "HND"), _desc(v, "HND")
    if out is None:
        out = alloc_fp4(dq.B, dq.H, dk.H, dq.N, dk.N, dq.d, q.device, per_block_mean, q.dtype)
    out.dtype = q.dtype
    if workspace is None:
        workspace = fp4_workspace(dq.B, dq.H, dk.H, dq.N, dk.N, dq.d, q.device)
    cs = out.cstruct()
    _check(L.sage_fp4_quantize_qkv(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(cs),
                                   workspace.data_ptr(), workspace.numel(), _stream(q)), "sage_fp4_quantize_qkv")
    return out


def attn_fwd_fp4(qkv: QuantizedFP4, *, is_causal: bool = False, sm_scale: float | None = None,
                 return_lse: bool = False, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                 out_dtype: torch.dtype | None = None):
    """Attention on the packed FP4 tensors.  Returns out [B, H, Nq, d] (default: the input dtype) or
    (out, lse) with lse fp32 [B, H, Nq]."""
    L = load_library()
    dev = qkv.q4.device
    if out is None:
        out = torch.empty(qkv.B, qkv.H, qkv.Nq, qkv.d, dtype=out_dtype or qkv.dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty(qkv.B, qkv.H, qkv.Nq, dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != qkv.B * qkv.H * qkv.Nq):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    cs = qkv.cstruct()
    _check(L.sage_fp4_attn_fwd(ctypes.byref(cs), 1 if is_causal else 0, sm_scale_arg(sm_scale),
                               out.data_ptr(), _dtype_code(out.dtype, "out", allow_f32=True), out.stride(0),
                               out.stride(1), out.stride(2), None if lse is None else lse.data_ptr(), _stream(out)),
           "sage_fp4_attn_fwd")
    return (out, lse) if return_lse else out


def sageattn_fp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool = False,
                 per_block_mean: bool = True, sm_scale: float | None = None, return_lse: bool = False):
    """FP4 microscaling attention forward.  q: bf16 or fp16 [B, H, N, 128] (HND); k, v: the same
    dtype with Hkv heads dividing H.  Returns out (q's dtype) or (out, lse)."""
    if q.shape[-1] != 128:
        raise ValueError("head_dim must be 128")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must have the same dtype")
    qkv = quantize_qkv_fp4(q, k, v, per_block_mean=per_block_mean)
    return attn_fwd_fp4(qkv, is_causal=is_causal, sm_scale=sm_scale, return_lse=return_lse)


def debug_scores_fp4(qkv: QuantizedFP4, b: int, h: int, row0: int, nrows: int, col0: int, ncols: int) -> torch.Tensor:
    """Raw fp32 scores S (before sm_scale) of a window, by the attention kernel's tile code."""
    L = load_library()
    out = torch.empty(nrows, ncols, dtype=torch.float32, device=qkv.q4.device)
    cs = qkv.cstruct()
    _check(L.sage_fp4_debug_scores(ctypes.byref(cs), b, h, row0, nrows, col0, ncols, out.data_ptr(), _stream(out)),
           "sage_fp4_debug_scores")
    return out
