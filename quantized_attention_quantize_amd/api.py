"""ctypes binding of libsage_mi355x (include/sage_mi355x.h).

Argument marshalling only: torch tensors are turned into device pointers, strides and the current
HIP stream; every step of the computation runs in the library's gfx950 kernels.  If the library
is missing, every call raises -- there is no fallback path.

User-level entry point, shaped like the pages' ``sageattn`` (SageAttention docs digest, context7
llms.txt, section "sageattn -- Auto-selecting attention kernel") plus the boolean or float32
``attn_mask`` of the Triton INT8/FP16 kernel section and the FP8 PV option of
``sageattn_qk_int8_pv_fp8_cuda``; q, k and v are bf16 or fp16 and the output takes their dtype::

    out = sageattn(q, k, v, tensor_layout="HND", is_causal=False, attn_mask=None,
                   sm_scale=None, return_lse=False, pv_dtype="fp16")

Lower-level, mirroring the quantize -> attention split of the FlashInfer API doc
(flashinfer.nvfp4_attention_sm120_fwd): ``quantize_qk`` then ``attn_fwd``.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsage_mi355x.so")

SAGE_BF16, SAGE_FP16, SAGE_F32 = 0, 1, 2
SAGE_MASK_BOOL, SAGE_MASK_F32 = 0, 1
PV_CODES = {"fp16": 0, "fp8": 1, "fp8_e4m3": 1}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}


class SageError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_STATUS.get(status, status)} (status {status})")
        self.status = status


class QKVDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("N", ctypes.c_int64), ("d", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class QKQuant(ctypes.Structure):
    _fields_ = [("q8", ctypes.c_void_p), ("k8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("k_mean", ctypes.c_void_p), ("lse_corr", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("Nq", ctypes.c_int64),
                ("Nk", ctypes.c_int64), ("d", ctypes.c_int64), ("Nq_pad", ctypes.c_int64), ("Nk_pad", ctypes.c_int64),
                ("k_block_mean", ctypes.c_void_p), ("blk_corr", ctypes.c_void_p)]


class FP4QKV(ctypes.Structure):
    """sage_fp4_qkv (include/sage_fp4.h)."""
    _fields_ = [("q4", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k4", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v4t", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_mean", ctypes.c_void_p), ("q_mean", ctypes.c_void_p), ("qk_corr", ctypes.c_void_p),
                ("lse_corr", ctypes.c_void_p), ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64), ("d", ctypes.c_int64), ("Nq_pad", ctypes.c_int64),
                ("Nk_pad", ctypes.c_int64), ("per_block_mean", ctypes.c_int)]


_lib = None

EXPORTS = ("sage_pad_tokens", "sage_block_n", "sage_softmax_tau", "sage_rowsum_rounded", "sage_quantize_workspace_bytes", "sage_quantize_qk",
           "sage_prepare_v_workspace_bytes", "sage_prepare_v", "sage_mask_workspace_bytes",
           "sage_fwd_workspace_bytes", "sage_attn_fwd", "sage_attn_fwd_prepared", "sage_quantize_qk_varlen",
           "sage_attn_fwd_varlen", "sage_prepare_v_varlen", "sage_attn_fwd_prepared_varlen", "sage_merge_lse",
           "sage_debug_qk_int32", "sage_status_string", "sage_fp4_q_blocks", "sage_fp4_softmax_tau",
           "sage_fp4_workspace_bytes",
           "sage_fp4_quantize_qkv", "sage_fp4_attn_fwd", "sage_fp4_debug_scores", "sage_qk_quant_bytes",
           "sage_qk_quant_init", "sage_quantize_qk_noalloc", "sage_sclk_probe")


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsage_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m quantized_attention_quantize_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.sage_pad_tokens.argtypes = [I64]
    L.sage_pad_tokens.restype = I64
    L.sage_block_n.argtypes = [I]
    L.sage_block_n.restype = I
    L.sage_softmax_tau.argtypes = [I]
    L.sage_softmax_tau.restype = ctypes.c_double
    L.sage_rowsum_rounded.argtypes = [I]
    L.sage_rowsum_rounded.restype = I
    L.sage_quantize_workspace_bytes.argtypes = [I64, I64, I64, I64]
    L.sage_quantize_workspace_bytes.restype = SZ
    L.sage_quantize_qk.argtypes = [ctypes.POINTER(QKVDesc), ctypes.POINTER(QKVDesc), ctypes.POINTER(QKQuant), P, SZ, P]
    L.sage_quantize_qk.restype = I
    L.sage_prepare_v_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    L.sage_prepare_v_workspace_bytes.restype = SZ
    L.sage_prepare_v.argtypes = [ctypes.POINTER(QKVDesc), I, P, P, P, P, SZ, P]
    L.sage_prepare_v.restype = I
    L.sage_mask_workspace_bytes.argtypes = [I64, I64, I64, I64]
    L.sage_mask_workspace_bytes.restype = SZ
    L.sage_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I, I64]
    L.sage_fwd_workspace_bytes.restype = SZ
    L.sage_attn_fwd.argtypes = [ctypes.POINTER(QKQuant), ctypes.POINTER(QKVDesc), P, I, I64, I64, I64, I64, I, F, I, I,
                                P, I,
                                I64, I64, I64, P, P, SZ, P]
    L.sage_attn_fwd.restype = I
    L.sage_attn_fwd_prepared.argtypes = [ctypes.POINTER(QKQuant), P, P, P, I, P, I, I64, I64, I64, I64, I, F, P, I, I64,
                                         I64,
                                         I64, P, P, SZ, P]
    L.sage_attn_fwd_prepared.restype = I
    L.sage_quantize_qk_varlen.argtypes = [ctypes.POINTER(QKVDesc), ctypes.POINTER(QKVDesc), P, P, I64, I64,
                                          ctypes.POINTER(QKQuant), P, SZ, P]
    L.sage_quantize_qk_varlen.restype = I
    L.sage_attn_fwd_varlen.argtypes = [ctypes.POINTER(QKQuant), ctypes.POINTER(QKVDesc), P, P, I64, I64, I, F, I, I, P,
                                       I, I64, I64, P, P, SZ, P]
    L.sage_attn_fwd_varlen.restype = I
    L.sage_prepare_v_varlen.argtypes = [ctypes.POINTER(QKVDesc), P, I64, I, P, P, P, P, SZ, P]
    L.sage_prepare_v_varlen.restype = I
    L.sage_attn_fwd_prepared_varlen.argtypes = [ctypes.POINTER(QKQuant), P, P, P, I, P, P, I64, I64, I, F, P, I, I64,
                                                I64, P, P]
    L.sage_attn_fwd_prepared_varlen.restype = I
    L.sage_merge_lse.argtypes = [I64, I64, I64, I64, I64, P, I, P, P, I, I64, I64, I64, P, P]
    L.sage_merge_lse.restype = I
    L.sage_debug_qk_int32.argtypes = [ctypes.POINTER(QKQuant), I64, I64, I64, I64, I64, I64, P, P]
    L.sage_debug_qk_int32.restype = I
    L.sage_qk_quant_bytes.argtypes = [I64, I64, I64, I64, I64, I64, I]
    L.sage_qk_quant_bytes.restype = SZ
    L.sage_qk_quant_init.argtypes = [P, SZ, I64, I64, I64, I64, I64, I64, I, ctypes.POINTER(QKQuant)]
    L.sage_qk_quant_init.restype = I
    L.sage_quantize_qk_noalloc.argtypes = [ctypes.POINTER(QKVDesc), ctypes.POINTER(QKVDesc), ctypes.POINTER(QKQuant),
                                           P]
    L.sage_quantize_qk_noalloc.restype = I
    L.sage_status_string.argtypes = [I]
    L.sage_status_string.restype = ctypes.c_char_p
    L.sage_sclk_probe.argtypes = [I64, I64, I, P, P]
    L.sage_sclk_probe.restype = I
    L.sage_fp4_q_blocks.argtypes = [I64, I]
    L.sage_fp4_q_blocks.restype = I64
    L.sage_fp4_softmax_tau.argtypes = []
    L.sage_fp4_softmax_tau.restype = ctypes.c_double
    L.sage_fp4_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I64]
    L.sage_fp4_workspace_bytes.restype = SZ
    D = ctypes.POINTER(QKVDesc)
    L.sage_fp4_quantize_qkv.argtypes = [D, D, D, ctypes.POINTER(FP4QKV), P, SZ, P]
    L.sage_fp4_quantize_qkv.restype = I
    L.sage_fp4_attn_fwd.argtypes = [ctypes.POINTER(FP4QKV), I, F, P, I, I64, I64, I64, P, P]
    L.sage_fp4_attn_fwd.restype = I
    L.sage_fp4_debug_scores.argtypes = [ctypes.POINTER(FP4QKV), I64, I64, I64, I64, I64, I64, P, P]
    L.sage_fp4_debug_scores.restype = I
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise SageError(status, where)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def pad_tokens(n: int) -> int:
    return int(load_library().sage_pad_tokens(n))


def block_n(pv_dtype: str = "fp16") -> int:
    """Keys per online-softmax tile of the attention kernel."""
    return int(load_library().sage_block_n(PV_CODES[pv_dtype]))


def softmax_tau(pv_dtype: str = "fp16") -> float:
    """Lazy-maximum threshold (log2 units) of the attention kernel's online softmax."""
    return float(load_library().sage_softmax_tau(PV_CODES[pv_dtype]))


def rowsum_rounded(pv_dtype: str = "fp16") -> bool:
    """Whether the attention kernel's softmax denominator sums P as rounded for the PV product."""
    return bool(load_library().sage_rowsum_rounded(PV_CODES[pv_dtype]))


def _dtype_code(dt: torch.dtype, what: str, allow_f32: bool = False) -> int:
    if dt == torch.bfloat16:
        return SAGE_BF16
    if dt == torch.float16:
        return SAGE_FP16
    if allow_f32 and dt == torch.float32:
        return SAGE_F32
    raise ValueError(f"{what} must be bfloat16 or float16{' or float32' if allow_f32 else ''}, got {dt}")


def _desc(t: torch.Tensor, layout: str) -> QKVDesc:
    if t.dim() != 4:
        raise ValueError("q/k/v must be 4-D")
    dt = _dtype_code(t.dtype, "q/k/v")
    if t.stride(3) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    if layout == "HND":
        B, H, N, d = t.shape
        sb, sh, sn = t.stride(0), t.stride(1), t.stride(2)
    elif layout == "NHD":
        B, N, H, d = t.shape
        sb, sh, sn = t.stride(0), t.stride(2), t.stride(1)
    else:
        raise ValueError(f"tensor_layout must be HND or NHD, got {layout}")
    return QKVDesc(t.data_ptr(), dt, B, H, N, d, sb, sh, sn)


@dataclass
class QuantizedQK:
    """Device buffers produced by quantize_qk (see sage_qk_quant in the header).  Q has H heads,
    K has Hkv heads (group-query attention when Hkv < H); dtype is the input dtype of Q and K."""
    q8: torch.Tensor
    k8: torch.Tensor
    q_scale: torch.Tensor
    k_scale: torch.Tensor
    k_mean: torch.Tensor
    lse_corr: torch.Tensor
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    Hkv: int
    dtype: torch.dtype = torch.bfloat16
    k_block_mean: torch.Tensor | None = None  # per_block_mean: [B, Hkv, ceil(Nk/64), d]
    blk_corr: torch.Tensor | None = None  # per_block_mean: [B, H, ceil(Nk/64), Nq]

    def cstruct(self) -> QKQuant:
        return QKQuant(self.q8.data_ptr(), self.k8.data_ptr(), self.q_scale.data_ptr(), self.k_scale.data_ptr(),
                       self.k_mean.data_ptr(), self.lse_corr.data_ptr(), self.B, self.H, self.Hkv, self.Nq, self.Nk,
                       self.d, self.q8.shape[2], self.k8.shape[2],
                       None if self.k_block_mean is None else self.k_block_mean.data_ptr(),
                       None if self.blk_corr is None else self.blk_corr.data_ptr())


def alloc_quantized(B, H, Nq, Nk, d, device, Hkv=None, dtype=torch.bfloat16, per_block_mean=False) -> QuantizedQK:
    Hkv = H if Hkv is None else Hkv
    nq, nk = pad_tokens(Nq), pad_tokens(Nk)
    nbk = (Nk + 63) // 64
    pbm = dict(k_block_mean=torch.empty(B, Hkv, nbk, d, dtype=torch.float32, device=device),
               blk_corr=torch.empty(B, H, nbk, Nq, dtype=torch.float32, device=device)) if per_block_mean else {}
    return QuantizedQK(torch.empty(B, H, nq, d, dtype=torch.int8, device=device),
                       torch.empty(B, Hkv, nk, d, dtype=torch.int8, device=device),
                       torch.empty(B, H, (Nq + 63) // 64, dtype=torch.float32, device=device),
                       torch.empty(B, Hkv, (Nk + 63) // 64, dtype=torch.float32, device=device),
                       torch.empty(B, Hkv, d, dtype=torch.float32, device=device),
                       torch.empty(B, H, Nq, dtype=torch.float32, device=device), B, H, Nq, Nk, d, Hkv, dtype, **pbm)


def quantize_workspace(B, Hkv, Nk, d, device) -> torch.Tensor:
    n = int(load_library().sage_quantize_workspace_bytes(B, Hkv, Nk, d))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def quantize_qk(q: torch.Tensor, k: torch.Tensor, tensor_layout: str = "HND", out: QuantizedQK | None = None,
                workspace: torch.Tensor | None = None, per_block_mean: bool = False) -> QuantizedQK:
    """K mean, per-64-token-block INT8 Q and smoothed K, scales and the LSE shift.  k may have fewer
    heads than q (group-query attention: query head h reads key head h // (H // Hkv)).
    per_block_mean: each 64-token K block is smoothed by its own mean (score terms in blk_corr)."""
    L = load_library()
    dq, dk = _desc(q, tensor_layout), _desc(k, tensor_layout)
    if out is None:
        out = alloc_quantized(dq.B, dq.H, dq.N, dk.N, dq.d, q.device, Hkv=dk.H, dtype=q.dtype,
                              per_block_mean=per_block_mean)
    out.dtype = q.dtype
    if workspace is None:
        workspace = quantize_workspace(dk.B, dk.H, dk.N, dk.d, q.device)
    qs = out.cstruct()
    _check(L.sage_quantize_qk(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(qs), workspace.data_ptr(),
                              workspace.numel(), _stream(q)), "sage_quantize_qk")
    return out


def fwd_workspace(B, Hkv, Nq, Nk, d, pv_dtype, mask_h, device) -> torch.Tensor:
    n = int(load_library().sage_fwd_workspace_bytes(B, Hkv, Nq, Nk, d, PV_CODES[pv_dtype], mask_h))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def sm_scale_arg(sm_scale) -> float:
    """The C ABI's sm_scale: 0 selects 1/sqrt(d) when none is given; an explicit value must be a
    positive finite number."""
    if sm_scale is None:
        return 0.0
    s = float(sm_scale)
    if not math.isfinite(s) or s <= 0.0:
        raise ValueError(f"sm_scale must be a positive finite number, got {sm_scale!r}")
    return s


def _mask_args(attn_mask, B, H, Nq, Nk):
    """(mask, mask dtype code, mask_h, stride_b, stride_h, stride_q) for the C call."""
    if attn_mask is None:
        return None, SAGE_MASK_BOOL, 0, 0, 0, 0
    if attn_mask.dtype == torch.bool:
        code = SAGE_MASK_BOOL
    elif attn_mask.dtype == torch.float32:
        code = SAGE_MASK_F32
    else:
        raise ValueError(f"attn_mask must be bool (True = attend) or float32 (additive), got {attn_mask.dtype}")
    m = attn_mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if m.shape[-1] != Nk or m.shape[-2] not in (1, Nq) or m.shape[0] not in (1, B) or m.shape[1] not in (1, H):
        raise ValueError(f"attn_mask of shape {tuple(attn_mask.shape)} does not broadcast to {(B, H, Nq, Nk)}")
    if m.stride(3) != 1:
        m = m.contiguous()
    mh = m.shape[1]
    sb = m.stride(0) if m.shape[0] == B else 0
    sh = m.stride(1) if mh == H and H > 1 else 0
    sq = m.stride(2) if m.shape[2] == Nq and Nq > 1 else 0  # one row of keys broadcast over the queries
    return m, code, (mh if mh == H else 1), sb, sh, sq


def attn_fwd(qk: QuantizedQK, v: torch.Tensor, *, tensor_layout: str = "HND", is_causal: bool = False,
             attn_mask: torch.Tensor | None = None, sm_scale: float | None = None, pv_dtype: str = "fp16",
             return_lse: bool = False, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None, smooth_v: bool = False):
    """Attention on pre-quantized Q/K (from quantize_qk) with bf16 or fp16 V.  Returns out or (out, lse);
    out defaults to V's dtype.  smooth_v: V's channel means are subtracted before its FP16 rounding
    and added back to O (FP16 PV only)."""
    L = load_library()
    dv = _desc(v, tensor_layout)
    B, H, Nq, Nk, d = qk.B, qk.H, qk.Nq, qk.Nk, qk.d
    if out is None:
        shape = (B, H, Nq, d) if tensor_layout == "HND" else (B, Nq, H, d)
        out = torch.empty(shape, dtype=v.dtype, device=v.device)
    if tensor_layout == "HND":
        osb, osh, osn = out.stride(0), out.stride(1), out.stride(2)
    else:
        osb, osh, osn = out.stride(0), out.stride(2), out.stride(1)
    if return_lse and lse is None:
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=v.device)
    m, mcode, mh, msb, msh, msq = _mask_args(attn_mask, B, H, Nq, Nk)
    if workspace is None:
        workspace = fwd_workspace(B, qk.Hkv, Nq, Nk, d, pv_dtype, mh, v.device)
    qs = qk.cstruct()
    odt = _dtype_code(out.dtype, "out", allow_f32=True)
    _check(L.sage_attn_fwd(ctypes.byref(qs), ctypes.byref(dv), None if m is None else m.data_ptr(), mcode, mh, msb,
                           msh, msq,
                           1 if is_causal else 0, sm_scale_arg(sm_scale), PV_CODES[pv_dtype],
                           1 if smooth_v else 0, out.data_ptr(), odt, osb, osh, osn, None if lse is None else lse.data_ptr(),
                           workspace.data_ptr(), workspace.numel(), _stream(v)), "sage_attn_fwd")
    return (out, lse) if return_lse else out


def sageattn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tensor_layout: str = "HND", is_causal: bool = False,
             attn_mask: torch.Tensor | None = None, sm_scale: float | None = None, return_lse: bool = False,
             pv_dtype: str = "fp16", smooth_v: bool = False, per_block_mean: bool = False):
    """Quantized attention forward: INT8 Q/K with K smoothing, FP16 (or FP8 e4m3) PV.

    q: bf16 or fp16 [B, H, N, d] ("HND") or [B, N, H, d] ("NHD"), d in {64, 128}; k, v: the same
    dtype with Hkv heads, Hkv dividing H (group-query attention: query head h reads key/value head
    h // (H // Hkv)).
    attn_mask: optional, broadcastable to [B, H, Nq, Nk]: bool (True = attend) or float32 (added to
    the scaled scores; -inf masks).
    sm_scale: defaults to 1/sqrt(d).  Returns out (same layout and dtype as q) or (out, lse) with
    lse fp32 [B, H, Nq] (natural log, of the unsmoothed scaled scores).
    """
    if q.shape[-1] not in (64, 128):
        raise ValueError("head_dim must be 64 or 128")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must have the same dtype")
    hk = k.shape[1] if tensor_layout == "HND" else k.shape[2]
    hq = q.shape[1] if tensor_layout == "HND" else q.shape[2]
    if hq % hk != 0:
        raise ValueError(f"the {hk} key/value heads do not divide the {hq} query heads")
    qk = quantize_qk(q, k, tensor_layout, per_block_mean=per_block_mean)
    return attn_fwd(qk, v, tensor_layout=tensor_layout, is_causal=is_causal, attn_mask=attn_mask, sm_scale=sm_scale,
                    pv_dtype=pv_dtype, return_lse=return_lse, smooth_v=smooth_v)


def debug_qk_int32(qk: QuantizedQK, b: int, h: int, row0: int, nrows: int, col0: int, ncols: int) -> torch.Tensor:
    """Raw int32 Q8 . K8^T window of head (b, h) from the attention kernel's own tile code."""
    L = load_library()
    out = torch.empty(nrows, ncols, dtype=torch.int32, device=qk.q8.device)
    qs = qk.cstruct()
    _check(L.sage_debug_qk_int32(ctypes.byref(qs), b, h, row0, nrows, col0, ncols, out.data_ptr(), _stream(out)),
           "sage_debug_qk_int32")
    return out


def alloc_prepared_v(B, H, Nk, d, pv_dtype, device):
    """Buffers for prepare_v: (v_t, v_scale) with v_t [B,H,d,Nk_pad] (int16 fp16 bits or uint8 e4m3)."""
    nkp = pad_tokens(Nk)
    if pv_dtype == "fp16":
        return torch.empty(B, H, d, nkp, dtype=torch.int16, device=device), None
    return (torch.empty(B, H, d, nkp, dtype=torch.uint8, device=device),
            torch.empty(B, H, d, dtype=torch.float32, device=device))


def prepare_v_workspace(B, H, Nk, d, pv_dtype, device) -> torch.Tensor:
    n = int(load_library().sage_prepare_v_workspace_bytes(B, H, Nk, d, PV_CODES[pv_dtype]))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def prepare_v(v: torch.Tensor, pv_dtype: str = "fp16", tensor_layout: str = "HND", out=None,
              workspace: torch.Tensor | None = None, v_mean: torch.Tensor | None = None):
    """V preparation: returns (v_t, v_scale); see sage_prepare_v for the storage order.  v_mean
    (fp32 [B, H, d], FP16 PV only): smooth_v -- the channel means are written there and
    subtracted; pass the same tensor to attn_fwd_prepared."""
    L = load_library()
    dv = _desc(v, tensor_layout)
    vt, vs = alloc_prepared_v(dv.B, dv.H, dv.N, dv.d, pv_dtype, v.device) if out is None else out
    if workspace is None:
        workspace = prepare_v_workspace(dv.B, dv.H, dv.N, dv.d, pv_dtype, v.device)
    _check(L.sage_prepare_v(ctypes.byref(dv), PV_CODES[pv_dtype], vt.data_ptr(), None if vs is None else vs.data_ptr(),
                            None if v_mean is None else v_mean.data_ptr(), workspace.data_ptr(), workspace.numel(),
                            _stream(v)), "sage_prepare_v")
    return vt, vs


def mask_workspace(B, Nq, Nk, mask_h, device) -> torch.Tensor:
    n = int(load_library().sage_mask_workspace_bytes(B, Nq, Nk, mask_h))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def attn_fwd_prepared(qk: QuantizedQK, v_t: torch.Tensor, v_scale: torch.Tensor | None, *, pv_dtype: str = "fp16",
                      tensor_layout: str = "HND", is_causal: bool = False, attn_mask: torch.Tensor | None = None,
                      sm_scale: float | None = None, return_lse: bool = False, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      v_mean: torch.Tensor | None = None):
    """Attention on pre-quantized Q/K and prepared V (from prepare_v; v_mean as given to it for
    smooth_v).  Returns out or (out, lse); out defaults to the dtype Q and K had."""
    L = load_library()
    B, H, Nq, Nk, d = qk.B, qk.H, qk.Nq, qk.Nk, qk.d
    dev = qk.q8.device
    if out is None:
        shape = (B, H, Nq, d) if tensor_layout == "HND" else (B, Nq, H, d)
        out = torch.empty(shape, dtype=qk.dtype, device=dev)
    if tensor_layout == "HND":
        osb, osh, osn = out.stride(0), out.stride(1), out.stride(2)
    else:
        osb, osh, osn = out.stride(0), out.stride(2), out.stride(1)
    if return_lse and lse is None:
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=dev)
    m, mcode, mh, msb, msh, msq = _mask_args(attn_mask, B, H, Nq, Nk)
    if workspace is None and mh > 0:
        workspace = mask_workspace(B, Nq, Nk, mh, dev)
    qs = qk.cstruct()
    odt = _dtype_code(out.dtype, "out", allow_f32=True)
    _check(L.sage_attn_fwd_prepared(ctypes.byref(qs), v_t.data_ptr(), None if v_scale is None else v_scale.data_ptr(),
                                    None if v_mean is None else v_mean.data_ptr(), PV_CODES[pv_dtype], None if m is None else m.data_ptr(), mcode, mh, msb, msh, msq,
                                    1 if is_causal else 0, sm_scale_arg(sm_scale),
                                    out.data_ptr(), odt, osb, osh, osn, None if lse is None else lse.data_ptr(),
                                    None if workspace is None else workspace.data_ptr(),
                                    0 if workspace is None else workspace.numel(), _stream(out)),
           "sage_attn_fwd_prepared")
    return (out, lse) if return_lse else out


def default_sm_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def sclk_probe(device=None, nblocks: int = 1024, iters: int = 20000, load: bool = True, stream=None,
               out: torch.Tensor | None = None):
    """The shader clock (sage_sclk_probe).  load=True: under the probe's own MFMA + VALU load, run
    now and read back: returns median, min and max MHz over its workgroups and how long it ran.
    load=False: the idle form is only enqueued on `stream` (a torch.cuda.Stream) into `out`
    (int64 [4 * nblocks]); read it later with sclk_result(out)."""
    L = load_library()
    dev = torch.device("cuda") if device is None else torch.device(device)
    if out is None:
        out = torch.zeros(4 * nblocks, dtype=torch.int64, device=dev)
    st = _stream(out) if stream is None else stream.cuda_stream
    _check(L.sage_sclk_probe(nblocks, iters, 1 if load else 0, out.data_ptr(), st), "sage_sclk_probe")
    return sclk_result(out) if load else out


def sclk_result(out: torch.Tensor) -> dict:
    """MHz per workgroup from sage_sclk_probe's counters: median, min, max, and the window length."""
    c = out.view(-1, 4).cpu().numpy().astype("float64")
    dt, dr = c[:, 2] - c[:, 0], c[:, 3] - c[:, 1]
    ok = dr > 0
    mhz = sorted((100.0 * dt[ok] / dr[ok]).tolist())
    if not mhz:
        raise RuntimeError("sage_sclk_probe: no workgroup reported a duration")
    return {"median_mhz": round(mhz[len(mhz) // 2], 1), "min_mhz": round(mhz[0], 1), "max_mhz": round(mhz[-1], 1),
            "probe_ms": round(float(dr[ok].max()) / 1e5, 3), "workgroups": len(mhz)}


def merge_lse(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None, out_dtype: torch.dtype | None = None, return_lse: bool = True):
    """Merge S partial attention results over disjoint key sets (e.g. key slices of one sequence).

    o_parts: [S, B, H, Nq, d] (bf16, fp16 or fp32; contiguous), lse_parts: fp32 [S, B, H, Nq] as
    returned with return_lse=True.  Returns out [B, H, Nq, d] (out_dtype, default that of the
    parts) or (out, lse)."""
    L = load_library()
    if o_parts.dim() != 5 or lse_parts.shape != o_parts.shape[:4]:
        raise ValueError("o_parts must be [S,B,H,Nq,d] and lse_parts [S,B,H,Nq]")
    if lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be float32")
    o_parts, lse_parts = o_parts.contiguous(), lse_parts.contiguous()
    S, B, H, Nq, d = o_parts.shape
    pdt = _dtype_code(o_parts.dtype, "o_parts", allow_f32=True)
    if out is None:
        out = torch.empty(B, H, Nq, d, dtype=out_dtype or o_parts.dtype, device=o_parts.device)
    odt = _dtype_code(out.dtype, "out", allow_f32=True)
    if return_lse and lse is None:
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=o_parts.device)
    _check(L.sage_merge_lse(S, B, H, Nq, d, o_parts.data_ptr(), pdt, lse_parts.data_ptr(), out.data_ptr(), odt,
                            out.stride(0), out.stride(1), out.stride(2), None if lse is None else lse.data_ptr(),
                            _stream(o_parts)), "sage_merge_lse")
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------------------------------------
# packed variable-length batches
# ---------------------------------------------------------------------------------------------
def _packed_desc(t: torch.Tensor, nseq: int, max_seqlen: int) -> QKVDesc:
    """A packed [total, H, d] tensor as the descriptor of nseq sequences of at most max_seqlen rows."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("packed q/k/v must be [total, H, d] with a contiguous head_dim")
    return QKVDesc(t.data_ptr(), _dtype_code(t.dtype, "q/k/v"), nseq, t.shape[1], max_seqlen, t.shape[2], 0,
                   t.stride(1), t.stride(0))


def _cu(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_cuda:
        raise ValueError(f"{what} must be a 1-D int32 device tensor")
    return t.contiguous()


def quantize_qk_varlen(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                       max_seqlen_q: int, max_seqlen_k: int, out: QuantizedQK | None = None,
                       workspace: torch.Tensor | None = None, per_block_mean: bool = False) -> QuantizedQK:
    """Per-sequence K mean and INT8 quantization of packed q [total_q, H, d] and k [total_k, Hkv, d]
    into the dense padded layout of len(cu_seqlens) - 1 sequences of max_seqlen tokens."""
    L = load_library()
    cq, ck = _cu(cu_seqlens_q, "cu_seqlens_q"), _cu(cu_seqlens_k, "cu_seqlens_k")
    nseq = cq.numel() - 1
    if ck.numel() != nseq + 1 or nseq < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold nseq + 1 >= 2 entries")
    dq, dk = _packed_desc(q, nseq, max_seqlen_q), _packed_desc(k, nseq, max_seqlen_k)
    if out is None:
        out = alloc_quantized(nseq, dq.H, max_seqlen_q, max_seqlen_k, dq.d, q.device, Hkv=dk.H, dtype=q.dtype,
                              per_block_mean=per_block_mean)
    out.dtype = q.dtype
    ws = quantize_workspace(nseq, dk.H, max_seqlen_k, dk.d, q.device) if workspace is None else workspace
    qs = out.cstruct()
    _check(L.sage_quantize_qk_varlen(ctypes.byref(dq), ctypes.byref(dk), cq.data_ptr(), ck.data_ptr(), q.shape[0],
                                     k.shape[0], ctypes.byref(qs), ws.data_ptr(), ws.numel(), _stream(q)),
           "sage_quantize_qk_varlen")
    return out


def sageattn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, is_causal: bool = False,
                    sm_scale: float | None = None, smooth_k: bool = True, return_lse: bool = False,
                    pv_dtype: str = "fp16", smooth_v: bool = False, per_block_mean: bool = False):
    """Quantized attention of packed variable-length sequences (the docs digest's ``sageattn_varlen``).

    q: [total_q, H, d], k and v: [total_k, Hkv, d] (bf16 or fp16, one dtype); cu_seqlens_*: int32
    device tensors of nseq + 1 cumulative lengths starting at 0; max_seqlen_*: the longest
    sequence.  Each sequence is its own attention problem (own K mean; causal aligned at its first
    query and key).  Returns out [total_q, H, d] (q's dtype) or (out, lse) with lse fp32
    [H, total_q]."""
    if not smooth_k:
        raise ValueError("this library always smooths K (smooth_k=True)")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must have the same dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"the {k.shape[1]} key/value heads do not divide the {q.shape[1]} query heads")
    L = load_library()
    qk = quantize_qk_varlen(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                            per_block_mean=per_block_mean)
    cq, ck = _cu(cu_seqlens_q, "cu_seqlens_q"), _cu(cu_seqlens_k, "cu_seqlens_k")
    dv = _packed_desc(v, qk.B, max_seqlen_k)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device) if return_lse else None
    ws = fwd_workspace(qk.B, qk.Hkv, max_seqlen_q, max_seqlen_k, qk.d, pv_dtype, 0, q.device)
    qs = qk.cstruct()
    _check(L.sage_attn_fwd_varlen(ctypes.byref(qs), ctypes.byref(dv), cq.data_ptr(), ck.data_ptr(), q.shape[0],
                                  k.shape[0], 1 if is_causal else 0, sm_scale_arg(sm_scale),
                                  PV_CODES[pv_dtype], 1 if smooth_v else 0, out.data_ptr(), _dtype_code(out.dtype, "out"), out.stride(1),
                                  out.stride(0), None if lse is None else lse.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream(q)), "sage_attn_fwd_varlen")
    return (out, lse) if return_lse else out


def prepare_v_varlen(v: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_k: int, pv_dtype: str = "fp16",
                     out=None, workspace: torch.Tensor | None = None, v_mean: torch.Tensor | None = None):
    """V preparation of a packed [total_k, Hkv, d] V into the dense padded layout: (v_t, v_scale)."""
    L = load_library()
    ck = _cu(cu_seqlens_k, "cu_seqlens_k")
    nseq = ck.numel() - 1
    dv = _packed_desc(v, nseq, max_seqlen_k)
    vt, vs = alloc_prepared_v(nseq, dv.H, max_seqlen_k, dv.d, pv_dtype, v.device) if out is None else out
    if workspace is None:
        workspace = prepare_v_workspace(nseq, dv.H, max_seqlen_k, dv.d, pv_dtype, v.device)
    _check(L.sage_prepare_v_varlen(ctypes.byref(dv), ck.data_ptr(), v.shape[0], PV_CODES[pv_dtype], vt.data_ptr(),
                                   None if vs is None else vs.data_ptr(),
                                   None if v_mean is None else v_mean.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream(v)), "sage_prepare_v_varlen")
    return vt, vs


def attn_fwd_prepared_varlen(qk: QuantizedQK, v_t: torch.Tensor, v_scale: torch.Tensor | None,
                             cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, total_q: int, total_k: int, *,
                             pv_dtype: str = "fp16", is_causal: bool = False, sm_scale: float | None = None,
                             return_lse: bool = False, out: torch.Tensor | None = None,
                             lse: torch.Tensor | None = None, v_mean: torch.Tensor | None = None):
    """Attention of a packed variable-length batch on pre-quantized Q/K and prepared V.  Returns out
    [total_q, H, d] or (out, lse [H, total_q])."""
    L = load_library()
    cq, ck = _cu(cu_seqlens_q, "cu_seqlens_q"), _cu(cu_seqlens_k, "cu_seqlens_k")
    dev = qk.q8.device
    if out is None:
        out = torch.empty(total_q, qk.H, qk.d, dtype=qk.dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty(qk.H, total_q, dtype=torch.float32, device=dev)
    qs = qk.cstruct()
    _check(L.sage_attn_fwd_prepared_varlen(ctypes.byref(qs), v_t.data_ptr(),
                                           None if v_scale is None else v_scale.data_ptr(),
                                           None if v_mean is None else v_mean.data_ptr(), PV_CODES[pv_dtype],
                                           cq.data_ptr(), ck.data_ptr(), total_q, total_k, 1 if is_causal else 0,
                                           sm_scale_arg(sm_scale), out.data_ptr(),
                                           _dtype_code(out.dtype, "out", allow_f32=True), out.stride(1),
                                           out.stride(0), None if lse is None else lse.data_ptr(), _stream(out)),
           "sage_attn_fwd_prepared_varlen")
    return (out, lse) if return_lse else out
