"""CPU oracle for SageAttention-style quantized attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product path (``quantized_attention_quantize_amd``) never imports it and shares
no code with it.  Arithmetic lives in ``sage_oracle.c`` (plain C loops, fp64 where the method's
definition calls for it); this module only compiles that file with gcc and marshals numpy arrays
through ctypes.

Entry points (all inputs are host numpy arrays; bf16 and fp16 tensors travel as their uint16 bit
patterns, with ``dtype="bf16"`` or ``"fp16"`` saying which; masks are uint8/bool, nonzero = attend,
or float32, added to the scaled scores):

* codecs: ``f32_to_f16``, ``f16_to_f32``, ``f32_to_bf16``, ``f32_to_e4m3``, ``e4m3_to_f32``
* ``kmean(K)``                      -- per-(b,h,channel) token mean of K, fp64 sum -> fp32
* ``quant_qk(Q, K, kmean, ...)``    -- per-64-token-block INT8 Q and smoothed K, scales, LSE shift
* ``prep_v(V, pv)``                 -- fp16 V or per-channel e4m3 V with its scales
* ``scores(q8, k8, ...)``           -- exact int32 Q8 . K8^T window of one head
* ``attn_qe(...)``                  -- the quantized emulation (online softmax over BN-key tiles)
* ``attn_ex(...)``                  -- fp64 exact attention on the unquantized inputs
* ``run_qe(...)``                   -- convenience: all the steps above for given rows
* ``merge_lse(o_parts, lse_parts)`` -- partial results over disjoint key sets -> the result over their union
* ``run_qe_varlen`` / ``attn_ex_varlen`` -- packed variable-length batches, one sequence at a time
* FP4 microscaling method (``sage_fp4_oracle.c``): ``f32_to_e2m1``, ``e2m1_to_f32``, ``mx_exp``,
  ``fp4_quant_qk``, ``fp4_prep_v``, ``fp4_scores``, ``fp4_attn_qe``, ``run_fp4``
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_SRC_FP4 = os.path.join(_HERE, "sage_fp4_oracle.c")
_LIB = os.path.join(_HERE, "libsage_oracle.so")
QBLK = 64

_lib = None


def build(force: bool = True) -> str:
    """Compile sage_oracle.c into libsage_oracle.so with gcc (OpenMP, no fast-math, no FP contraction)."""
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_FP4))):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-o", tmp, _SRC, _SRC_FP4, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """The same sources built with AddressSanitizer and UndefinedBehaviorSanitizer (any finding
    aborts), without OpenMP, into ``out``.  A process loads it through SAGE_ORACLE_LIB with gcc's
    libasan preloaded."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall",
           "-Wno-unknown-pragmas", "-o", out, _SRC, _SRC_FP4, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("SAGE_ORACLE_LIB")
        if not path:
            path = build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        i32 = ctypes.c_int
        f32 = ctypes.c_float
        f64 = ctypes.c_double
        L.orc_num_threads.restype = i32
        for name in ("orc_f32_to_f16_n", "orc_f16_to_f32_n", "orc_f32_to_bf16_n", "orc_f32_to_e4m3_n",
                     "orc_e4m3_to_f32_n"):
            getattr(L, name).argtypes = [P, P, I]
            getattr(L, name).restype = None
        L.orc_kmean.argtypes = [P, i32, I, I, I, I, P]
        L.orc_block_mean.argtypes = [P, i32, I, I, I, I, P]
        L.orc_quant_qk.argtypes = [P, P, i32, P, i32, I, I, I, I, I, I, I, I, P, P, P, P, P, P]
        L.orc_prep_v_fp16.argtypes = [P, i32, I, I, I, I, P, P]
        L.orc_prep_v_fp8.argtypes = [P, i32, I, I, I, I, P, P]
        L.orc_scores.argtypes = [P, P, I, I, I, I, I, P]
        L.orc_attn_qe.argtypes = [P, P, P, P, P, P, P, P, P, i32, P, i32, I, i32, f32, I, I, I, I, I, I, I, I, I, f64, i32,
                                  P, I, P, i32, P, P]
        L.orc_attn_ex.argtypes = [P, P, P, i32, P, i32, I, i32, f64, I, I, I, I, I, I, P, I, P, P]
        L.orc_merge_lse.argtypes = [P, P, I, I, I, P, P]
        # FP4 microscaling method (sage_fp4_oracle.c)
        for name in ("orc_f32_to_e2m1_n", "orc_e2m1_to_f32_n", "orc_mx_exp_n"):
            getattr(L, name).argtypes = [P, P, I]
        L.orc_fp4_quant_qk.argtypes = [P, P, i32, i32, I, I, I, I, I, I, P, P, P, P, P, P, P, P]
        L.orc_fp4_prep_v.argtypes = [P, i32, I, I, I, I, P, P]
        L.orc_fp4_scores.argtypes = [P, P, P, P, P, i32, I, I, I, I, I, I, I, I, I, I, I, P]
        L.orc_fp4_attn_qe.argtypes = [P, P, P, P, P, i32, P, P, P, i32, f32, I, I, I, I, I, I, I, f64, P, I, P, i32, P,
                                      P]
        for name in ("orc_kmean", "orc_block_mean", "orc_quant_qk", "orc_prep_v_fp16", "orc_prep_v_fp8", "orc_scores",
                     "orc_attn_qe", "orc_attn_ex", "orc_merge_lse", "orc_f32_to_e2m1_n", "orc_e2m1_to_f32_n",
                     "orc_mx_exp_n", "orc_fp4_quant_qk", "orc_fp4_prep_v", "orc_fp4_scores", "orc_fp4_attn_qe"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------------------------
def f32_to_f16(x):
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_p(x), _p(y), x.size)
    return y


def f16_to_f32(x):
    x = _c(x, np.uint16)
    y = np.empty(x.shape, np.float32)
    lib().orc_f16_to_f32_n(_p(x), _p(y), x.size)
    return y


def f32_to_bf16(x):
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_p(x), _p(y), x.size)
    return y


def bf16_to_f32(x):
    """bf16 bits -> fp32: the bf16 pattern is the upper half of the binary32 pattern."""
    x = _c(x, np.uint16)
    return (x.astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3(x):
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint8)
    lib().orc_f32_to_e4m3_n(_p(x), _p(y), x.size)
    return y


def e4m3_to_f32(x):
    x = _c(x, np.uint8)
    y = np.empty(x.shape, np.float32)
    lib().orc_e4m3_to_f32_n(_p(x), _p(y), x.size)
    return y


# ---------------------------------------------------------------------------------------------
# the method's steps
# ---------------------------------------------------------------------------------------------
def pad_n(n: int) -> int:
    """Padded token extent used for the int8 / prepared-V buffers: a multiple of 128."""
    return (n + 127) // 128 * 128


def _in_fp16(dtype: str) -> int:
    if dtype not in ("bf16", "fp16"):
        raise ValueError(dtype)
    return 1 if dtype == "fp16" else 0


def kmean(K, dtype="bf16"):
    """K: uint16 bf16 or fp16 bits [B,H,Nk,d] -> fp32 [B,H,d]."""
    K = _c(K, np.uint16)
    B, H, Nk, d = K.shape
    out = np.empty((B, H, d), np.float32)
    lib().orc_kmean(_p(K), _in_fp16(dtype), B, H, Nk, d, _p(out))
    return out


def block_mean(K, dtype="bf16"):
    """K: [B,H,Nk,d] bits -> per-64-token-block means fp32 [B,H,ceil(Nk/64),d] (per_block_mean)."""
    K = _c(K, np.uint16)
    B, H, Nk, d = K.shape
    out = np.empty((B, H, (Nk + QBLK - 1) // QBLK, d), np.float32)
    lib().orc_block_mean(_p(K), _in_fp16(dtype), B, H, Nk, d, _p(out))
    return out


@dataclass
class QuantQK:
    q8: np.ndarray  # int8 [B,H,Nq_pad,d]
    k8: np.ndarray  # int8 [B,Hkv,Nk_pad,d]
    qs: np.ndarray  # fp32 [B,H,ceil(Nq/64)]
    ks: np.ndarray  # fp32 [B,Hkv,ceil(Nk/64)]
    kmean: np.ndarray  # fp32 [B,Hkv,d], or the block means [B,Hkv,ceil(Nk/64),d] with per_block_mean
    corr: np.ndarray  # fp32 [B,H,Nq] (0 with per_block_mean)
    corr_blk: np.ndarray | None = None  # per_block_mean: fp32 [B,H,ceil(Nk/64),Nq]


def quant_qk(Q, K, km=None, Nq_pad=None, Nk_pad=None, dtype="bf16", per_block_mean=False) -> QuantQK:
    """Q [B,H,Nq,d], K [B,Hkv,Nk,d] (Hkv divides H; query head h reads key head h // (H // Hkv)),
    both of ``dtype``.  per_block_mean: K is smoothed by its 64-token block's mean and the
    per-block score terms come out in corr_blk."""
    Q = _c(Q, np.uint16)
    K = _c(K, np.uint16)
    B, H, Nq, d = Q.shape
    Hkv, Nk = K.shape[1], K.shape[2]
    assert K.shape[0] == B and K.shape[3] == d and H % Hkv == 0
    if km is None:
        km = block_mean(K, dtype) if per_block_mean else kmean(K, dtype)
    km = _c(km, np.float32)
    Nq_pad = pad_n(Nq) if Nq_pad is None else Nq_pad
    Nk_pad = pad_n(Nk) if Nk_pad is None else Nk_pad
    q8 = np.empty((B, H, Nq_pad, d), np.int8)
    k8 = np.empty((B, Hkv, Nk_pad, d), np.int8)
    qs = np.empty((B, H, (Nq + QBLK - 1) // QBLK), np.float32)
    ks = np.empty((B, Hkv, (Nk + QBLK - 1) // QBLK), np.float32)
    corr = np.empty((B, H, Nq), np.float32)
    cb = np.empty((B, H, (Nk + QBLK - 1) // QBLK, Nq), np.float32) if per_block_mean else None
    lib().orc_quant_qk(_p(Q), _p(K), _in_fp16(dtype), _p(km), 1 if per_block_mean else 0, B, H, Hkv, Nq, Nk, d, Nq_pad,
                       Nk_pad, _p(q8), _p(k8), _p(qs), _p(ks), _p(corr), _p(cb))
    return QuantQK(q8, k8, qs, ks, km, corr, cb)


def prep_v(V, pv: str = "fp16", dtype="bf16", vmean=None):
    """V of ``dtype``.  Returns (vhat, vs): fp16 bits uint16 [B,H,Nk,d] and None, or e4m3 uint8
    [B,H,Nk,d] and fp32 [B,H,d].  vmean (fp32 [B,H,d], FP16 PV only): smooth_v, V - vmean is
    prepared instead of V."""
    V = _c(V, np.uint16)
    B, H, Nk, d = V.shape
    if pv == "fp16":
        out = np.empty(V.shape, np.uint16)
        vm = None if vmean is None else _c(vmean, np.float32)
        lib().orc_prep_v_fp16(_p(V), _in_fp16(dtype), B, H, Nk, d, _p(vm), _p(out))
        return out, None
    if vmean is not None:
        raise ValueError("smooth_v is defined for FP16 PV only")
    if pv == "fp8":
        out = np.empty(V.shape, np.uint8)
        vs = np.empty((B, H, d), np.float32)
        lib().orc_prep_v_fp8(_p(V), _in_fp16(dtype), B, H, Nk, d, _p(out), _p(vs))
        return out, vs
    raise ValueError(pv)


def scores(q8, k8, b, h, row0, nrows, col0, ncols):
    """Exact int32 scores for rows [row0,row0+nrows) x keys [col0,col0+ncols) of head (b,h)."""
    d = q8.shape[3]
    qh = np.ascontiguousarray(q8[b, h])
    kh = np.ascontiguousarray(k8[b, h])
    assert row0 + nrows <= qh.shape[0] and col0 + ncols <= kh.shape[0]
    out = np.empty((nrows, ncols), np.int32)
    lib().orc_scores(_p(qh), _p(kh), d, row0, nrows, col0, ncols, _p(out))
    return out


def default_sm_scale(d: int) -> float:
    """sm_scale default 1/sqrt(head_dim), rounded to fp32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _mask_arg(mask, B, H, Nq, Nk):
    """(array, mask_h, is_f32): a floating mask is additive (float32), anything else boolean (uint8)."""
    if mask is None:
        return None, 0, 0
    f32 = np.issubdtype(np.asarray(mask).dtype, np.floating)
    m = np.ascontiguousarray(mask, dtype=np.float32 if f32 else np.uint8)
    assert m.ndim == 4 and m.shape[0] == B and m.shape[2] == Nq and m.shape[3] == Nk and m.shape[1] in (1, H)
    return m, m.shape[1], int(f32)


def attn_qe(qk: QuantQK, vhat, vs, pv, Nq, Nk, *, causal=False, mask=None, sm_scale=None, BN=64, tau=0.0,
            lsum_rounded=False, rows=None, out_dtype="bf16", vmean=None):
    """Quantized emulation.  Returns (o32 [R,d] fp32, o16 [R,d] bits of out_dtype, lse [R] fp32).

    BN: keys per online-softmax tile; tau: the reference maximum is raised only when a tile's
    maximum exceeds it by more than tau (log2 units); 0 = exact running maximum.  For pv = "fp8"
    tau is a whole number and P = e4m3(448 * 2^-tau * p).
    lsum_rounded: the denominator sums P as rounded for the PV product instead of the fp32 p.
    vmean: smooth_v's V mean [B,Hkv,d] (vhat then holds V - vmean), added back to the output."""
    if pv == "fp8" and (int(tau) != tau or tau < 0):
        raise ValueError("with e4m3 P, tau must be a non-negative whole number")
    B, H, Nq_pad, d = qk.q8.shape
    Hkv, Nk_pad = qk.k8.shape[1], qk.k8.shape[2]
    sm = default_sm_scale(d) if sm_scale is None else float(np.float32(sm_scale))
    m, mh, mf = _mask_arg(mask, B, H, Nq, Nk)
    if rows is None:
        R = B * H * Nq
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R = rows.size
        rp = rows
    o32 = np.empty((R, d), np.float32)
    o16 = np.empty((R, d), np.uint16)
    lse = np.empty((R,), np.float32)
    vm = None if vmean is None else _c(vmean, np.float32)
    lib().orc_attn_qe(_p(qk.q8), _p(qk.k8), _p(qk.qs), _p(qk.ks), _p(qk.corr), _p(qk.corr_blk),
                      _p(np.ascontiguousarray(vhat)),
                      _p(vs), _p(vm), 1 if pv == "fp8" else 0, _p(m), mf, mh, 1 if causal else 0, sm, B, H, Hkv, Nq, Nk, d,
                      Nq_pad, Nk_pad, BN, float(tau), 1 if lsum_rounded else 0, _p(rp), R, _p(o32),
                      _in_fp16(out_dtype), _p(o16), _p(lse))
    return o32, o16, lse


def attn_ex(Q, K, V, *, causal=False, mask=None, sm_scale=None, rows=None, dtype="bf16"):
    """fp64 exact attention on the inputs (bits of ``dtype``).  Returns (out [R,d] fp64, lse [R] fp64)."""
    Q = _c(Q, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    B, H, Nq, d = Q.shape
    Hkv, Nk = K.shape[1], K.shape[2]
    assert H % Hkv == 0 and V.shape[1] == Hkv
    sm = default_sm_scale(d) if sm_scale is None else float(np.float32(sm_scale))
    m, mh, mf = _mask_arg(mask, B, H, Nq, Nk)
    if rows is None:
        R = B * H * Nq
        rp = None
    else:
        rp = np.ascontiguousarray(rows, dtype=np.int64)
        R = rp.size
    out = np.empty((R, d), np.float64)
    lse = np.empty((R,), np.float64)
    lib().orc_attn_ex(_p(Q), _p(K), _p(V), _in_fp16(dtype), _p(m), mf, mh, 1 if causal else 0, sm, B, H, Hkv, Nq, Nk, d, _p(rp), R,
                      _p(out), _p(lse))
    return out, lse


@dataclass
class QEResult:
    qk: QuantQK
    vhat: np.ndarray
    vs: np.ndarray | None
    o32: np.ndarray
    o16: np.ndarray  # output bits (bf16 or fp16)
    lse: np.ndarray


def run_qe(Q, K, V, *, pv="fp16", causal=False, mask=None, sm_scale=None, BN=64, tau=0.0, lsum_rounded=False,
           rows=None, dtype="bf16", out_dtype=None, smooth_v=False, per_block_mean=False) -> QEResult:
    """All quantized-emulation steps: kmean -> quant_qk -> prep_v -> attn_qe.  The output dtype
    defaults to the input dtype.  smooth_v: V's token mean (taken as K's) is subtracted before the
    FP16 rounding of V and added back to the output."""
    qk = quant_qk(Q, K, dtype=dtype, per_block_mean=per_block_mean)
    vmean = kmean(V, dtype) if smooth_v else None
    vhat, vs = prep_v(V, pv, dtype=dtype, vmean=vmean)
    Nq, Nk = Q.shape[2], K.shape[2]
    o32, o16, lse = attn_qe(qk, vhat, vs, pv, Nq, Nk, causal=causal, mask=mask, sm_scale=sm_scale, BN=BN, tau=tau,
                            lsum_rounded=lsum_rounded, rows=rows, out_dtype=out_dtype or dtype, vmean=vmean)
    return QEResult(qk, vhat, vs, o32, o16, lse)


def merge_lse(o_parts, lse_parts):
    """Merge S partial attention results over disjoint key sets.

    o_parts: [S, R, d] (any float dtype; taken as fp32), lse_parts: [S, R] natural-log LSEs.
    Returns (out [R, d] fp64, lse [R] fp64)."""
    o = _c(o_parts, np.float32)
    lp = _c(lse_parts, np.float32)
    S, R, d = o.shape
    assert lp.shape == (S, R)
    out = np.empty((R, d), np.float64)
    lse = np.empty((R,), np.float64)
    lib().orc_merge_lse(_p(o), _p(lp), S, R, d, _p(out), _p(lse))
    return out, lse


# ---------------------------------------------------------------------------------------------
# variable-length batches (packed sequences with cumulative lengths)
# ---------------------------------------------------------------------------------------------
def _seq_heads(X, lo, hi):
    """Rows [lo, hi) of a packed [total, H, d] array as one-sequence HND [1, H, n, d]."""
    return np.ascontiguousarray(np.transpose(X[lo:hi], (1, 0, 2))[None])


def run_qe_varlen(Q, K, V, cu_q, cu_k, *, pv="fp16", causal=False, sm_scale=None, BN=64, tau=0.0,
                  lsum_rounded=False, dtype="bf16", out_dtype=None, smooth_v=False, per_block_mean=False):
    """Quantized emulation of packed variable-length batches (the docs digest's ``sageattn_varlen``).

    Q: [total_q, H, d], K and V: [total_k, Hkv, d] (bits of ``dtype``); sequence b holds query rows
    [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]).  Reading: each sequence is its own
    attention problem, so the whole method (K mean, 64-token blocks, online softmax, causal mask
    aligned at the sequence's first query and key) runs on each sequence alone.
    Returns (o32 [total_q, H, d] fp32, o16 [total_q, H, d] bits, lse [H, total_q] fp32)."""
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    Tq, H, d = Q.shape
    o32 = np.zeros((Tq, H, d), np.float32)
    o16 = np.zeros((Tq, H, d), np.uint16)
    lse = np.full((H, Tq), -np.inf, np.float32)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0:
            continue
        if k1 == k0:  # no keys: every row sees nothing
            continue
        r = run_qe(_seq_heads(Q, q0, q1), _seq_heads(K, k0, k1), _seq_heads(V, k0, k1), pv=pv, causal=causal,
                   sm_scale=sm_scale, BN=BN, tau=tau, lsum_rounded=lsum_rounded, dtype=dtype, out_dtype=out_dtype,
                   smooth_v=smooth_v, per_block_mean=per_block_mean)
        n = q1 - q0
        o32[q0:q1] = r.o32.reshape(H, n, d).transpose(1, 0, 2)
        o16[q0:q1] = r.o16.reshape(H, n, d).transpose(1, 0, 2)
        lse[:, q0:q1] = r.lse.reshape(H, n)
    return o32, o16, lse


def attn_ex_varlen(Q, K, V, cu_q, cu_k, *, causal=False, sm_scale=None, dtype="bf16"):
    """fp64 exact attention of packed variable-length batches, one sequence at a time.
    Returns (out [total_q, H, d] fp64, lse [H, total_q] fp64)."""
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    Tq, H, d = Q.shape
    out = np.zeros((Tq, H, d), np.float64)
    lse = np.full((H, Tq), -np.inf, np.float64)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        o, l = attn_ex(_seq_heads(Q, q0, q1), _seq_heads(K, k0, k1), _seq_heads(V, k0, k1), causal=causal,
                       sm_scale=sm_scale, dtype=dtype)
        n = q1 - q0
        out[q0:q1] = o.reshape(H, n, d).transpose(1, 0, 2)
        lse[:, q0:q1] = l.reshape(H, n)
    return out, lse


# ---------------------------------------------------------------------------------------------
# FP4 microscaling method (sage_fp4_oracle.c): MX FP4 Q, K (per 32 channels) and V (per 32 tokens),
# Q smoothed by its 128-token block means (or global mean) with the FP32 correction rows, e4m3 P
# ---------------------------------------------------------------------------------------------
MX = 32
QMBLK = 128


def f32_to_e2m1(x):
    """fp32 -> e2m1 codes (sign in bit 3), nearest with ties to the even code, saturating at 6."""
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint8)
    lib().orc_f32_to_e2m1_n(_p(x), _p(y), x.size)
    return y


def e2m1_to_f32(x):
    x = _c(x, np.uint8)
    y = np.empty(x.shape, np.float32)
    lib().orc_e2m1_to_f32_n(_p(x), _p(y), x.size)
    return y


def mx_exp(amax):
    """Shared exponent X of MX blocks with the given largest magnitudes (E8M0 byte = X + 127)."""
    a = _c(amax, np.float32)
    y = np.empty(a.shape, np.int32)
    lib().orc_mx_exp_n(_p(a), _p(y), a.size)
    return y


def mx_dequant(codes, e8, axis):
    """Dequantized values of MX codes whose E8M0 bytes cover 32 consecutive elements along axis."""
    v = e2m1_to_f32(codes).astype(np.float64)
    sc = np.ldexp(1.0, e8.astype(np.int64) - 127)
    sc = np.repeat(sc, MX, axis=axis)
    sl = [slice(None)] * v.ndim
    sl[axis] = slice(0, v.shape[axis])
    return v * sc[tuple(sl)]


@dataclass
class FP4QK:
    kmean: np.ndarray     # [B,Hkv,d]
    qmean: np.ndarray     # [B,H,nqm,d]
    q4: np.ndarray        # [B,H,Nq,d] e2m1 codes
    qe: np.ndarray        # [B,H,Nq,d/32] E8M0
    k4: np.ndarray        # [B,Hkv,Nk,d]
    ke: np.ndarray        # [B,Hkv,Nk,d/32]
    qk_corr: np.ndarray   # [B,H,nqm,Nk]
    lse_corr: np.ndarray  # [B,H,Nq]
    per_block: bool


def fp4_quant_qk(Q, K, dtype="bf16", per_block_mean=True) -> FP4QK:
    Q = _c(Q, np.uint16)
    K = _c(K, np.uint16)
    B, H, Nq, d = Q.shape
    Hkv, Nk = K.shape[1], K.shape[2]
    if d % MX or H % Hkv:
        raise ValueError("d must be a multiple of 32 and Hkv must divide H")
    nqm = (Nq + QMBLK - 1) // QMBLK if per_block_mean else 1
    km = kmean(K, dtype)
    qm = np.empty((B, H, nqm, d), np.float32)
    q4 = np.empty((B, H, Nq, d), np.uint8)
    qe = np.empty((B, H, Nq, d // MX), np.uint8)
    k4 = np.empty((B, Hkv, Nk, d), np.uint8)
    ke = np.empty((B, Hkv, Nk, d // MX), np.uint8)
    corr = np.empty((B, H, nqm, Nk), np.float32)
    lc = np.empty((B, H, Nq), np.float32)
    lib().orc_fp4_quant_qk(_p(Q), _p(K), _in_fp16(dtype), 1 if per_block_mean else 0, B, H, Hkv, Nq, Nk, d, _p(km),
                           _p(qm), _p(q4), _p(qe), _p(k4), _p(ke), _p(corr), _p(lc))
    return FP4QK(km, qm, q4, qe, k4, ke, corr, lc, bool(per_block_mean))


def fp4_prep_v(V, dtype="bf16"):
    """V [B,Hkv,Nk,d] bits -> (v4 [B,Hkv,Nk,d] codes, ve [B,Hkv,ceil(Nk/32),d] E8M0)."""
    V = _c(V, np.uint16)
    B, Hkv, Nk, d = V.shape
    v4 = np.empty((B, Hkv, Nk, d), np.uint8)
    ve = np.empty((B, Hkv, (Nk + MX - 1) // MX, d), np.uint8)
    lib().orc_fp4_prep_v(_p(V), _in_fp16(dtype), B, Hkv, Nk, d, _p(v4), _p(ve))
    return v4, ve


def fp4_scores(qk: FP4QK, b, h, row0, nrows, col0, ncols):
    """Raw scores (before sm_scale) of a window of head (b, h): fp32 [nrows, ncols]."""
    B, H, Nq, d = qk.q4.shape
    Hkv, Nk = qk.k4.shape[1], qk.k4.shape[2]
    out = np.empty((nrows, ncols), np.float32)
    lib().orc_fp4_scores(_p(qk.q4), _p(qk.qe), _p(qk.k4), _p(qk.ke), _p(qk.qk_corr), 1 if qk.per_block else 0, H, Hkv,
                         Nq, Nk, d, b, h, row0, nrows, col0, ncols, _p(out))
    return out


def fp4_attn_qe(qk: FP4QK, v4, ve, *, causal=False, sm_scale=None, BN=64, tau=0, rows=None, out_dtype="bf16"):
    """Returns (o32 [R,d] fp32, o16 [R,d] output bits, lse [R] fp32) for the requested flattened rows.
    tau: whole log2 units by which a tile's maximum must exceed the reference maximum to move it
    (0: the exact running maximum); P is e4m3(448 * 2^-tau * p)."""
    if int(tau) != tau or tau < 0:
        raise ValueError("tau must be a non-negative whole number")
    B, H, Nq, d = qk.q4.shape
    Hkv, Nk = qk.k4.shape[1], qk.k4.shape[2]
    sm = default_sm_scale(d) if sm_scale is None else float(np.float32(sm_scale))
    if rows is None:
        R = B * H * Nq
        rp = None
    else:
        rp = np.ascontiguousarray(rows, dtype=np.int64)
        R = rp.size
    o32 = np.empty((R, d), np.float32)
    o16 = np.empty((R, d), np.uint16)
    lse = np.empty((R,), np.float32)
    lib().orc_fp4_attn_qe(_p(qk.q4), _p(qk.qe), _p(qk.k4), _p(qk.ke), _p(qk.qk_corr), 1 if qk.per_block else 0,
                          _p(qk.lse_corr), _p(_c(v4, np.uint8)), _p(_c(ve, np.uint8)), 1 if causal else 0, sm, B, H,
                          Hkv, Nq, Nk, d, BN, float(tau), _p(rp), R, _p(o32), 1 if out_dtype == "fp16" else 0,
                          _p(o16), _p(lse))
    return o32, o16, lse


@dataclass
class FP4Result:
    qk: FP4QK
    v4: np.ndarray
    ve: np.ndarray
    o32: np.ndarray
    o16: np.ndarray
    lse: np.ndarray


def run_fp4(Q, K, V, *, causal=False, per_block_mean=True, sm_scale=None, BN=64, tau=0, rows=None, dtype="bf16",
            out_dtype=None) -> FP4Result:
    """All FP4 emulation steps: Q/K smoothing and quantization, V quantization, attention."""
    qk = fp4_quant_qk(Q, K, dtype=dtype, per_block_mean=per_block_mean)
    v4, ve = fp4_prep_v(V, dtype)
    o32, o16, lse = fp4_attn_qe(qk, v4, ve, causal=causal, sm_scale=sm_scale, BN=BN, tau=tau, rows=rows,
                                out_dtype=out_dtype or dtype)
    return FP4Result(qk, v4, ve, o32, o16, lse)
