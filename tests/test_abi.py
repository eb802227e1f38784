"""The C-ABI library loads, exports every symbol include/*.h declares, and rejects bad arguments
with the documented status codes before touching any device (so these run without a GPU)."""

import ctypes
import glob
import os
import re

import pytest

from quantized_attention_quantize_amd import api

from schedule import BLOCK_N, ROWSUM_ROUNDED, TAU, TAU_FP4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(sage_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def L():
    return api.load_library()


def test_every_declared_symbol_is_exported(L):
    names = declared_symbols()
    assert {"sage_quantize_qk", "sage_attn_fwd", "sage_debug_qk_int32", "sage_prepare_v", "sage_attn_fwd_prepared"} <= names
    for n in names:
        assert hasattr(L, n), n
    assert set(api.EXPORTS) == names


def test_host_queries(L):
    assert L.sage_pad_tokens(1) == 128 and L.sage_pad_tokens(128) == 128 and L.sage_pad_tokens(17776) == 17792
    assert L.sage_pad_tokens(0) == 0
    assert L.sage_block_n(0) == 64 and L.sage_block_n(1) == 64
    # the library reports the online schedule the parity tests fix as constants (gpu_helpers)
    L.sage_softmax_tau.restype = ctypes.c_double
    assert L.sage_block_n(0) == BLOCK_N and L.sage_block_n(1) == BLOCK_N
    assert L.sage_softmax_tau(0) == TAU["fp16"] and L.sage_softmax_tau(1) == TAU["fp8"]
    assert L.sage_rowsum_rounded(0) == int(ROWSUM_ROUNDED) and L.sage_rowsum_rounded(1) == int(ROWSUM_ROUNDED)
    assert L.sage_quantize_workspace_bytes(2, 32, 8192, 128) == 2 * 32 * 32 * 128 * 8
    assert L.sage_quantize_workspace_bytes(0, 1, 1, 64) == 0
    # prepared fp16 V of the 8192-token, 64-head workload
    # prepared V, the smooth_v V mean and the fp64 partial sums (one per 256-token chunk)
    assert L.sage_fwd_workspace_bytes(2, 32, 8192, 8192, 128, 0, 0) == 2 * 32 * 128 * (8192 * 2 + 4 + 32 * 8)
    base8 = L.sage_fwd_workspace_bytes(1, 24, 17776, 17776, 128, 1, 0)
    assert base8 >= 24 * 128 * 17792 + 24 * 128 * 4
    with_mask = L.sage_fwd_workspace_bytes(2, 32, 8192, 8192, 128, 0, 1)
    assert with_mask - L.sage_fwd_workspace_bytes(2, 32, 8192, 8192, 128, 0, 0) >= 2 * 32 * 128
    assert L.sage_fwd_workspace_bytes(1, 1, 1, 1, 64, 7, 0) == 0
    assert L.sage_fwd_workspace_bytes(1, 1, 1, 1, 64, -1, 0) == 0
    for s, txt in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace missing or too small")]:
        assert L.sage_status_string(s) == txt


FAKE = 0x100000  # a 16-byte aligned non-null address; validation fails before anything dereferences it


def desc(B=1, H=2, N=256, d=64, dtype=0, data=FAKE, sb=None, sh=None, sn=None):
    sn = d if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = H * sh if sb is None else sb
    return api.QKVDesc(data, dtype, B, H, N, d, sb, sh, sn)


def quant(B=1, H=2, Nq=256, Nk=256, d=64, pad=None, null=None, Hkv=None):
    ptrs = [FAKE] * 6
    if null is not None:
        ptrs[null] = 0
    npq = L_pad(Nq) if pad is None else pad
    return api.QKQuant(*ptrs, B, H, H if Hkv is None else Hkv, Nq, Nk, d, npq, L_pad(Nk), None, None)


def L_pad(n):
    return (n + 127) // 128 * 128


def call_quant(L, q, k, out, ws=FAKE, wsb=1 << 20):
    return L.sage_quantize_qk(ctypes.byref(q) if q else None, ctypes.byref(k) if k else None,
                              ctypes.byref(out) if out else None, ws, wsb, None)


@pytest.mark.parametrize("case,status", [
    ("null_q", INVALID), ("null_data", INVALID), ("zero_B", INVALID), ("neg_N", INVALID), ("d96", UNSUPPORTED),
    ("qk_dtype_mismatch", INVALID), ("bad_dtype", INVALID), ("neg_dtype", INVALID), ("max_dtype", INVALID),
    ("misaligned", INVALID), ("odd_stride", INVALID),
    ("small_stride_n", INVALID), ("qk_mismatch_H", INVALID), ("out_null_ptr", INVALID), ("out_bad_pad", INVALID),
    ("out_wrong_N", INVALID), ("no_workspace", WORKSPACE), ("small_workspace", WORKSPACE),
    ("gqa_out_hkv", INVALID), ("gqa_not_divisor", INVALID),
])
def test_quantize_validation(L, case, status):
    q, k, out = desc(), desc(), quant()
    ws, wsb = FAKE, 1 << 20
    if case == "null_q":
        q = None
    elif case == "null_data":
        q = desc(data=0)
    elif case == "zero_B":
        q = desc(B=0)
    elif case == "neg_N":
        k = desc(N=-5)
    elif case == "d96":
        q, k = desc(d=96), desc(d=96)
    elif case == "qk_dtype_mismatch":  # fp16 Q with bf16 K
        q = desc(dtype=1)
    elif case == "bad_dtype":
        q = desc(dtype=9)
    elif case == "neg_dtype":  # any int is a value of the C enum; unknown ones are rejected
        q, k = desc(dtype=-1), desc(dtype=-1)
    elif case == "max_dtype":
        q, k = desc(dtype=0x7FFFFFFF), desc(dtype=0x7FFFFFFF)
    elif case == "misaligned":
        q = desc(data=FAKE + 2)
    elif case == "odd_stride":
        k = desc(sn=68)
    elif case == "small_stride_n":
        k = desc(sn=32)
    elif case == "qk_mismatch_H":
        k = desc(H=3)
    elif case == "out_null_ptr":
        out = quant(null=3)
    elif case == "out_bad_pad":
        out = quant(pad=200)
    elif case == "out_wrong_N":
        out = quant(Nq=255)
    elif case == "no_workspace":
        ws = 0
    elif case == "small_workspace":
        wsb = 16
    elif case == "gqa_out_hkv":  # K has 1 head, the output struct says 2
        k = desc(H=1)
    elif case == "gqa_not_divisor":  # 3 key heads cannot serve 4 query heads
        q, k, out = desc(H=4), desc(H=3), quant(H=4, Hkv=3)
    assert call_quant(L, q, k, out, ws, wsb) == status


def call_fwd(L, qk, v, mask=None, mdt=0, mask_h=0, msq=256, pv=0, out=FAKE, odt=0, osn=64, ws=FAKE, wsb=1 << 30,
             smooth_v=0, sm=0.0):
    return L.sage_attn_fwd(ctypes.byref(qk) if qk else None, ctypes.byref(v) if v else None, mask, mdt, mask_h, 0, 0,
                           msq, 0, sm, pv, smooth_v, out, odt, 2 * 256 * 64, 256 * 64, osn, None, ws, wsb, None)


@pytest.mark.parametrize("case,status", [
    ("null_qk", INVALID), ("v_shape", INVALID), ("pv_bad", UNSUPPORTED), ("out_null", INVALID),
    ("out_bad_dtype", INVALID), ("out_misaligned", INVALID), ("mask_dtype_bad", INVALID),
    ("mask_f32_misaligned", INVALID), ("smooth_v_fp8", UNSUPPORTED), ("mask_h_bad", INVALID), ("mask_stride_small", INVALID),
    ("ws_small", WORKSPACE), ("ws_null", WORKSPACE), ("qk_d", UNSUPPORTED), ("gqa_v_heads", INVALID),
    ("gqa_hkv_zero", INVALID), ("sm_nan", INVALID), ("sm_inf", INVALID),
    # a key-padding mask (one row of keys for every query, mask_stride_q = 0) passes validation:
    # the call then stops at the workspace check, before anything is enqueued
    ("mask_stride_q_zero", WORKSPACE),
])
def test_attn_validation(L, case, status):
    qk, v = quant(), desc()
    kw = {}
    if case == "null_qk":
        qk = None
    elif case == "v_shape":
        v = desc(N=128)
    elif case == "pv_bad":
        kw["pv"] = 5
    elif case == "out_null":
        kw["out"] = 0
    elif case == "out_bad_dtype":
        kw["odt"] = 7
    elif case == "mask_dtype_bad":
        kw.update(mask=FAKE, mdt=5, mask_h=1)
    elif case == "mask_f32_misaligned":  # an fp32 mask must be 4-byte aligned
        kw.update(mask=FAKE + 2, mdt=1, mask_h=1)
    elif case == "smooth_v_fp8":  # smooth_v belongs to the FP16 PV path
        kw.update(pv=1, smooth_v=1)
    elif case == "out_misaligned":
        kw["out"] = FAKE + 8
    elif case == "mask_h_bad":
        kw.update(mask=FAKE, mask_h=3)
    elif case == "mask_stride_small":
        kw.update(mask=FAKE, mask_h=1, msq=100)
    elif case == "ws_small":
        kw["wsb"] = 100
    elif case == "ws_null":
        kw["ws"] = 0
    elif case == "qk_d":
        qk = quant(d=80)
    elif case == "gqa_v_heads":  # V must have the Hkv heads of K
        qk = quant(H=2, Hkv=1)
    elif case == "gqa_hkv_zero":
        qk = quant(Hkv=0)
    elif case == "sm_nan":
        kw["sm"] = float("nan")
    elif case == "sm_inf":
        kw["sm"] = float("inf")
    elif case == "mask_stride_q_zero":
        kw.update(mask=FAKE, mask_h=1, msq=0, wsb=100)
    assert call_fwd(L, qk, v, **kw) == status


@pytest.mark.parametrize("pv,Nk,status", [
    # one head's prepared V is addressed through a 32-bit buffer range: Nk_pad * d * esz < 2^31
    (0, (1 << 23) - 128, WORKSPACE), (0, 1 << 23, UNSUPPORTED),  # FP16 V, 2 bytes per element
    (1, 1 << 23, WORKSPACE), (1, (1 << 24) - 128, WORKSPACE),    # e4m3 V, 1 byte per element
])
def test_attn_buffer_range_limit(L, pv, Nk, status):
    """Past the 32-bit buffer ranges of the attention kernel's prepared-V addressing the call is
    UNSUPPORTED (host validation, nothing enqueued); just below it the call passes validation and
    stops at the (deliberately small) workspace."""
    qk, v = quant(Nk=Nk, d=128), desc(N=Nk, d=128)
    assert call_fwd(L, qk, v, pv=pv, osn=128, wsb=100) == status


@pytest.mark.parametrize("Nk,status", [((1 << 24) - 128, WORKSPACE), (1 << 24, UNSUPPORTED)])
def test_quantize_buffer_range_limit(L, Nk, status):
    """One head's K8 rows (Nk_pad * d bytes) are addressed through a 32-bit buffer range."""
    q, k, out = desc(d=128), desc(N=Nk, d=128), quant(Nk=Nk, d=128)
    assert call_quant(L, q, k, out, wsb=16) == status


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,pbm", [(1, 2, 2, 256, 256, 64, 0), (2, 32, 8, 8192, 8192, 128, 0),
                                                  (1, 3, 1, 300, 417, 128, 1), (2, 4, 4, 1, 17776, 64, 1)])
def test_qk_quant_bytes_and_init(L, B, H, Hkv, Nq, Nk, d, pbm):
    """sage_qk_quant_bytes sizes one allocation for every buffer of the quantized Q/K (each on a
    256-byte boundary, in the documented order), and sage_qk_quant_init lays the struct out in it:
    pointers at those offsets, the sizes and pads filled in.  The buffer sizes are the shapes the
    Python binding allocates (alloc_quantized)."""
    import torch
    g = api.alloc_quantized(B, H, Nq, Nk, d, "cpu", Hkv=Hkv, per_block_mean=bool(pbm))
    bufs = [g.q8, g.k8, g.q_scale, g.k_scale, g.k_mean, g.lse_corr]
    if pbm:
        bufs += [g.k_block_mean, g.blk_corr]
    offs, off = [], 0
    for t in bufs:
        offs.append(off)
        off += (t.numel() * t.element_size() + 255) // 256 * 256
    assert L.sage_qk_quant_bytes(B, H, Hkv, Nq, Nk, d, pbm) == off
    base = 0x40000000
    st = api.QKQuant()
    assert L.sage_qk_quant_init(base, off, B, H, Hkv, Nq, Nk, d, pbm, ctypes.byref(st)) == 0
    ptrs = [st.q8, st.k8, st.q_scale, st.k_scale, st.k_mean, st.lse_corr] + \
        ([st.k_block_mean, st.blk_corr] if pbm else [])
    assert [p - base for p in ptrs] == offs
    assert (st.B, st.H, st.Hkv, st.Nq, st.Nk, st.d) == (B, H, Hkv, Nq, Nk, d)
    assert (st.Nq_pad, st.Nk_pad) == (L_pad(Nq), L_pad(Nk))
    if not pbm:
        assert not st.k_block_mean and not st.blk_corr
    # too small, misaligned, or invalid sizes
    assert L.sage_qk_quant_init(base, off - 1, B, H, Hkv, Nq, Nk, d, pbm, ctypes.byref(st)) == INVALID
    assert L.sage_qk_quant_init(base + 16, off, B, H, Hkv, Nq, Nk, d, pbm, ctypes.byref(st)) == INVALID
    assert L.sage_qk_quant_bytes(B, H, 5, Nq, Nk, d, pbm) == 0 and L.sage_qk_quant_bytes(B, H, Hkv, Nq, Nk, 96, pbm) == 0
    del torch


def test_per_block_mean_validation(L):
    qk = quant()
    qk.k_block_mean = FAKE  # without blk_corr
    assert call_fwd(L, qk, desc()) == INVALID
    qk.blk_corr = FAKE  # per_block_mean with an fp32 mask is not offered
    assert call_fwd(L, qk, desc(), mask=FAKE, mdt=1, mask_h=1) == UNSUPPORTED


def test_per_block_mean_size_limit(L):
    """One head's per_block_mean score terms are addressed through a 32-bit buffer range, so
    ceil(Nk/64) * Nq * 4 bytes past 2^31 is UNSUPPORTED.  A null workspace (checked later) shows
    that the limit is what rejects the call, and only with per_block_mean."""
    n = 1 << 20  # 16384 key blocks x 2^20 rows x 4 B = 64 GiB per head
    q, k = desc(N=n), desc(N=n)
    out = quant(Nq=n, Nk=n)
    assert call_quant(L, q, k, out, ws=0) == WORKSPACE
    out.k_block_mean = FAKE
    out.blk_corr = FAKE
    assert call_quant(L, q, k, out, ws=0) == UNSUPPORTED
    m = 1 << 14  # 256 x 16384 x 4 B = 16 MiB
    small = quant(Nq=m, Nk=m)
    small.k_block_mean = FAKE
    small.blk_corr = FAKE
    assert call_quant(L, desc(N=m), desc(N=m), small, ws=0) == WORKSPACE


def test_debug_validation(L):
    qk = quant()
    out = FAKE
    assert L.sage_debug_qk_int32(ctypes.byref(qk), 0, 0, 0, 10, 0, 10, 0, None) == INVALID
    assert L.sage_debug_qk_int32(ctypes.byref(qk), 1, 0, 0, 10, 0, 10, out, None) == INVALID  # b >= B
    assert L.sage_debug_qk_int32(ctypes.byref(qk), 0, 0, 200, 100, 0, 10, out, None) == INVALID  # past Nq_pad
    assert L.sage_debug_qk_int32(ctypes.byref(qk), 0, 0, 0, 10, -1, 10, out, None) == INVALID
    v = desc()
    assert L.sage_prepare_v(ctypes.byref(v), 1, FAKE, None, None, FAKE, 1 << 20, None) == INVALID  # fp8 needs v_scale
    assert L.sage_prepare_v(ctypes.byref(v), 1, FAKE, FAKE, None, FAKE, 10, None) == WORKSPACE
    assert L.sage_prepare_v(ctypes.byref(v), 1, FAKE, FAKE, None, 0, 1 << 20, None) == WORKSPACE
    assert L.sage_prepare_v(ctypes.byref(v), 3, FAKE, None, None, FAKE, 1 << 20, None) == UNSUPPORTED
    assert L.sage_prepare_v(ctypes.byref(v), 0, FAKE + 4, None, None, None, 0, None) == INVALID  # misaligned v_t
    assert L.sage_prepare_v(ctypes.byref(v), 1, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == UNSUPPORTED  # fp8 + smooth_v
    assert L.sage_prepare_v(ctypes.byref(v), 0, FAKE, None, FAKE, None, 0, None) == WORKSPACE  # smooth_v needs scratch


def test_prepared_attn_validation(L):
    qk = quant()
    args = [0, None, 0, 0, 0, 0, 0, 0, 0.0, FAKE, 0, 2 * 256 * 64, 256 * 64, 64, None]
    f = L.sage_attn_fwd_prepared
    assert f(ctypes.byref(qk), 0, None, None, *args, None, 0, None) == INVALID  # no v_t
    assert f(ctypes.byref(qk), FAKE, None, None, 1, *args[1:], None, 0, None) == INVALID  # fp8 without v_scale
    masked = [0, FAKE, 0, 1, 0, 0, 256, 0, 0.0, FAKE, 0, 2 * 256 * 64, 256 * 64, 64, None]
    assert f(ctypes.byref(qk), FAKE, None, None, *masked, None, 0, None) == WORKSPACE  # mask needs tile workspace
    assert L.sage_mask_workspace_bytes(2, 8192, 8192, 1) == 2 * 32 * 128 * 4  # one int32 state per tile
    assert L.sage_mask_workspace_bytes(2, 8192, 8192, 0) == 0
    assert L.sage_prepare_v_workspace_bytes(1, 24, 17776, 128, 0) >= 24 * 70 * 128 * 8  # smooth_v's fp64 sums
    assert L.sage_prepare_v_workspace_bytes(1, 24, 17776, 128, 1) >= 24 * 70 * 128 * 4


def test_no_oracle_on_product_path():
    """The product package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "quantized_attention_quantize_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if path.endswith((".py", ".cpp", ".hip", ".h")):
            text = open(path).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b|libsage_oracle|sage_oracle\.c", text, flags=re.M), path


@pytest.mark.parametrize("case", ["S0", "d_odd", "d_big", "bad_part_dtype", "bad_out_dtype", "null_parts", "null_lse",
                                  "null_out", "parts_misaligned", "out_stride_small", "out_stride_odd"])
def test_merge_validation(L, case):
    a = dict(S=2, B=1, H=2, Nq=64, d=64, parts=FAKE, pdt=0, lse=FAKE, out=FAKE, odt=0, sb=2 * 64 * 64, sh=64 * 64, sn=64)
    if case == "S0":
        a["S"] = 0
    elif case == "d_odd":
        a["d"] = 60
    elif case == "d_big":
        a["d"] = 2048
    elif case == "bad_part_dtype":
        a["pdt"] = 3
    elif case == "bad_out_dtype":
        a["odt"] = -1
    elif case == "null_parts":
        a["parts"] = 0
    elif case == "null_lse":
        a["lse"] = 0
    elif case == "null_out":
        a["out"] = 0
    elif case == "parts_misaligned":
        a["parts"] = FAKE + 4
    elif case == "out_stride_small":
        a["sn"] = 32
    elif case == "out_stride_odd":
        a["sn"] = 68
    st = L.sage_merge_lse(a["S"], a["B"], a["H"], a["Nq"], a["d"], a["parts"], a["pdt"], a["lse"], a["out"], a["odt"],
                          a["sb"], a["sh"], a["sn"], None, None)
    assert st == INVALID


def _fp4_struct(B=1, H=2, Hkv=2, Nq=300, Nk=200, d=128, pbm=1, ptr=None):
    p = FAKE if ptr is None else ptr
    return api.FP4QKV(p, p, p, p, p, p, p, p, p, p, B, H, Hkv, Nq, Nk, d, L_pad(Nq), L_pad(Nk), pbm)


def L_pad(n):
    return (n + 127) // 128 * 128


def test_fp4_host_queries(L):
    assert L.sage_fp4_q_blocks(300, 1) == 3 and L.sage_fp4_q_blocks(300, 0) == 1 and L.sage_fp4_q_blocks(0, 1) == 0
    assert L.sage_fp4_softmax_tau() == TAU_FP4  # the exact running maximum: P = e4m3(448 * p)
    # fp64 partial sums of the larger of the Q and K token-mean reductions (256-token chunks)
    assert L.sage_fp4_workspace_bytes(2, 32, 8, 8192, 8192, 128) == 2 * 32 * 32 * 128 * 8
    assert L.sage_fp4_workspace_bytes(0, 1, 1, 1, 1, 128) == 0


def test_fp4_validation(L):
    q = desc(B=1, H=2, N=300, d=128)
    k = desc(B=1, H=2, N=200, d=128)
    x = _fp4_struct()
    f = L.sage_fp4_quantize_qkv
    ws = 1 << 20
    assert f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(x), FAKE, 10, None) == WORKSPACE
    assert f(ctypes.byref(q), ctypes.byref(k), None, ctypes.byref(x), FAKE, ws, None) == INVALID
    k64 = desc(B=1, H=2, N=200, d=64)
    assert f(ctypes.byref(q), ctypes.byref(k64), ctypes.byref(k64), ctypes.byref(x), FAKE, ws, None) == INVALID
    q64 = desc(B=1, H=2, N=300, d=64)
    x64 = _fp4_struct(d=64)
    assert f(ctypes.byref(q64), ctypes.byref(k64), ctypes.byref(k64), ctypes.byref(x64), FAKE, ws, None) == UNSUPPORTED
    assert f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(_fp4_struct(pbm=2)), FAKE, ws,
             None) == INVALID
    assert f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(_fp4_struct(ptr=FAKE + 8)), FAKE, ws,
             None) == INVALID  # misaligned buffers
    assert f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(_fp4_struct(Nk=201)), FAKE, ws,
             None) == INVALID  # shape mismatch with k
    big = _fp4_struct(Nq=1 << 24, Nk=1 << 24)  # correction rows of one head past 2 GiB
    a = L.sage_fp4_attn_fwd
    assert a(ctypes.byref(big), 0, 0.0, FAKE, 0, 128, 128, 128, None, None) == UNSUPPORTED
    assert a(ctypes.byref(x), 0, 0.0, None, 0, 128, 128, 128, None, None) == INVALID
    assert a(ctypes.byref(x), 0, 0.0, FAKE, 7, 128, 128, 128, None, None) == INVALID  # unknown out dtype
    assert a(ctypes.byref(x), 0, 0.0, FAKE, 0, 128, 128, 100, None, None) == INVALID  # stride_n < d
    assert a(ctypes.byref(x), 0, 0.0, FAKE + 2, 0, 128, 128, 128, None, None) == INVALID
    g = L.sage_fp4_debug_scores
    assert g(ctypes.byref(x), 0, 2, 0, 10, 0, 10, FAKE, None) == INVALID  # h >= H
    assert g(ctypes.byref(x), 0, 0, 300, 100, 0, 10, FAKE, None) == INVALID  # past Nq_pad
    assert g(ctypes.byref(x), 0, 0, 0, 10, 0, 10, None, None) == INVALID


def test_python_sm_scale_argument():
    """The binding passes 0 (the C default, 1/sqrt(d)) only when no sm_scale is given; an explicit
    zero, negative or non-finite value is refused instead of silently replaced."""
    assert api.sm_scale_arg(None) == 0.0
    assert api.sm_scale_arg(0.125) == 0.125
    for bad in (0.0, -0.5, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            api.sm_scale_arg(bad)


def test_noalloc_quantize_validation(L):
    """The allocation-free quantize entry point validates like sage_quantize_qk (host only, before
    any HIP call) and refuses sizes whose K-mean partial sums would not fit its 8 MiB scratch array:
    B * Hkv * ceil(Nk/256) * d doubles."""
    def call(q, k, out):
        return L.sage_quantize_qk_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(out), None)
    assert call(desc(data=0), desc(), quant()) == INVALID
    assert call(desc(d=96), desc(d=96), quant(d=96)) == UNSUPPORTED
    assert L.sage_quantize_workspace_bytes(1, 64, 40000, 128) > (8 << 20)
    big_q, big_k, big_out = desc(H=64, N=40000, d=128), desc(H=64, N=40000, d=128), quant(H=64, Nq=40000, Nk=40000,
                                                                                           d=128)
    assert call(big_q, big_k, big_out) == WORKSPACE


def test_sclk_probe_validation(L):
    """The clock probe rejects bad sizes and a misaligned or null buffer before anything runs."""
    f = L.sage_sclk_probe
    assert f(0, 10, 1, FAKE, None) == INVALID
    assert f(65537, 10, 1, FAKE, None) == INVALID
    assert f(8, 0, 0, FAKE, None) == INVALID
    assert f(8, (1 << 24) + 1, 1, FAKE, None) == INVALID
    assert f(8, 10, 2, FAKE, None) == INVALID
    assert f(8, 10, 1, None, None) == INVALID
    assert f(8, 10, 0, FAKE + 4, None) == INVALID
