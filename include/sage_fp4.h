/*
 * sage_fp4.h -- C ABI of libsage_mi355x's FP4 microscaling attention forward on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (SageAttention docs digest, context7 llms.txt, sections "FP4 Attention for Blackwell
 * GPUs" and "sageattn3_blackwell"; FlashInfer API doc "flashinfer.nvfp4_attention_sm120_fwd"):
 *   O = softmax(Q K^T * sm_scale [causal]) V with Q, K and V quantized to FP4 with 8-bit block
 *   scales, split into a quantize call and an attention call on the packed tensors, as the
 *   FlashInfer page splits nvfp4_attention_sm120_quantize_qkv and nvfp4_attention_sm120_fwd.
 *   - K is smoothed by its per-channel token mean (it cancels in the softmax; the LSE adds
 *     sm_scale * q_i . k_mean back through lse_corr).
 *   - Q is smoothed by the mean of its own 128-token block (per_block_mean, the default on the
 *     sageattn3_blackwell section) or by its global token mean.  The smoothed-away part of the
 *     scores, qk_corr[u][j] = q_mean_u . (K_j - k_mean) -- one FP32 row per 128-token Q block, as
 *     the FlashInfer page describes its qk_correction -- is added back to every score of block u.
 *   - FP4 here is OCP MX FP4 (OCP Microscaling Formats v1.0): e2m1 elements (magnitudes 0, 0.5, 1,
 *     1.5, 2, 3, 4, 6) with one E8M0 scale byte 2^(e - 127) per 32 elements -- along the head
 *     dimension for Q and K, along the tokens for V.  The block exponent is floor(log2 amax) - 2
 *     (clamped to [-127, 127]; -127 for an all-zero block), elements round to the nearest e2m1
 *     value with ties to the even code and saturate at 6.  This is the block-scale format that
 *     gfx950's scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) applies in hardware.
 *   - P is quantized to e4m3 as in the FP8 PV path: over 64-key tiles against the exact running
 *     maximum (sage_fp4_softmax_tau() = 0), p = exp(s - m) <= 1 and P = e4m3(448 * p); the
 *     softmax denominator sums the unquantized p; O accumulates in fp32.
 *
 * Conventions as in sage_mi355x.h: device pointers, caller-owned buffers, no allocation or
 * synchronization, host validation before anything is enqueued, stream as void*.  head_dim must
 * be 128.  Every buffer below must be 16-byte aligned.  Limits: Nq, Nk <= 2^24 and
 * nqm * Nk_pad * 4 < 2^31 (the correction rows of one head fit a 32-bit buffer range).
 * The rule for non-finite inputs stated in sage_mi355x.h covers the INT8 method only: here the
 * inputs must be finite (a NaN or infinity gives unspecified values).
 */
#ifndef SAGE_FP4_H
#define SAGE_FP4_H

#include "sage_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantized Q, K, V of sage_fp4_quantize_qkv (device buffers, caller-owned, contiguous).  Q has H
 * heads, K and V Hkv heads (Hkv divides H; query head h reads key/value head h / (H / Hkv)).
 * Nq_pad / Nk_pad = sage_pad_tokens(Nq / Nk); nqm = sage_fp4_q_blocks(Nq, per_block_mean).
 *   q4       uint8 [B][H][Nq_pad][d/2]    e2m1 pairs, low nibble = even channel; pad rows zero
 *   q_scale  uint8 [B][H][Nq_pad][d/32]   E8M0 bytes in lane order: the scale of channels
 *                                         [32 k, 32 k + 32) sits at byte (k & 1) * (d/64) + k / 2
 *   k4       uint8 [B][Hkv][Nk_pad][d/2]  as q4 (smoothed K)
 *   k_scale  uint8 [B][Hkv][Nk_pad][d/32] as q_scale
 *   v4t      uint8 [B][Hkv][d][Nk_pad/2]  V transposed: e2m1 pairs along tokens, low nibble = even
 *                                         token; tokens >= Nk are zero
 *   v_scale  uint8 [B][Hkv][Nk_pad/32][d] E8M0 of (32-token block, channel c) at byte
 *                                         (c % 32) * (d/32) + c / 32 of the block's row
 *   k_mean   fp32  [B][Hkv][d]            K's token mean (fp64 sums, one rounding)
 *   q_mean   fp32  [B][H][nqm][d]         Q's 128-token block means, or its global mean (nqm = 1)
 *   qk_corr  fp32  [B][H][nqm][Nk_pad]    q_mean_u . (K_j - k_mean), zero for j >= Nk
 *   lse_corr fp32  [B][H][Nq]             sum_c Q[i,c] * k_mean[c] (fp64 sums) */
typedef struct {
  uint8_t* q4;
  uint8_t* q_scale;
  uint8_t* k4;
  uint8_t* k_scale;
  uint8_t* v4t;
  uint8_t* v_scale;
  float* k_mean;
  float* q_mean;
  float* qk_corr;
  float* lse_corr;
  int64_t B, H, Hkv, Nq, Nk, d, Nq_pad, Nk_pad;
  int per_block_mean;
} sage_fp4_qkv;

/* Rows of q_mean / qk_corr per head: ceil(Nq/128) with per_block_mean, else 1.  Host only. */
int64_t sage_fp4_q_blocks(int64_t Nq, int per_block_mean);

/* Threshold of sage_fp4_attn_fwd's online softmax in log2 units: the reference maximum moves when
 * a 64-key tile's maximum exceeds it by more than this.  It is 0, the exact running maximum, so
 * P = e4m3(448 * p) with p <= 1.  Host only. */
double sage_fp4_softmax_tau(void);

/* Workspace bytes sage_fp4_quantize_qkv needs (fp64 partial sums of the token means).  Host only. */
size_t sage_fp4_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d);

/* Step 1 (quantize): reads q [B,H,Nq,d], k and v [B,Hkv,Nk,d] (all bf16 or all fp16, d = 128) and
 * writes every buffer of *out (out->per_block_mean selects the Q smoothing).  Per head:
 *   k_mean = fp32(sum_t fp64(K_t) / Nk);  Ktilde = fp32(K - k_mean);
 *   q_mean_u = fp32(sum_{t in block u} fp64(Q_t) / count) (or over all Nq tokens);
 *   Qtilde = fp32(Q - q_mean_u);  MX FP4 codes and scales of Qtilde, Ktilde (per 32 channels) and
 *   of V (per 32 tokens); qk_corr and lse_corr as above.  The GPU forms qk_corr as
 *   q_mean_u . K_j - q_mean_u . k_mean: exact products of bf16 parts of both (three for q_mean,
 *   one for a bf16 K, two for an fp16 K) accumulated in fp32 from -(q_mean_u . k_mean), which is
 *   summed in fp64; its error scales with |q_mean| |K|.
 * Sources: docs digest "FP4 Attention for Blackwell GPUs" / "sageattn3_blackwell"; FlashInfer API
 * doc, parameters q_fp4 / k_fp4 / v_fp4_t, q_scale / k_scale / v_scale_t, qk_correction,
 * per_block_mean.
 * Errors: INVALID_ARGUMENT (null or misaligned pointers, shape / dtype mismatch, wrong pads or
 * per_block_mean not 0/1), UNSUPPORTED (d != 128, sizes past the limits, non-gfx950 device),
 * WORKSPACE (smaller than sage_fp4_workspace_bytes), HIP. */
sage_status sage_fp4_quantize_qkv(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qkv_desc* v,
                                  const sage_fp4_qkv* out, void* workspace, size_t workspace_bytes, void* stream);

/* Step 2 (attention) on the packed tensors of step 1.
 *   causal: key j is visible to query i only if j <= i (top-left aligned).
 *   sm_scale: <= 0 selects 1/sqrt(d) (FlashInfer API doc, parameter sm_scale); NaN or +-inf is
 *        INVALID_ARGUMENT.
 *   out: [B,H,Nq,d] of out_dtype (SAGE_BF16 / SAGE_FP16 rounded to nearest even, or SAGE_F32),
 *        addressed with out_stride_{b,h,n} in elements (rows 16-byte aligned).
 *   lse: NULL, or fp32 [B][H][Nq] contiguous: natural-log log-sum-exp of the scaled scores of the
 *        unsmoothed K (lse_corr added back).
 * Scores S_ij = sum_c deq(q)_ic deq(k)_jc + qk_corr[u(i)][j] accumulate in fp32 on the MFMA; the
 * online softmax runs over 64-key tiles in increasing key order with the lazy reference maximum of
 * sage_fp4_softmax_tau(); keys j >= Nk are masked before the softmax (FlashInfer API doc, parameter
 * unpadded_k_len).  A row with no visible key gets O = 0 and LSE = -inf.
 * Errors: INVALID_ARGUMENT (null or misaligned pointers, bad strides or out_dtype), UNSUPPORTED,
 * HIP. */
sage_status sage_fp4_attn_fwd(const sage_fp4_qkv* qkv, int causal, float sm_scale, void* out, sage_dtype out_dtype,
                              int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse,
                              void* stream);

/* Debug: the raw fp32 scores S (before sm_scale) of query head (b, h) for rows [row0, row0+nrows)
 * and keys [col0, col0+ncols), computed by the attention kernel's tile code.  out: fp32
 * [nrows][ncols] device buffer.  The window must lie inside [0,Nq_pad) x [0,Nk_pad). */
sage_status sage_fp4_debug_scores(const sage_fp4_qkv* qkv, int64_t b, int64_t h, int64_t row0, int64_t nrows,
                                  int64_t col0, int64_t ncols, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_FP4_H */
