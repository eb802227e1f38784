/*
 * sage_mi355x.h -- C ABI of libsage_mi355x: SageAttention-style quantized attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (SageAttention docs digest, context7 llms.txt; sections
 * "sageattn_qk_int8_pv_fp16_triton -- Triton INT8/FP16 kernel (Ampere/Ada)",
 * "SageAttention CUDA INT8/FP16 Kernel (Ampere sm80)", "sageattn_qk_int8_pv_fp8_cuda"):
 *   O = softmax(Q K^T * sm_scale [masked]) V, where
 *   - K is smoothed by subtracting its per-channel mean over tokens (exact under softmax);
 *   - Q and the smoothed K are quantized to INT8 with one scale per 64-token block;
 *   - Q K^T runs as an INT8 product with int32 accumulation and is then dequantized;
 *   - the softmax is computed online over 64-key tiles;
 *   - P V runs in FP16 (P and V rounded to fp16) or in FP8 e4m3 (V per channel, P with the static
 *     scale 448), accumulated in FP32.
 * The split into a quantize call and an attention call on pre-quantized tensors, and the
 * caller-supplied out / lse buffers, follow the FlashInfer API doc
 * "flashinfer.nvfp4_attention_sm120_fwd" (parameters out, lse, sm_scale, unpadded_k_len).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device; the caller allocates and
 *    owns every buffer, including workspaces.  The library never allocates, frees or synchronizes
 *    and keeps no mutable global state (one cached per-device architecture check aside).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is enqueued on it
 *    and the call returns without waiting; asynchronous faults surface at the caller's next sync.
 *  - Host-side argument validation runs before any HIP call and before any launch; a non-OK status
 *    means nothing was enqueued.  Launch failures report SAGE_ERR_HIP.
 *  - Inputs are bf16 or fp16, q, k and v alike (the input types the SageAttention usage section
 *    names), with a contiguous channel (head_dim) axis; batch, head and token
 *    strides are free (HND or NHD), given in elements, and must keep every row 16-byte aligned.
 *    An fp16 input is decoded exactly; the method then runs as for bf16.
 *  - head_dim d must be 64 or 128.  Index arithmetic is 64-bit.
 *  - Non-finite inputs (no page covers them; this library's rule) are never dropped and never
 *    turn into finite values.  A NaN in a quantization group (a 64-token block of Q or of the
 *    smoothed K, an FP8 V channel) makes the group's scale NaN, and every code of a group whose
 *    scale is NaN or +inf is 0; means are plain sums.  A row's O and LSE are NaN when one of its
 *    visible keys has a NaN score (its Q block's scale, its key block's scale or mean, or K's
 *    mean is NaN).  A NaN in fp16 V at (key j, channel c) makes O[i,c] NaN for every row i with a
 *    visible key whose key loop covers j's 64-key tile: the rows that see key j and, because a
 *    zero probability times NaN is NaN, the other rows of that loop (the loop of a 256-row query
 *    block: under causal masking the tiles up to the block's last row; tiles that the mask hides
 *    from the whole block are skipped).  A NaN FP8 V channel scale or smooth_v channel mean
 *    reaches that channel of every row with a visible key; V never reaches the LSE.  A row
 *    without a visible key gives O = 0 and LSE = -inf whatever the inputs hold.  Infinities in Q
 *    or K give NaN scores the same way.
 */
#ifndef SAGE_MI355X_H
#define SAGE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride, alignment or dtype mismatch */
  SAGE_ERR_UNSUPPORTED = 2,      /* head_dim not 64/128, or a device other than gfx950 */
  SAGE_ERR_WORKSPACE = 3,        /* workspace smaller than the matching *_workspace_bytes() value */
  SAGE_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} sage_status;

/* The input enums below span every 32-bit int (the *_MIN_ / *_MAX_ enumerators are not values to
 * pass): whatever int a caller stores in one is a value of the type, and the entry points reject
 * an unknown one with SAGE_ERR_INVALID_ARGUMENT. */

/* Element type of Q, K, V (bf16 or fp16) and of the output O (any of the three; fp32 for partial
 * results that sage_merge_lse combines later). */
typedef enum {
  SAGE_BF16 = 0,
  SAGE_FP16 = 1,
  SAGE_F32 = 2,
  SAGE_DTYPE_MIN_ = -0x7fffffff - 1,
  SAGE_DTYPE_MAX_ = 0x7fffffff
} sage_dtype;

/* Attention mask element type (optional boolean or float32 mask: Triton INT8/FP16 kernel section).
 *   SAGE_MASK_BOOL: uint8, nonzero = attend, 0 = masked out.
 *   SAGE_MASK_F32:  fp32 added to the scaled score sm_scale * q.k (natural-log units) before the
 *                   softmax; -inf masks the key.  Entries must be finite or -inf. */
typedef enum {
  SAGE_MASK_BOOL = 0,
  SAGE_MASK_F32 = 1,
  SAGE_MASK_DTYPE_MIN_ = -0x7fffffff - 1,
  SAGE_MASK_DTYPE_MAX_ = 0x7fffffff
} sage_mask_dtype;

typedef enum {
  SAGE_PV_FP16 = 0,
  SAGE_PV_FP8_E4M3 = 1,
  SAGE_PV_DTYPE_MIN_ = -0x7fffffff - 1,
  SAGE_PV_DTYPE_MAX_ = 0x7fffffff
} sage_pv_dtype;

/* A Q, K or V tensor of shape [B, H, N, d] addressed as
 *   data + b*stride_b + h*stride_h + n*stride_n + c      (element offsets, c contiguous). */
typedef struct {
  const void* data;
  sage_dtype dtype;
  int64_t B, H, N, d;
  int64_t stride_b, stride_h, stride_n;
} sage_qkv_desc;

/* Quantized Q/K produced by sage_quantize_qk (all device buffers, caller-owned, contiguous).
 * Q has H heads; K and V have Hkv heads, Hkv dividing H (group-query attention: query head h
 * reads key/value head h / (H / Hkv); Hkv = H is ordinary attention).  (Group-query attention,
 * 16 query heads over 4 key/value heads: sageattn section of the SageAttention docs digest.)
 *   q8       int8  [B][H][Nq_pad][d]     rows >= Nq are zero
 *   k8       int8  [B][Hkv][Nk_pad][d]   smoothed K codes; rows >= Nk are zero
 *   q_scale  fp32  [B][H][ceil(Nq/64)]   per-64-token-block scale  (amax/127; 0 for an all-zero block)
 *   k_scale  fp32  [B][Hkv][ceil(Nk/64)]
 *   k_mean   fp32  [B][Hkv][d]           per-channel token mean of K (fp64 sum, rounded once)
 *   lse_corr fp32  [B][H][Nq]            sum_c Q[i,c]*k_mean[c] with the query head's key head mean:
 *                                        adds the smoothing shift back to the LSE
 * Nq_pad and Nk_pad must equal sage_pad_tokens(Nq) and sage_pad_tokens(Nk).
 * per_block_mean (the sageattn3_blackwell usage section's option; both pointers set, else both
 * NULL): K is smoothed by the mean of its own 64-token block instead of the global mean.  That
 * shift differs between blocks, so its score terms are kept and added back to the scores:
 *   k_block_mean fp32 [B][Hkv][ceil(Nk/64)][d]  block means (fp64 sum over the block's tokens,
 *                                               one rounding)
 *   blk_corr     fp32 [B][H][ceil(Nk/64)][Nq]   sum_c Q[i,c] * k_block_mean[u,c] (fp32 sums)
 * and k_mean, lse_corr hold zeros (the LSE then needs no shift).  Not combined with an fp32 mask.
 * One head's terms must fit 2 GiB: ceil(Nk/64) * Nq * 4 < 2^31 bytes, else UNSUPPORTED. */
typedef struct {
  int8_t* q8;
  int8_t* k8;
  float* q_scale;
  float* k_scale;
  float* k_mean;
  float* lse_corr;
  int64_t B, H, Hkv, Nq, Nk, d, Nq_pad, Nk_pad;
  float* k_block_mean;
  float* blk_corr;
} sage_qk_quant;

/* Bytes of one device allocation holding every buffer of a sage_qk_quant for these sizes: q8, k8,
 * q_scale, k_scale, k_mean, lse_corr and, with per_block_mean nonzero, k_block_mean and blk_corr,
 * in that order, each starting on a 256-byte boundary.  0 if the sizes are invalid (non-positive,
 * Hkv not dividing H, d not in {64,128}).  Host only.  (The separate quantize -> attention steps
 * with caller-owned buffers: FlashInfer API doc, flashinfer.nvfp4_attention_sm120_fwd.) */
size_t sage_qk_quant_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int per_block_mean);

/* Lays a sage_qk_quant out in one caller allocation: fills every pointer of *out (offsets as in
 * sage_qk_quant_bytes from base), the sizes and the pads.  base must be 256-byte aligned and hold
 * at least sage_qk_quant_bytes(...) bytes.  Host only: touches neither HIP nor the memory; the
 * caller still owns the allocation.  Errors: INVALID_ARGUMENT (null base or out, misaligned base,
 * bytes too small, invalid sizes). */
sage_status sage_qk_quant_init(void* base, size_t bytes, int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                               int64_t d, int per_block_mean, sage_qk_quant* out);

/* Padded token extent of q8 / k8 / prepared V: n rounded up to a multiple of 128. Host only. */
int64_t sage_pad_tokens(int64_t n);

/* Keys per online-softmax tile used by sage_attn_fwd (the running maximum is updated once per
 * tile, which fixes where P is rounded).  Host only. */
int sage_block_n(sage_pv_dtype pv);

/* Threshold of the online softmax's reference maximum, in log2 units: sage_attn_fwd moves a row's
 * reference maximum only when a tile's maximum exceeds it by more than this (0 = the exact running
 * maximum).  The normalized result does not depend on it; only the point at which P is rounded
 * does.  8 for SAGE_PV_FP16 (a lazy maximum: P <= 256 fits fp16), 0 for SAGE_PV_FP8_E4M3 (the
 * exact running maximum: P = e4m3(448 * p) with p <= 1).  Host only. */
double sage_softmax_tau(sage_pv_dtype pv);

/* 1 if sage_attn_fwd's softmax denominator sums P as rounded for the PV product, 0 if it sums the
 * unrounded fp32 p.  It is 0 for both PV types: the denominator is the plain softmax sum.  Host
 * only. */
int sage_rowsum_rounded(sage_pv_dtype pv);

/* Bytes of workspace sage_quantize_qk needs (fp64 partial sums of the K mean); Hkv = heads of K.
 * Host only. */
size_t sage_quantize_workspace_bytes(int64_t B, int64_t Hkv, int64_t Nk, int64_t d);

/* Step 1 (quantize).  Reads q [B,H,Nq,d] and k [B,Hkv,Nk,d] (both bf16 or both fp16, same B and d, Hkv dividing H;
 * out->H = H, out->Hkv = Hkv), writes every buffer of *out.
 * Per key head (b,h): k_mean = fp32(sum_t fp64(K[t,:]) / Nk); Ks = fp32(K - k_mean); for every 64-token
 * block of Q and of Ks: scale = amax/127, code = clamp(rne(x * (127/amax)), -127, 127)
 * (IEEE fp32 divisions, round-to-nearest-even); lse_corr[i] = fp32(sum_c fp64(Q[i,c])*fp64(k_mean[c])).
 * Sources: per-block INT8 Q/K and smooth_k on the Triton INT8/FP16 kernel section; smoothing by
 * the global token mean on the sageattn3_blackwell usage section (per_block_mean=False).
 * Errors: INVALID_ARGUMENT for null pointers, non-positive sizes, mismatched B/H/d/dtype, wrong
 * pads or misaligned rows; UNSUPPORTED for d not in {64,128}, for one head's K8 rows past a 32-bit buffer
 * range (Nk_pad * d >= 2^31) or per_block_mean past its size limit; WORKSPACE if
 * workspace_bytes < sage_quantize_workspace_bytes(). */
sage_status sage_quantize_qk(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qk_quant* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free step 1, for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The same computation, arguments and results
 * as sage_quantize_qk, without the workspace: the K-mean partial sums go to a library-owned device
 * array of SAGE_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the device's first call until the
 * process ends.  Sizes whose sage_quantize_workspace_bytes(B, Hkv, Nk, d) exceeds it are refused
 * with WORKSPACE (8 MiB holds B * Hkv * ceil(Nk/256) * d <= 1,048,576, e.g. 64 key heads of
 * 32768 tokens at d = 128).  Every call on a GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialized by the caller.  Allocates and
 * frees nothing.  Errors: as sage_quantize_qk; HIP if the array's address cannot be obtained. */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
sage_status sage_quantize_qk_noalloc(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qk_quant* out,
                                     void* stream);

/* Bytes of workspace sage_prepare_v needs: per-chunk partial maxima of |V| (fp8) or fp64 partial
 * sums of V (FP16 with smooth_v); an FP16 call without smooth_v needs none.  Host only. */
size_t sage_prepare_v_workspace_bytes(int64_t B, int64_t H, int64_t Nk, int64_t d, sage_pv_dtype pv);

/* Step 2a (V preparation).  v bf16 or fp16 [B,H,Nk,d].
 *   SAGE_PV_FP16:     v_t = fp16 (round to nearest even) of V, 2-byte elements [B][H][d][Nk_pad];
 *                     v_scale is not used (may be NULL).  With v_mean non-NULL (smooth_v: the
 *                     sm80 INT8/FP16 kernel section's option for biased value tensors), v_mean fp32
 *                     [B][H][d] receives V's per-channel token mean (fp64 sum over the Nk tokens,
 *                     one rounding, as the K mean) and v_t holds fp16(fp32(V - v_mean)); the
 *                     attention adds v_mean back (pass it to sage_attn_fwd_prepared).
 *   SAGE_PV_FP8_E4M3: v_scale fp32 [B][H][d] = max_t |V[t,c]| / 448 (0 for an all-zero channel),
 *                     v_t = e4m3 (round to nearest even, saturating at +-448) of
 *                     V * (448 / max_t |V[t,c]|), bytes [B][H][d][Nk_pad].
 * (Per-channel FP8 V: section "sageattn_qk_int8_pv_fp8_cuda"; transposed V storage as v_fp4_t in the
 * FlashInfer API doc.)  Key order inside v_t is the order the PV MFMA consumes: fp16 stores each
 * group of 16 keys as [0-3, 8-11, 4-7, 12-15]; e4m3 stores key kb*32 + w of each group of 64 at
 * position ((w/4)%2)*32 + kb*16 + (w/8)*4 + w%4.  Pad keys (>= Nk) are zero.
 * Errors: INVALID_ARGUMENT (descriptor, null/misaligned v_t, fp8 without v_scale), UNSUPPORTED (also
 * v_mean with SAGE_PV_FP8_E4M3), WORKSPACE (fp8 or smooth_v with a workspace below
 * sage_prepare_v_workspace_bytes), HIP. */
sage_status sage_prepare_v(const sage_qkv_desc* v, sage_pv_dtype pv, void* v_t, float* v_scale, float* v_mean,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace the mask tile classification needs (0 when mask_h == 0).  Host only.
 * mask_h: 0 = no mask, 1 = mask broadcast over heads, H = one mask per head. */
size_t sage_mask_workspace_bytes(int64_t B, int64_t Nq, int64_t Nk, int64_t mask_h);

/* Bytes of workspace sage_attn_fwd needs: prepared V, the fp8 V scales or the smooth_v V mean,
 * sage_prepare_v's scratch and the mask tile classification.  Hkv = heads of V.  Host only. */
size_t sage_fwd_workspace_bytes(int64_t B, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, sage_pv_dtype pv,
                                int64_t mask_h);

/* Step 2 (attention, all in one): sage_prepare_v into the workspace, then sage_attn_fwd_prepared.
 *   qk: from sage_quantize_qk; v: bf16 or fp16 [B,Hkv,Nk,d].
 *   mask: NULL, or a mask of mask_dtype (see sage_mask_dtype), shape [B][mask_h][Nq][Nk],
 *         addressed as mask + b*mask_stride_b + h*mask_stride_h + i*mask_stride_q + j (element
 *         offsets; mask_h in {1, H}; mask_stride_h is ignored when mask_h == 1; mask_stride_b may
 *         be 0 to broadcast over the batch and mask_stride_q 0 to broadcast one row of keys over
 *         the queries, a key-padding mask [B,1|H,1,Nk]; otherwise mask_stride_q >= Nk; an fp32
 *         mask must be 4-byte aligned).  (Boolean mask
 *         semantics: Triton INT8/FP16 kernel examples section, where False entries are masked out.)
 *   causal: key j is visible to query i only if j <= i (top-left aligned).
 *   sm_scale: <= 0 selects 1/sqrt(d) (FlashInfer API doc, parameter sm_scale); NaN or +-inf is
 *        INVALID_ARGUMENT.
 *   smooth_v: nonzero subtracts V's per-channel token mean before the FP16 rounding of V and adds
 *        it back to O (see sage_prepare_v); SAGE_PV_FP16 only, else UNSUPPORTED.
 *   out: [B,H,Nq,d] of out_dtype (SAGE_BF16 or SAGE_FP16, rounded to nearest even, or SAGE_F32)
 *        addressed with out_stride_{b,h,n} (every row 16-byte aligned).
 *   lse: NULL, or fp32 [B][H][Nq] contiguous: natural-log log-sum-exp of the scaled, unsmoothed
 *        scores (lse_corr added back), for merging partial results ("return_lse" on the
 *        sageattn section and on "Utilize SageAttention for Distributed Inference").
 * The online softmax runs over sage_block_n() keys per tile in increasing key order; a row's
 * reference maximum moves when a tile's maximum exceeds it by more than sage_softmax_tau() (log2
 * units); P is rounded to fp16 (or to e4m3 of 448*p) against the reference maximum; the denominator
 * sums the unrounded fp32 p (sage_rowsum_rounded() = 0); O and l accumulate in fp32.  Keys j >= Nk are masked
 * before the softmax (FlashInfer API doc, parameter unpadded_k_len).  A row with no visible key
 * gets O = 0 and LSE = -inf.
 * Errors: INVALID_ARGUMENT (null pointers, shape/stride mismatch with qk, misalignment, unknown
 * dtype or mask_dtype, mask_h not in {1,H}, sm_scale not finite), UNSUPPORTED (d, pv, non-gfx950
 * device, or one head's prepared V past a 32-bit buffer range: Nk_pad * d * (2 for FP16 PV, 1 for
 * e4m3) >= 2^31, i.e. more than 8,388,480 keys per head at d = 128 with FP16 PV), WORKSPACE (too
 * small), HIP. */
sage_status sage_attn_fwd(const sage_qk_quant* qk, const sage_qkv_desc* v, const void* mask,
                          sage_mask_dtype mask_dtype, int64_t mask_h,
                          int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_q, int causal,
                          float sm_scale, sage_pv_dtype pv, int smooth_v, void* out, sage_dtype out_dtype,
                          int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Step 2b (attention on prepared V): mask tile classification (if a mask is given) and the
 * attention kernel.  v_t / v_scale / v_mean as written by sage_prepare_v for the same B, Hkv, Nk, d
 * and pv (v_mean NULL unless V was prepared with it).
 * workspace: at least sage_mask_workspace_bytes(B, Nq, Nk, mask_h) bytes (may be NULL without a
 * mask).  Other arguments and errors as for sage_attn_fwd. */
sage_status sage_attn_fwd_prepared(const sage_qk_quant* qk, const void* v_t, const float* v_scale,
                                   const float* v_mean, sage_pv_dtype pv,
                                   const void* mask, sage_mask_dtype mask_dtype, int64_t mask_h, int64_t mask_stride_b, int64_t mask_stride_h,
                                   int64_t mask_stride_q, int causal, float sm_scale, void* out,
                                   sage_dtype out_dtype, int64_t out_stride_b, int64_t out_stride_h,
                                   int64_t out_stride_n, float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Packed variable-length batches (sageattn_varlen section of the SageAttention docs digest:
 * packed tensors with cumulative sequence lengths, as flash_attn_varlen_func takes them).
 * Sequence b holds query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of a packed q of total_q rows
 * and key/value rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) of packed k / v of total_k rows;
 * cu_seqlens_* are device int32 arrays of B+1 nondecreasing entries starting at 0 (the library
 * reads them only on the device: lengths are clamped to [0, max] and rows to the packed buffers,
 * so malformed arrays give wrong results but no out-of-bounds access).  Each sequence is its own
 * attention problem: its own K mean, 64-token blocks from its first token, and causality aligned
 * at its first query and key.
 *   q, k, v: descriptors with B = number of sequences, N = the longest sequence (max_seqlen_q for
 *            q, max_seqlen_k for k and v), H heads, and the strides of one packed row
 *            (stride_n) and head (stride_h); stride_b is ignored.  Packed [total, H, d] has
 *            stride_n = H*d, stride_h = d.
 *   out (quantize): a sage_qk_quant for B sequences of Nq = max_seqlen_q, Nk = max_seqlen_k (the
 *            dense padded layout; rows past a sequence's end are zero).
 * Workspace and errors as for sage_quantize_qk; also INVALID_ARGUMENT for null cu_seqlens or a
 * negative / too large total. */
sage_status sage_quantize_qk_varlen(const sage_qkv_desc* q, const sage_qkv_desc* k, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k,
                                    const sage_qk_quant* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Attention of a packed variable-length batch (V preparation into the workspace included).
 *   qk: from sage_quantize_qk_varlen with the same cu_seqlens; v as k there.
 *   out: packed [total_q, H, d] of out_dtype, row stride out_stride_n and head stride
 *        out_stride_h (elements).
 *   lse: NULL, or fp32 [H][total_q] (the layout flash_attn_varlen_func uses for its LSE).
 * No mask.  A sequence without keys gives O = 0 and LSE = -inf for its rows.  Workspace: at least
 * sage_fwd_workspace_bytes(B, Hkv, max_seqlen_q, max_seqlen_k, d, pv, 0).  Errors as for
 * sage_attn_fwd. */
sage_status sage_attn_fwd_varlen(const sage_qk_quant* qk, const sage_qkv_desc* v, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k, int causal,
                                 float sm_scale, sage_pv_dtype pv, int smooth_v, void* out, sage_dtype out_dtype,
                                 int64_t out_stride_h, int64_t out_stride_n, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The two steps of sage_attn_fwd_varlen, for callers that reuse a prepared V: sage_prepare_v of a
 * packed V (v as for sage_attn_fwd_varlen; v_t / v_scale in the dense padded layout of B
 * sequences of max_seqlen_k keys, as sage_prepare_v writes for B, Hkv, max_seqlen_k), then the
 * attention on it.  Workspace of the first: sage_prepare_v_workspace_bytes(B, Hkv, max_seqlen_k, d,
 * pv); the second needs none.  Errors as for sage_attn_fwd_varlen. */
sage_status sage_prepare_v_varlen(const sage_qkv_desc* v, const int32_t* cu_seqlens_k, int64_t total_k,
                                  sage_pv_dtype pv, void* v_t, float* v_scale, float* v_mean, void* workspace,
                                  size_t workspace_bytes, void* stream);
sage_status sage_attn_fwd_prepared_varlen(const sage_qk_quant* qk, const void* v_t, const float* v_scale,
                                          const float* v_mean, sage_pv_dtype pv, const int32_t* cu_seqlens_q,
                                          const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k,
                                          int causal, float sm_scale, void* out, sage_dtype out_dtype,
                                          int64_t out_stride_h, int64_t out_stride_n, float* lse, void* stream);

/* Merge S partial attention results over disjoint key sets into the result over their union
 * (what the LSE output is for: "Utilize SageAttention for Distributed Inference" on the
 * SageAttention docs digest -- sequence parallelism, Ring Attention).  With part s covering the
 * keys K_s: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the softmax identity; a
 * part with LSE_s = -inf adds nothing and its O_s is not read; all -inf gives O = 0, LSE = -inf;
 * a NaN LSE_s makes the row's O and LSE NaN).  Computed in fp32.
 *   o_parts:   S contiguous [B][H][Nq][d] outputs of part_dtype (fp32 keeps the parts unrounded),
 *              16-byte aligned; e.g. sage_attn_fwd outputs over key slices.
 *   lse_parts: fp32 [S][B][H][Nq], natural log, as sage_attn_fwd writes them.
 *   out:       [B,H,Nq,d] of out_dtype with out_stride_{b,h,n} (elements; rows 16-byte aligned).
 *   lse:       NULL, or fp32 [B][H][Nq] contiguous.
 * d must be a positive multiple of 8 (at most 1024).  No workspace.
 * Errors: INVALID_ARGUMENT (sizes, null or misaligned pointers, dtypes), UNSUPPORTED (device), HIP. */
sage_status sage_merge_lse(int64_t S, int64_t B, int64_t H, int64_t Nq, int64_t d, const void* o_parts,
                           sage_dtype part_dtype, const float* lse_parts, void* out, sage_dtype out_dtype,
                           int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse,
                           void* stream);

/* Debug: the raw int32 scores acc[i,j] = sum_c q8[i,c]*k8[j,c] of query head (b,h) (and its key
 * head h / (H / Hkv)) for rows
 * [row0, row0+nrows) and keys [col0, col0+ncols), computed by the same tile code as
 * sage_attn_fwd.  out: int32 [nrows][ncols] device buffer.  The window must lie inside
 * [0,Nq_pad) x [0,Nk_pad). */
sage_status sage_debug_qk_int32(const sage_qk_quant* qk, int64_t b, int64_t h, int64_t row0, int64_t nrows,
                                int64_t col0, int64_t ncols, int32_t* out, void* stream);

/* Measurement aid: the shader clock.  Launches nblocks workgroups; load = 1: each keeps its SIMDs
 * busy with FP16 MFMAs and VALU work for iters loop trips (the clock under such a load); load = 0:
 * one wave each sleeps iters times (s_sleep 127, about 8k clocks) and adds no load, so that,
 * launched on a second stream beside other kernels, it measures the clock they run at.  The first
 * wave of workgroup i writes out[4i .. 4i+3] = shader clock counter (s_memtime) and 100 MHz
 * counter (s_memrealtime) at its start, then both at its end; the clock in MHz is
 * 100 * (out[4i+2] - out[4i]) / (out[4i+3] - out[4i+1]).  out: device buffer of 4 * nblocks
 * uint64 (8-byte aligned).  1 <= nblocks <= 65536, 1 <= iters <= 2^24, load 0 or 1.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP. */
sage_status sage_sclk_probe(int64_t nblocks, int64_t iters, int load, unsigned long long* out, void* stream);

/* Static description of a status code. Host only. */
const char* sage_status_string(sage_status s);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_MI355X_H */
