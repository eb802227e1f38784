/*
 * sage_oracle.c -- plain, slow CPU oracle for SageAttention-style quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or constant generator with the HIP library; it is written from the
 * method's description and from the number-format definitions, one step at a time.
 *
 * What it follows (page title, section):
 *  - "SageAttention docs digest (context7 llms.txt)", section "sageattn_qk_int8_pv_fp16_triton --
 *    Triton INT8/FP16 kernel (Ampere/Ada)": per-block INT8 quantization of Q and K, key smoothing
 *    (smooth_k), boolean mask, FP16 PV.
 *  - same page, section "SageAttention CUDA INT8/FP16 Kernel (Ampere sm80)": pv_accum_dtype="fp32"
 *    (FP16 products, FP32 accumulation), return_lse.
 *  - same page, section "sageattn_qk_int8_pv_fp8_cuda": INT8 Q/K with per-channel FP8 V.
 *  - same page, section "sageattn3_blackwell" usage: smoothing by the *global* mean of K over tokens.
 *  - same page, section "sageattn -- Auto-selecting attention kernel": sm_scale default, LSE shape.
 *  - "flashinfer.nvfp4_attention_sm120_fwd" (FlashInfer API doc), parameters sm_scale
 *    (default 1/sqrt(head_dim)), unpadded_k_len (keys at or beyond the logical length are masked
 *    before the softmax), out / lse buffers.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - quantization block = 64 tokens for Q and K; symmetric scale = absmax/127, codes in [-127,127];
 *    an all-zero block has scale 0 and codes 0;
 *  - every rounding is round-to-nearest-even (int8 codes, fp16, e4m3, bf16 or fp16 output);
 *  - Q, K and V are all bf16 or all fp16 ("in_fp16"); each value is decoded exactly to fp32 and
 *    the method then runs unchanged; the output has its own dtype (bf16 or fp16);
 *  - a float32 attention mask is additive: M_ij is added to the scaled score sm_scale * q_i.k_j
 *    (natural-log units) before the softmax, and -inf entries drop the key; a boolean (uint8)
 *    mask drops the keys whose entry is zero;
 *  - the K mean is summed in fp64 over all Nk tokens (mask and causality ignored), divided by Nk
 *    in fp64 and rounded once to fp32;
 *  - P for FP8 PV is quantized as e4m3(ps * p) with ps = 448 * 2^-tau (tau a whole number, see
 *    below: p <= 2^tau, so ps * p <= 448) and saturation, V per channel as
 *    e4m3(V * 448 / max_t |V|);
 *  - the softmax denominator l sums, per the lsum_rounded argument, either the unquantized fp32 p
 *    (0) or P as rounded for the PV product (1: the fp16 value, or e4m3(ps*p)/ps);
 *  - the online softmax runs over key tiles of BN keys in increasing key order.  Its reference
 *    maximum m starts at -inf and, after each tile, is replaced by the running maximum whenever
 *    that exceeds m by more than tau*ln(2) (tau = 0: the exact running maximum); p = exp(s - m)
 *    is then at most 2^tau.  The normalized result does not depend on tau; only where P is
 *    rounded does;
 *  - a row with no valid key gives O = 0 and LSE = -inf;
 *  - per_block_mean (the sageattn3_blackwell usage section's option): K is smoothed by the mean of
 *    its own 64-token quantization block (fp64 sum over the block's tokens, one rounding) instead
 *    of the global mean.  That shift differs between blocks, so it does not cancel in the softmax:
 *    the term sm_scale * (q_i . m_u) of key block u is added to each score (computed as
 *    fp32(sum_c fp64(Q_ic) * fp64(m_uc))), and the LSE needs no further correction;
 *  - smooth_v (FP16 PV only, as the pages tie it to the FP16 kernel): V's per-channel token mean is
 *    taken exactly like K's (fp64 sum over all Nk tokens, one rounding to fp32), V - mean is
 *    rounded once to fp32 and then to fp16, and the mean is added back to the normalized output
 *    of every row that has a visible key (exact, since the probabilities sum to one);
 *  - LSE is natural-log and adds back the smoothing shift sm_scale * (q_i . kmean), so it is the
 *    LSE of the unsmoothed scores;
 *  - non-finite inputs poison what depends on them and never vanish: the absolute maximum that
 *    sets a scale (a Q or K block, an FP8 V channel) is NaN when its group holds a NaN (IEEE
 *    754-2019 "maximum"), the scale is then NaN, and a code is 0 wherever x * (1/scale) is NaN
 *    (every code of a NaN or +inf scale).  Means are plain sums.  NaN scores leave the running
 *    maximum alone and give NaN probabilities; a tile is never skipped because nothing in the row
 *    was visible so far, and under causal masking a row's key loop ends at the last tile holding
 *    one of its keys.  A row with no visible key still gives O = 0 and LSE = -inf.
 *
 * Index arithmetic is 64-bit throughout.  Compile without -ffast-math and with -ffp-contract=off.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_QBLK 64 /* tokens per quantization block */

/* ------------------------------------------------------------------------------------------ */
/* Number formats, written from their definitions.                                            */
/* ------------------------------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormal unit 2^-24. */
float orc_f16_to_f32(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -24);
  else
    v = ldexp((double)(1024 + m), e - 25);
  return (float)(s ? -v : v);
}

/* An input element: bf16 (in_fp16 = 0) or IEEE binary16 (in_fp16 = 1) bits. */
static float orc_in_to_f32(uint16_t h, int in_fp16) { return in_fp16 ? orc_f16_to_f32(h) : orc_bf16_to_f32(h); }

/* fp32 -> binary16, round to nearest, ties to even; overflow to infinity. */
uint16_t orc_f32_to_f16(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return sign | 0x7e00;
  if (isinf(x)) return sign | 0x7c00;
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int E = e - 1; /* a in [2^E, 2^(E+1)) */
  if (E < -14) {
    /* subnormal range: count units of 2^-24; a result of 1024 is the smallest normal */
    double r = nearbyint(ldexp(a, 24));
    return sign | (uint16_t)r;
  }
  double r = nearbyint(ldexp(a, 10 - E)); /* 11 significant bits, in [1024, 2048] */
  if (r == 2048.0) {
    r = 1024.0;
    E += 1;
  }
  if (E > 15) return sign | 0x7c00;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0);
}

/* fp32 -> bfloat16 (8 significant bits, binary32 exponent range), round to nearest even. */
uint16_t orc_f32_to_bf16(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return sign | 0x7fc0;
  if (isinf(x)) return sign | 0x7f80;
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < -126) {
    double r = nearbyint(ldexp(a, 133)); /* subnormal unit 2^-133; 128 = smallest normal */
    return sign | (uint16_t)r;
  }
  double r = nearbyint(ldexp(a, 7 - E)); /* in [128, 256] */
  if (r == 256.0) {
    r = 128.0;
    E += 1;
  }
  if (E > 127) return sign | 0x7f80;
  return sign | (uint16_t)((E + 127) << 7) | (uint16_t)(r - 128.0);
}

/* OCP 8-bit floating point, E4M3 ("fn" flavour): bias 7, no infinities, S.1111.111 = NaN,
 * largest finite 448 = 1.75 * 2^8, subnormal unit 2^-9. */
float orc_e4m3_to_f32(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (float)(s ? -v : v);
}

/* fp32 -> E4M3, round to nearest even, saturating: finite magnitudes that would round past 448
 * (and infinities) give +-448; NaN gives NaN. */
uint8_t orc_f32_to_e4m3(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return sign | 0x7f;
  if (isinf(x)) return sign | 0x7e;
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < -6) {
    double r = nearbyint(ldexp(a, 9)); /* units of 2^-9; 8 = smallest normal 2^-6 */
    return sign | (uint8_t)r;
  }
  double r = nearbyint(ldexp(a, 3 - E)); /* 4 significant bits, in [8, 16] */
  if (r == 16.0) {
    r = 8.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && r > 14.0)) return sign | 0x7e;
  return sign | (uint8_t)(((E + 7) << 3) | ((int)r - 8));
}

/* Vector forms for the codec tests. */
void orc_f32_to_f16_n(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_f16(x[i]);
}
void orc_f16_to_f32_n(const uint16_t* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f16_to_f32(x[i]);
}
void orc_f32_to_bf16_n(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(x[i]);
}
void orc_f32_to_e4m3_n(const float* x, uint8_t* y, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_e4m3(x[i]);
}
void orc_e4m3_to_f32_n(const uint8_t* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_e4m3_to_f32(x[i]);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* Step 1: K mean over tokens (smooth_k).                                                     */
/* K is bf16 or fp16 (in_fp16) [B][H][Nk][d]; kmean is fp32 [B][H][d].                       */
/* ------------------------------------------------------------------------------------------ */
void orc_kmean(const uint16_t* K, int in_fp16, int64_t B, int64_t H, int64_t Nk, int64_t d, float* kmean) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t c = 0; c < d; ++c) {
      double s = 0.0;
      for (int64_t t = 0; t < Nk; ++t) s += (double)orc_in_to_f32(K[(bh * Nk + t) * d + c], in_fp16);
      kmean[bh * d + c] = (float)(s / (double)Nk);
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Step 2: per-block symmetric INT8 quantization of an fp32 matrix X [N][d] (one head).       */
/* Block u covers rows [64u, min(64u+64, N)) and all d channels.                              */
/* x8 gets N_pad rows (rows >= N are zero); scale gets ceil(N/64) entries.                    */
/* ------------------------------------------------------------------------------------------ */
/* Running absolute maximum with IEEE 754-2019 "maximum" semantics: once a NaN is seen the
 * maximum is NaN. */
static float absmax_fold(float m, float x) {
  float a = fabsf(x);
  if (isnan(m) || isnan(a)) return NAN;
  return a > m ? a : m;
}

/* INT8 code of a scaled value y: round to nearest even, clamp to [-127, 127]; NaN gives 0. */
static int8_t int8_code(float y) {
  if (isnan(y)) return 0;
  float q = nearbyintf(y); /* ties to even */
  if (q > 127.0f) q = 127.0f;
  if (q < -127.0f) q = -127.0f;
  return (int8_t)q;
}

static void quantize_blocks(const float* X, int64_t N, int64_t N_pad, int64_t d, int8_t* x8, float* scale) {
  int64_t nblk = (N + ORC_QBLK - 1) / ORC_QBLK;
  for (int64_t u = 0; u < nblk; ++u) {
    int64_t r0 = u * ORC_QBLK, r1 = r0 + ORC_QBLK < N ? r0 + ORC_QBLK : N;
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = 0; c < d; ++c) amax = absmax_fold(amax, X[r * d + c]);
    float sc = 0.0f, inv = 0.0f;
    if (amax != 0.0f) { /* NaN and +inf included: scale NaN / +inf, inverse NaN / 0 */
      sc = amax / 127.0f; /* IEEE binary32 division */
      inv = 127.0f / amax;
    }
    scale[u] = sc;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = 0; c < d; ++c) x8[r * d + c] = int8_code(X[r * d + c] * inv); /* one rounding */
  }
  memset(x8 + N * d, 0, (size_t)((N_pad - N) * d));
}

/* Per-block K means for per_block_mean: bmean [B][H][ceil(Nk/64)][d], block u's mean over its
 * tokens [64u, min(64u+64, Nk)), fp64 sum rounded once to fp32. */
void orc_block_mean(const uint16_t* K, int in_fp16, int64_t B, int64_t H, int64_t Nk, int64_t d, float* bmean) {
  int64_t nbk = (Nk + ORC_QBLK - 1) / ORC_QBLK;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh)
    for (int64_t u = 0; u < nbk; ++u) {
      int64_t t0 = u * ORC_QBLK, t1 = t0 + ORC_QBLK < Nk ? t0 + ORC_QBLK : Nk;
      for (int64_t c = 0; c < d; ++c) {
        double s = 0.0;
        for (int64_t t = t0; t < t1; ++t) s += (double)orc_in_to_f32(K[(bh * Nk + t) * d + c], in_fp16);
        bmean[(bh * nbk + u) * d + c] = (float)(s / (double)(t1 - t0));
      }
    }
}

/* Q [B][H][Nq][d], K [B][Hkv][Nk][d], both bf16 or both fp16 (in_fp16); kmean fp32 [B][Hkv][d]
 * (from orc_kmean).
 * Hkv divides H; query head h reads key/value head h / (H / Hkv) (group-query attention).
 * Outputs: q8 [B][H][Nq_pad][d], k8 [B][Hkv][Nk_pad][d], qs [B][H][ceil(Nq/64)],
 *          ks [B][Hkv][ceil(Nk/64)], corr [B][H][Nq] = fp32(sum_c fp64(Q_ic) * fp64(kmean_c)) with
 *          the K mean of the query head's key/value head.
 * K is smoothed as fp32(K - kmean) (one rounding) before quantizing.
 * per_block != 0: kmean holds the per-block means [B][Hkv][ceil(Nk/64)][d] (orc_block_mean); K is
 * smoothed by its block's mean, corr is 0, and corr_blk [B][H][ceil(Nk/64)][Nq] receives the
 * score terms fp32(sum_c fp64(Q_ic) * fp64(m_uc)) of the query head's key/value head. */
void orc_quant_qk(const uint16_t* Q, const uint16_t* K, int in_fp16, const float* kmean, int per_block, int64_t B,
                  int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t Nq_pad, int64_t Nk_pad, int8_t* q8,
                  int8_t* k8, float* qs, float* ks, float* corr, float* corr_blk) {
  int64_t nbq = (Nq + ORC_QBLK - 1) / ORC_QBLK, nbk = (Nk + ORC_QBLK - 1) / ORC_QBLK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * Hkv; ++bh) {
    float* xk = (float*)malloc((size_t)(Nk * d) * sizeof(float));
    for (int64_t t = 0; t < Nk; ++t) {
      const float* km = per_block ? kmean + (bh * nbk + t / ORC_QBLK) * d : kmean + bh * d;
      for (int64_t c = 0; c < d; ++c) xk[t * d + c] = orc_in_to_f32(K[(bh * Nk + t) * d + c], in_fp16) - km[c];
    }
    quantize_blocks(xk, Nk, Nk_pad, d, k8 + bh * Nk_pad * d, ks + bh * nbk);
    free(xk);
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    float* xq = (float*)malloc((size_t)(Nq * d) * sizeof(float));
    const int64_t bhk = (bh / H) * Hkv + (bh % H) / (H / Hkv);
    for (int64_t i = 0; i < Nq * d; ++i) xq[i] = orc_in_to_f32(Q[bh * Nq * d + i], in_fp16);
    quantize_blocks(xq, Nq, Nq_pad, d, q8 + bh * Nq_pad * d, qs + bh * nbq);
    for (int64_t i = 0; i < Nq; ++i) {
      if (per_block) {
        corr[bh * Nq + i] = 0.0f;
        for (int64_t u = 0; u < nbk; ++u) {
          const float* km = kmean + (bhk * nbk + u) * d;
          double s = 0.0;
          for (int64_t c = 0; c < d; ++c) s += (double)xq[i * d + c] * (double)km[c];
          corr_blk[(bh * nbk + u) * Nq + i] = (float)s;
        }
      } else {
        const float* km = kmean + bhk * d;
        double s = 0.0;
        for (int64_t c = 0; c < d; ++c) s += (double)xq[i * d + c] * (double)km[c];
        corr[bh * Nq + i] = (float)s;
      }
    }
    free(xq);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Step 3: V preparation.  Output keeps V's own layout [B][H][Nk][d].                         */
/* V is bf16 or fp16 (in_fp16).                                                               */
/* fp16: vhat = fp16_rne(V) (the identity for fp16 V); with smooth_v (vmean != NULL, from      */
/*       orc_kmean of V) vhat = fp16_rne(fp32(V - vmean)).                                    */
/* fp8:  vmax_c = max_t |V_tc|; vs_c = fp32(vmax_c / 448); vinv_c = fp32(448 / vmax_c)        */
/*       (0 when vmax_c = 0); vhat = e4m3_rne_sat(fp32(V * vinv_c)), 0 where that product is    */
/*       NaN.  vmax_c is NaN when the channel holds a NaN (as for the INT8 blocks).             */
/* ------------------------------------------------------------------------------------------ */
void orc_prep_v_fp16(const uint16_t* V, int in_fp16, int64_t B, int64_t H, int64_t Nk, int64_t d,
                     const float* vmean, uint16_t* vhat) {
  int64_t n = B * H * Nk * d;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float x = orc_in_to_f32(V[i], in_fp16);
    if (vmean) x = x - vmean[(i / (Nk * d)) * d + i % d]; /* one fp32 rounding */
    vhat[i] = orc_f32_to_f16(x);
  }
}

void orc_prep_v_fp8(const uint16_t* V, int in_fp16, int64_t B, int64_t H, int64_t Nk, int64_t d, uint8_t* vhat, float* vs) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t c = 0; c < d; ++c) {
      float vmax = 0.0f;
      for (int64_t t = 0; t < Nk; ++t) vmax = absmax_fold(vmax, orc_in_to_f32(V[(bh * Nk + t) * d + c], in_fp16));
      float sc = 0.0f, inv = 0.0f;
      if (vmax != 0.0f) {
        sc = vmax / 448.0f;
        inv = 448.0f / vmax;
      }
      vs[bh * d + c] = sc;
      for (int64_t t = 0; t < Nk; ++t) {
        int64_t idx = (bh * Nk + t) * d + c;
        float y = orc_in_to_f32(V[idx], in_fp16) * inv;
        vhat[idx] = isnan(y) ? 0 : orc_f32_to_e4m3(y);
      }
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Step 4: exact int32 scores acc_ij = sum_c q8_ic * k8_jc for a window of one head.          */
/* q8h = q8 + bh*Nq_pad*d, k8h = k8 + bh*Nk_pad*d; out is [nrows][ncols].                     */
/* ------------------------------------------------------------------------------------------ */
void orc_scores(const int8_t* q8h, const int8_t* k8h, int64_t d, int64_t row0, int64_t nrows, int64_t col0,
                int64_t ncols, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    const int8_t* q = q8h + (row0 + r) * d;
    for (int64_t j = 0; j < ncols; ++j) {
      const int8_t* k = k8h + (col0 + j) * d;
      int32_t acc = 0;
      for (int64_t c = 0; c < d; ++c) acc += (int32_t)q[c] * (int32_t)k[c];
      out[r * ncols + j] = acc;
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Step 5: quantized attention forward (the emulation the GPU path must reproduce).           */
/*                                                                                            */
/* rows: flattened row ids (b*H + h)*Nq + i to evaluate; NULL = all B*H*Nq rows in order.     */
/* mask: [B][mask_h][Nq][Nk]; mask_h is 1 (broadcast over heads) or H; NULL means no mask.     */
/*       mask_f32 = 0: uint8, nonzero = attend; mask_f32 = 1: fp32 added to the scaled score  */
/*       (natural-log units), -inf = drop.                                                     */
/* vhat: fp16 bits (pv_fp8 = 0) or e4m3 bytes (pv_fp8 = 1), layout [B][H][Nk][d].             */
/* vs:   per-channel V scale [B][H][d] (fp8 only).                                            */
/* vmean: smooth_v's per-channel V mean [B][Hkv][d], added back to the output, or NULL.        */
/* corr_blk: per_block_mean's score terms [B][H][ceil(Nk/64)][Nq] (orc_quant_qk), or NULL.      */
/* BN: keys per online-softmax tile; tau: lazy-maximum threshold in log2 units (0 = exact).    */
/* lsum_rounded: 0 = l sums the fp32 p, 1 = l sums P as rounded for PV.                       */
/* Outputs per requested row: o32 [nrows][d] (fp32 O before the output rounding, may be NULL),*/
/* o16 [nrows][d] (bf16 bits, or fp16 bits if out_fp16), lse [nrows] (natural log, fp32).     */
/* ------------------------------------------------------------------------------------------ */
void orc_attn_qe(const int8_t* q8, const int8_t* k8, const float* qs, const float* ks, const float* corr,
                 const float* corr_blk,
                 const void* vhat, const float* vs, const float* vmean, int pv_fp8, const void* mask, int mask_f32,
                 int64_t mask_h,
                 int causal,
                 float sm_scale, int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t Nq_pad,
                 int64_t Nk_pad, int64_t BN, double tau, int lsum_rounded, const int64_t* rows, int64_t nrows,
                 float* o32, int out_fp16, uint16_t* o16, float* lse) {
  int64_t nbq = (Nq + ORC_QBLK - 1) / ORC_QBLK, nbk = (Nk + ORC_QBLK - 1) / ORC_QBLK;
  const float ps = (float)ldexp(448.0, -(int)tau); /* e4m3 P scale (fp8: tau is a whole number) */
  if (rows == NULL) nrows = B * H * Nq;
#pragma omp parallel
  {
    float* o = (float*)malloc((size_t)d * sizeof(float));
    float* s = (float*)malloc((size_t)BN * sizeof(float));
    float* pq = (float*)malloc((size_t)BN * sizeof(float));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t rid = rows ? rows[r] : r;
      int64_t bh = rid / Nq, i = rid % Nq, b = bh / H, h = bh % H;
      int64_t bhk = b * Hkv + h / (H / Hkv); /* key/value head of this query head */
      const int8_t* q = q8 + (bh * Nq_pad + i) * d;
      const int8_t* kh = k8 + bhk * Nk_pad * d;
      const int64_t moff = ((b * mask_h + (mask_h == 1 ? 0 : h)) * Nq + i) * Nk;
      const uint8_t* mrow = (mask && !mask_f32) ? (const uint8_t*)mask + moff : NULL;
      const float* madd = (mask && mask_f32) ? (const float*)mask + moff : NULL;
      float qscale = qs[bh * nbq + i / ORC_QBLK];
      float m = -INFINITY, l = 0.0f;
      for (int64_t c = 0; c < d; ++c) o[c] = 0.0f;
      for (int64_t j0 = 0; j0 < Nk && !(causal && j0 > i); j0 += BN) {
        int64_t j1 = j0 + BN < Nk ? j0 + BN : Nk;
        /* scores of this key tile */
        float tmax = -INFINITY;
        for (int64_t j = j0; j < j1; ++j) {
          int valid = 1;
          if (causal && j > i) valid = 0;
          if (mrow && mrow[j] == 0) valid = 0;
          if (madd && madd[j] == -INFINITY) valid = 0;
          if (!valid) {
            s[j - j0] = -INFINITY;
            continue;
          }
          const int8_t* k = kh + j * d;
          int32_t acc = 0;
          for (int64_t c = 0; c < d; ++c) acc += (int32_t)q[c] * (int32_t)k[c];
          float cst = (qscale * ks[bhk * nbk + j / ORC_QBLK]) * sm_scale;
          s[j - j0] = (float)acc * cst;
          if (corr_blk) s[j - j0] += sm_scale * corr_blk[(bh * nbk + j / ORC_QBLK) * Nq + i]; /* per-block mean */
          if (madd) s[j - j0] += madd[j]; /* additive mask, natural-log units */
          if (s[j - j0] > tmax) tmax = s[j - j0];
        }
        /* NaN scores do not take part in the maximum (tmax skips them); with nothing finite seen so
         * far mnew stays -inf, masked keys get p = 0 and NaN scores p = NaN */
        float mnew = m;
        if (m == -INFINITY || (double)tmax > (double)m + tau * M_LN2) mnew = m > tmax ? m : tmax;
        float alpha = (m == -INFINITY) ? 0.0f : (float)exp((double)(m - mnew));
        float psum = 0.0f;
        for (int64_t j = j0; j < j1; ++j) {
          float p = (s[j - j0] == -INFINITY) ? 0.0f : (float)exp((double)(s[j - j0] - mnew));
          if (pv_fp8)
            pq[j - j0] = orc_e4m3_to_f32(orc_f32_to_e4m3(ps * p));
          else
            pq[j - j0] = orc_f16_to_f32(orc_f32_to_f16(p));
          if (!lsum_rounded)
            psum += p;
          else
            psum += pv_fp8 ? pq[j - j0] / ps : pq[j - j0];
        }
        l = alpha * l + psum;
        for (int64_t c = 0; c < d; ++c) {
          float acc = alpha * o[c];
          for (int64_t j = j0; j < j1; ++j) {
            int64_t vidx = (bhk * Nk + j) * d + c;
            float v = pv_fp8 ? orc_e4m3_to_f32(((const uint8_t*)vhat)[vidx])
                             : orc_f16_to_f32(((const uint16_t*)vhat)[vidx]);
            acc += pq[j - j0] * v;
          }
          o[c] = acc;
        }
        m = mnew;
      }
      for (int64_t c = 0; c < d; ++c) {
        float out;
        if (l == 0.0f)
          out = 0.0f;
        else if (pv_fp8)
          out = (float)((double)o[c] * (double)vs[bhk * d + c] / ((double)ps * (double)l));
        else
          out = o[c] / l;
        if (vmean && l != 0.0f) out = out + vmean[bhk * d + c]; /* smooth_v: add the mean back */
        if (o32) o32[r * d + c] = out;
        if (o16) o16[r * d + c] = out_fp16 ? orc_f32_to_f16(out) : orc_f32_to_bf16(out);
      }
      if (lse) {
        if (l == 0.0f)
          lse[r] = -INFINITY;
        else
          lse[r] = (float)((double)m + log((double)l) + (double)sm_scale * (double)corr[bh * Nq + i]);
      }
    }
    free(o);
    free(s);
    free(pq);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Exact attention in fp64 on the original bf16 or fp16 inputs: no smoothing, no quantization. */
/* s_ij = sm_scale * sum_c Q_ic K_jc (+ M_ij for an fp32 mask); invalid entries -inf;         */
/* two-pass softmax; O = P V;                                                                 */
/* LSE_i = log sum_j exp(s_ij).  A row with no valid key gives O = 0, LSE = -inf; a row with  */
/* a NaN score (a visible key) gives O = NaN and LSE = NaN.                                   */
/* ------------------------------------------------------------------------------------------ */
void orc_attn_ex(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int in_fp16, const void* mask, int mask_f32,
                 int64_t mask_h, int causal, double sm_scale, int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                 const int64_t* rows, int64_t nrows, double* out, double* lse) {
  if (rows == NULL) nrows = B * H * Nq;
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)Nk * sizeof(double));
    double* q = (double*)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t rid = rows ? rows[r] : r;
      int64_t bh = rid / Nq, i = rid % Nq, b = bh / H, h = bh % H;
      int64_t bhk = b * Hkv + h / (H / Hkv); /* key/value head of this query head */
      const int64_t moff = ((b * mask_h + (mask_h == 1 ? 0 : h)) * Nq + i) * Nk;
      const uint8_t* mrow = (mask && !mask_f32) ? (const uint8_t*)mask + moff : NULL;
      const float* madd = (mask && mask_f32) ? (const float*)mask + moff : NULL;
      for (int64_t c = 0; c < d; ++c) q[c] = (double)orc_in_to_f32(Q[(bh * Nq + i) * d + c], in_fp16);
      double mx = -INFINITY;
      int has_nan = 0;
      for (int64_t j = 0; j < Nk; ++j) {
        if ((causal && j > i) || (mrow && mrow[j] == 0) || (madd && madd[j] == -INFINITY)) {
          s[j] = -INFINITY;
          continue;
        }
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += q[c] * (double)orc_in_to_f32(K[(bhk * Nk + j) * d + c], in_fp16);
        s[j] = sm_scale * acc;
        if (madd) s[j] += (double)madd[j];
        if (isnan(s[j])) has_nan = 1;
        if (s[j] > mx) mx = s[j];
      }
      double* o = out + r * d;
      for (int64_t c = 0; c < d; ++c) o[c] = has_nan ? NAN : 0.0;
      if (has_nan || mx == -INFINITY) {
        if (lse) lse[r] = has_nan ? NAN : -INFINITY;
        continue;
      }
      double den = 0.0;
      for (int64_t j = 0; j < Nk; ++j) {
        if (s[j] == -INFINITY) continue;
        double p = exp(s[j] - mx);
        den += p;
        for (int64_t c = 0; c < d; ++c) o[c] += p * (double)orc_in_to_f32(V[(bhk * Nk + j) * d + c], in_fp16);
      }
      for (int64_t c = 0; c < d; ++c) o[c] /= den;
      if (lse) lse[r] = mx + log(den);
    }
    free(s);
    free(q);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Merging partial attention results over disjoint key sets (the use of the LSE output on    */
/* the docs digest, "Utilize SageAttention for Distributed Inference": sequence parallelism,  */
/* Ring Attention).  Written from the softmax's definition: if part s covers keys K_s with    */
/* O_s = sum_{j in K_s} e^{s_j} v_j / sum_{j in K_s} e^{s_j} and LSE_s = log sum_{j in K_s}    */
/* e^{s_j}, then over the union LSE = log sum_s e^{LSE_s} and O = sum_s e^{LSE_s - LSE} O_s.  */
/* A part with LSE_s = -inf (no visible key) contributes nothing (its O_s is not read); if    */
/* every part has -inf, O = 0 and LSE = -inf.  A NaN LSE_s makes the row's O and LSE NaN.     */
/* o_parts [S][R][d] (fp32), lse_parts [S][R]; out [R][d] and lse [R] in fp64.                */
/* ------------------------------------------------------------------------------------------ */
void orc_merge_lse(const float* o_parts, const float* lse_parts, int64_t S, int64_t R, int64_t d, double* out,
                   double* lse) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    double m = -INFINITY;
    int has_nan = 0;
    for (int64_t s = 0; s < S; ++s) {
      if (isnan(lse_parts[s * R + r])) has_nan = 1;
      if ((double)lse_parts[s * R + r] > m) m = (double)lse_parts[s * R + r];
    }
    for (int64_t c = 0; c < d; ++c) out[r * d + c] = has_nan ? NAN : 0.0;
    if (has_nan || m == -INFINITY) {
      lse[r] = has_nan ? NAN : -INFINITY;
      continue;
    }
    double tot = 0.0;
    for (int64_t s = 0; s < S; ++s) tot += exp((double)lse_parts[s * R + r] - m);
    double L = m + log(tot);
    for (int64_t s = 0; s < S; ++s) {
      if (lse_parts[s * R + r] == -INFINITY) continue; /* a part without visible keys */
      double w = exp((double)lse_parts[s * R + r] - L);
      for (int64_t c = 0; c < d; ++c) out[r * d + c] += w * (double)o_parts[(s * R + r) * d + c];
    }
    lse[r] = L;
  }
}
