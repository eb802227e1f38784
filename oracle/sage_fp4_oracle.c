/*
 * sage_fp4_oracle.c -- plain, slow CPU oracle for the FP4 microscaling attention method.
 *
 * TEST INFRASTRUCTURE ONLY, like sage_oracle.c (it is linked into the same oracle library and
 * uses that file's number-format codecs and K mean).  Nothing on the product path links, loads or
 * calls it, and it shares no code with the HIP library.
 *
 * What it follows (page title, section):
 *  - "SageAttention docs digest (context7 llms.txt)", sections "FP4 Attention for Blackwell GPUs"
 *    and "sageattn3_blackwell": microscaling FP4 quantization of Q, K and V; per_block_mean
 *    smoothing (on by default) or smoothing by the global mean; causal attention.
 *  - "flashinfer.nvfp4_attention_sm120_fwd" (FlashInfer API doc): packed FP4 Q and K with one
 *    8-bit scale per vector of elements; V stored transposed (its scales run along the tokens);
 *    a compact FP32 correction term with one row per 128-token Q block; sm_scale defaulting to
 *    1/sqrt(head_dim); keys at or beyond the logical length masked before the softmax; an
 *    optional LSE.
 *  - The number formats: OCP Microscaling Formats (MX) Specification v1.0 -- FP4 E2M1 elements
 *    (1 sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 *    and E8M0 block scales (2^(code - 127)) over blocks of 32 elements.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - the element format is MX FP4: e2m1 codes, one E8M0 scale per 32 consecutive elements --
 *    along the head dimension for Q and K, along the tokens for V;
 *  - the block scale follows the MX specification's conversion: X = floor(log2(amax)) - 2 (the
 *    largest element's exponent minus e2m1's largest exponent), clamped to [-127, 127]; an
 *    all-zero block takes X = -127; elements are x * 2^-X rounded to nearest e2m1 with ties to the
 *    even code and saturated at +-6; a negative value that rounds to zero keeps its sign bit;
 *  - K is smoothed by its global token mean, exactly as in the INT8 method (fp64 sums, one
 *    rounding; it cancels in the softmax and the LSE adds sm_scale * q_i . kmean back);
 *  - Q is smoothed by the mean of its own 128-token block (per_block_mean) or by its global token
 *    mean (fp64 sums over the valid tokens, one rounding to fp32); the subtracted part's scores,
 *    qk_corr[u][j] = qmean_u . Ktilde_j with Ktilde = fp32(K - kmean), are computed in fp64 from
 *    the unquantized values, rounded to fp32 and added to every score of block u's rows;
 *  - P is not named among the FP4 tensors: it is quantized to e4m3 as in the FP8 PV method, with
 *    the online schedule a parameter: over key tiles of BN keys the reference maximum m moves only
 *    when a tile's maximum exceeds it by more than tau log2 units (tau = 0: the exact running
 *    maximum), p = exp(s - m) <= 2^tau, and P = e4m3(448 * 2^-tau * p) keeps P <= 448; l sums the
 *    unquantized fp32 p.  The normalized result does not depend on tau, only where P is rounded;
 *  - scores are S_ij = fp32(sum_c deq(q)_ic deq(k)_jc + qk_corr) with the sum in fp64 (every
 *    product of two dequantized values is exact), then s = S * sm_scale in fp32.
 *
 * Index arithmetic is 64-bit throughout.  Compile without -ffast-math and with -ffp-contract=off.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* from sage_oracle.c (the same oracle library) */
float orc_bf16_to_f32(uint16_t h);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float x);
uint16_t orc_f32_to_bf16(float x);
float orc_e4m3_to_f32(uint8_t c);
uint8_t orc_f32_to_e4m3(float x);
void orc_kmean(const uint16_t* K, int in_fp16, int64_t B, int64_t H, int64_t Nk, int64_t d, float* kmean);

#define ORC_MX 32     /* elements per MX block */
#define ORC_QMBLK 128 /* tokens per Q smoothing block */

static float in_f32(uint16_t h, int in_fp16) { return in_fp16 ? orc_f16_to_f32(h) : orc_bf16_to_f32(h); }

/* ------------------------------------------------------------------------------------------ */
/* FP4 E2M1 and E8M0, from the MX specification's format definitions.                         */
/* ------------------------------------------------------------------------------------------ */
static const double ORC_E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float orc_e2m1_to_f32(uint8_t code) {
  double v = ORC_E2M1_MAG[code & 7];
  return (float)((code & 8) ? -v : v);
}

/* Nearest magnitude by search over the eight magnitudes (exact in fp64); a tie goes to the even
 * code; beyond 6 the largest magnitude.  The sign bit is the input's. */
uint8_t orc_f32_to_e2m1(float y) {
  double a = fabs((double)y);
  int best = 0;
  double bd = INFINITY;
  for (int k = 0; k < 8; ++k) {
    double dist = fabs(a - ORC_E2M1_MAG[k]);
    if (dist < bd || (dist == bd && (k & 1) == 0)) {
      bd = dist;
      best = k;
    }
  }
  return (uint8_t)(best | (signbit(y) ? 8 : 0));
}

/* Shared exponent X of a block with largest magnitude amax. */
int orc_mx_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int E;
  frexp((double)amax, &E); /* amax = m * 2^E, m in [0.5, 1): floor(log2(amax)) = E - 1 */
  int X = (E - 1) - 2;     /* e2m1's largest exponent is 2 (6 = 1.5 * 2^2) */
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  return X;
}

/* One MX block: n <= 32 elements x[k * xs] -> codes c[k * cs]; returns the E8M0 byte X + 127.
 * Elements past n (a ragged last block) are absent: they neither enter amax nor get codes. */
static uint8_t mx_block(const float* x, int64_t xs, int64_t n, uint8_t* c, int64_t cs) {
  float amax = 0.0f;
  for (int64_t k = 0; k < n; ++k)
    if (fabsf(x[k * xs]) > amax) amax = fabsf(x[k * xs]);
  int X = orc_mx_exp(amax);
  for (int64_t k = 0; k < n; ++k) c[k * cs] = orc_f32_to_e2m1((float)ldexp((double)x[k * xs], -X));
  return (uint8_t)(X + 127);
}

void orc_mx_quant_n(const float* x, int64_t nblk, int64_t n, uint8_t* codes, uint8_t* e8) {
  for (int64_t b = 0; b < nblk; ++b) {
    int64_t m = n - b * ORC_MX < ORC_MX ? n - b * ORC_MX : ORC_MX;
    e8[b] = mx_block(x + b * ORC_MX, 1, m, codes + b * ORC_MX, 1);
  }
}

static double deq(uint8_t code, uint8_t e8) { return ldexp((double)orc_e2m1_to_f32(code), (int)e8 - 127); }

/* ------------------------------------------------------------------------------------------ */
/* Quantization of Q and K with the two smoothings.                                           */
/*  kmean   [B][Hkv][d]      global K means (orc_kmean), input                                 */
/*  qmean   [B][H][nqm][d]   Q means: nqm = ceil(Nq/128) blocks (per_block) or 1 (global)      */
/*  q4 [B][H][Nq][d], qe [B][H][Nq][d/32]; k4 [B][Hkv][Nk][d], ke [B][Hkv][Nk][d/32]            */
/*  qk_corr [B][H][nqm][Nk]  fp32(sum_c fp64(qmean_uc) * fp64(Ktilde_jc))                      */
/*  lse_corr [B][H][Nq]      fp32(sum_c fp64(Q_ic) * fp64(kmean_c))                            */
/* ------------------------------------------------------------------------------------------ */
void orc_fp4_quant_qk(const uint16_t* Q, const uint16_t* K, int in_fp16, int per_block, int64_t B, int64_t H,
                      int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, const float* kmean, float* qmean, uint8_t* q4,
                      uint8_t* qe, uint8_t* k4, uint8_t* ke, float* qk_corr, float* lse_corr) {
  const int64_t nqm = per_block ? (Nq + ORC_QMBLK - 1) / ORC_QMBLK : 1, nb = d / ORC_MX;
  /* Q means */
  if (per_block) {
#pragma omp parallel for schedule(static)
    for (int64_t bu = 0; bu < B * H * nqm; ++bu) {
      int64_t bh = bu / nqm, u = bu % nqm;
      int64_t t0 = u * ORC_QMBLK, t1 = t0 + ORC_QMBLK < Nq ? t0 + ORC_QMBLK : Nq;
      for (int64_t c = 0; c < d; ++c) {
        double s = 0.0;
        for (int64_t t = t0; t < t1; ++t) s += (double)in_f32(Q[(bh * Nq + t) * d + c], in_fp16);
        qmean[bu * d + c] = (float)(s / (double)(t1 - t0));
      }
    }
  } else {
    orc_kmean(Q, in_fp16, B, H, Nq, d, qmean); /* the same fp64 token mean, over all Nq tokens */
  }
  /* Q: smoothed, MX-quantized per 32 channels; the LSE shift of K's smoothing */
#pragma omp parallel
  {
    float* x = (float*)malloc((size_t)d * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < B * H * Nq; ++r) {
      int64_t bh = r / Nq, i = r % Nq, b = bh / H, h = bh % H;
      int64_t bhk = b * Hkv + h / (H / Hkv);
      const float* qm = qmean + (bh * nqm + (per_block ? i / ORC_QMBLK : 0)) * d;
      double lc = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        float q = in_f32(Q[r * d + c], in_fp16);
        x[c] = q - qm[c];
        lc += (double)q * (double)kmean[bhk * d + c];
      }
      lse_corr[r] = (float)lc;
      orc_mx_quant_n(x, nb, d, q4 + r * d, qe + r * nb);
    }
    free(x);
  }
  /* K: smoothed by the global mean, MX-quantized per 32 channels */
#pragma omp parallel
  {
    float* x = (float*)malloc((size_t)d * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < B * Hkv * Nk; ++r) {
      int64_t bhk = r / Nk;
      for (int64_t c = 0; c < d; ++c) x[c] = in_f32(K[r * d + c], in_fp16) - kmean[bhk * d + c];
      orc_mx_quant_n(x, nb, d, k4 + r * d, ke + r * nb);
    }
    free(x);
  }
  /* the Q means' share of the scores, one row of Nk per Q block (or one row) */
#pragma omp parallel for schedule(static)
  for (int64_t bu = 0; bu < B * H * nqm; ++bu) {
    int64_t bh = bu / nqm, b = bh / H, h = bh % H;
    int64_t bhk = b * Hkv + h / (H / Hkv);
    const float* qm = qmean + bu * d;
    for (int64_t j = 0; j < Nk; ++j) {
      double s = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        float kt = in_f32(K[(bhk * Nk + j) * d + c], in_fp16) - kmean[bhk * d + c];
        s += (double)qm[c] * (double)kt;
      }
      qk_corr[bu * Nk + j] = (float)s;
    }
  }
}

/* V: MX-quantized along the tokens, per channel: v4 [B][Hkv][Nk][d], ve [B][Hkv][ceil(Nk/32)][d] */
void orc_fp4_prep_v(const uint16_t* V, int in_fp16, int64_t B, int64_t Hkv, int64_t Nk, int64_t d, uint8_t* v4,
                    uint8_t* ve) {
  const int64_t nkb = (Nk + ORC_MX - 1) / ORC_MX;
#pragma omp parallel
  {
    float* x = (float*)malloc((size_t)ORC_MX * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < B * Hkv * nkb; ++r) {
      int64_t bhk = r / nkb, u = r % nkb;
      int64_t t0 = u * ORC_MX, n = Nk - t0 < ORC_MX ? Nk - t0 : ORC_MX;
      for (int64_t c = 0; c < d; ++c) {
        for (int64_t k = 0; k < n; ++k) x[k] = in_f32(V[(bhk * Nk + t0 + k) * d + c], in_fp16);
        ve[r * d + c] = mx_block(x, 1, n, v4 + (bhk * Nk + t0) * d + c, d);
      }
    }
    free(x);
  }
}

/* Raw scores S_ij of one row against keys [j0, j1) of its head (no sm_scale). */
static void fp4_scores(const uint8_t* q4r, const uint8_t* qer, const uint8_t* k4h, const uint8_t* keh,
                       const float* corr_row, int64_t d, int64_t j0, int64_t j1, float* S) {
  const int64_t nb = d / ORC_MX;
  for (int64_t j = j0; j < j1; ++j) {
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c)
      acc += deq(q4r[c], qer[c / ORC_MX]) * deq(k4h[j * d + c], keh[j * nb + c / ORC_MX]);
    S[j - j0] = (float)(acc + (double)corr_row[j]);
  }
}

/* Raw scores of rows [row0, row0+nrows) x keys [col0, col0+ncols) of head (b, h), for checks. */
void orc_fp4_scores(const uint8_t* q4, const uint8_t* qe, const uint8_t* k4, const uint8_t* ke, const float* qk_corr,
                    int per_block, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t b, int64_t h,
                    int64_t row0, int64_t nrows, int64_t col0, int64_t ncols, float* out) {
  const int64_t nqm = per_block ? (Nq + ORC_QMBLK - 1) / ORC_QMBLK : 1, nb = d / ORC_MX;
  const int64_t bh = b * H + h, bhk = b * Hkv + h / (H / Hkv);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = row0 + r;
    fp4_scores(q4 + (bh * Nq + i) * d, qe + (bh * Nq + i) * nb, k4 + bhk * Nk * d, ke + bhk * Nk * nb,
               qk_corr + (bh * nqm + (per_block ? i / ORC_QMBLK : 0)) * Nk, d, col0, col0 + ncols,
               out + r * ncols);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* FP4 quantized attention forward (the emulation the GPU path must reproduce).              */
/* Key tiles of BN keys in increasing order; reference maximum m, moved to the running maximum */
/* when a tile's maximum exceeds it by more than tau log2 units; per tile p = exp(s - m) in     */
/* fp32, Phat = e4m3(ps * p) with ps = 448 * 2^-tau, l = alpha l + sum p,                      */
/* o = alpha o + Phat . Vdeq.  O = o / (ps l); LSE = m + ln l + sm_scale * lse_corr.           */
/* A row with no visible key: 0, -inf.                                                         */
/* rows: flattened (b*H + h)*Nq + i, or NULL for all.  Outputs as orc_attn_qe.               */
/* ------------------------------------------------------------------------------------------ */
void orc_fp4_attn_qe(const uint8_t* q4, const uint8_t* qe, const uint8_t* k4, const uint8_t* ke,
                     const float* qk_corr, int per_block, const float* lse_corr, const uint8_t* v4, const uint8_t* ve,
                     int causal, float sm_scale, int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                     int64_t BN, double tau, const int64_t* rows, int64_t nrows, float* o32, int out_fp16,
                     uint16_t* o16, float* lse) {
  const float ps = (float)ldexp(448.0, -(int)tau); /* tau is a whole number of log2 units */
  const int64_t nqm = per_block ? (Nq + ORC_QMBLK - 1) / ORC_QMBLK : 1, nb = d / ORC_MX;
  const int64_t nkb = (Nk + ORC_MX - 1) / ORC_MX;
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
      int64_t bhk = b * Hkv + h / (H / Hkv);
      const uint8_t* q4r = q4 + (bh * Nq + i) * d;
      const uint8_t* qer = qe + (bh * Nq + i) * nb;
      const float* crow = qk_corr + (bh * nqm + (per_block ? i / ORC_QMBLK : 0)) * Nk;
      int64_t jend = causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk; /* keys j < jend are visible */
      float m = -INFINITY, l = 0.0f;
      for (int64_t c = 0; c < d; ++c) o[c] = 0.0f;
      for (int64_t j0 = 0; j0 < jend; j0 += BN) {
        int64_t j1 = j0 + BN < jend ? j0 + BN : jend;
        fp4_scores(q4r, qer, k4 + bhk * Nk * d, ke + bhk * Nk * nb, crow, d, j0, j1, s);
        float tmax = -INFINITY;
        for (int64_t j = j0; j < j1; ++j) {
          s[j - j0] = s[j - j0] * sm_scale;
          if (s[j - j0] > tmax) tmax = s[j - j0];
        }
        float mnew = m;
        if (m == -INFINITY || (double)tmax > (double)m + tau * M_LN2) mnew = m > tmax ? m : tmax;
        float alpha = (m == -INFINITY) ? 0.0f : (float)exp((double)(m - mnew));
        float psum = 0.0f;
        for (int64_t j = j0; j < j1; ++j) {
          float p = (float)exp((double)(s[j - j0] - mnew));
          pq[j - j0] = orc_e4m3_to_f32(orc_f32_to_e4m3(ps * p));
          psum += p;
        }
        l = alpha * l + psum;
        for (int64_t c = 0; c < d; ++c) {
          float acc = alpha * o[c];
          for (int64_t j = j0; j < j1; ++j)
            acc += pq[j - j0] * (float)deq(v4[(bhk * Nk + j) * d + c], ve[(bhk * nkb + j / ORC_MX) * d + c]);
          o[c] = acc;
        }
        m = mnew;
      }
      for (int64_t c = 0; c < d; ++c) {
        float out = l == 0.0f ? 0.0f : (float)((double)o[c] / ((double)ps * (double)l));
        if (o32) o32[r * d + c] = out;
        if (o16) o16[r * d + c] = out_fp16 ? orc_f32_to_f16(out) : orc_f32_to_bf16(out);
      }
      if (lse)
        lse[r] = l == 0.0f ? -INFINITY
                           : (float)((double)m + log((double)l) + (double)sm_scale * (double)lse_corr[bh * Nq + i]);
    }
    free(o);
    free(s);
    free(pq);
  }
}

void orc_f32_to_e2m1_n(const float* x, uint8_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_e2m1(x[i]);
}
void orc_e2m1_to_f32_n(const uint8_t* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_e2m1_to_f32(x[i]);
}
void orc_mx_exp_n(const float* amax, int32_t* X, int64_t n) {
  for (int64_t i = 0; i < n; ++i) X[i] = orc_mx_exp(amax[i]);
}
