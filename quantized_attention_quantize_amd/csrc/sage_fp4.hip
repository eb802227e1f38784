// sage_fp4.hip -- the FP4 microscaling attention method on gfx950: MX FP4 quantization of Q, K
// and V, the FP32 correction rows of Q's smoothing, and the attention kernel.
//
// Method (page title, section): SageAttention docs digest (context7 llms.txt), "FP4 Attention for
// Blackwell GPUs" and "sageattn3_blackwell" -- FP4 microscaling quantization of Q, K and V,
// per_block_mean smoothing (default) or the global mean, causal attention; FlashInfer API doc
// "flashinfer.nvfp4_attention_sm120_fwd" -- packed FP4 Q and K with one 8-bit scale per vector, V
// and its scales stored transposed, an FP32 correction row per 128-token Q block, sm_scale
// (default 1/sqrt(d)), keys past the logical length masked, out / lse.  Element and scale formats:
// OCP Microscaling Formats (MX) v1.0 -- e2m1 elements, one E8M0 scale per 32 elements.
//
// Design (MI355X / CDNA4):
//  * gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 takes e2m1 operands with one E8M0 scale byte per
//    lane, that is per matrix row and 32-element k-block: MX FP4 is the matrix cores' own
//    microscaling format, so the block scales are applied inside the MFMA.
//  * Quantization: Q (its 128-token block means or global mean, smoothing, codes, the LSE shift of
//    K's smoothing), K (smoothed by its global mean, codes), V (codes along the tokens, written
//    transposed) and the correction rows qk_corr[u][j] = qmean_u . (K_j - kmean), formed as
//    qmean_u . K_j - qmean_u . kmean on the bf16 MFMA from exact bf16 parts of qmean and K.
//  * Attention: the INT8 kernel's organisation (8 waves x 32 query rows per workgroup, a
//    four-stage LDS ring filled by direct buffer-to-LDS loads two tiles ahead, one barrier per
//    64-key tile; each step a softmax phase and an MFMA phase, in opposite orders in the two waves
//    of a SIMD), with
//    - S^T = K Q^T on the f8f6f4 MFMA with both operands e2m1 and their scales; the MFMA's C
//      operand starts from the tile's correction values, so the accumulator holds the whole score;
//    - operand layouts of the 32x32x64 f8f6f4 MFMA: an e4m3 operand gives lane group g (lanes
//      32g..32g+31) the k-elements [32g, 32g+32); an e2m1 operand gives it [16g, 16g+16) in its
//      first 8 bytes and [32+16g, 48+16g) in the next 8, each lane's 32 elements under its own
//      scale byte (both measured on gfx950).  The K rows of a tile are therefore read from LDS in
//      the order key = 32 kb + 16 (r bit 2) + 4 (r >> 3) + (r & 3) for MFMA row r of key block kb:
//      the accumulators of lane group g then hold keys 32 kb + 16 g + [0, 16), P's e4m3 bytes land
//      on the k-elements that the e2m1 V operand of lane group g pairs with keys [32g, 32g+32), and
//      V^T needs no key permutation -- its MX blocks are 32 consecutive tokens;
//    - O^T += V^T P^T on the same MFMA with A = e2m1 V (scale per channel and 32-token block) and
//      B = e4m3 P with unit scale; P = e4m3(448 * p) against the exact running maximum (p <= 1,
//      the row maximum maps to 448).
//    The tile's correction values and K / V scale bytes travel through the LDS ring with the K and
//    V codes.  Head dimension 128.
#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kMX = 32;     // elements per MX block
constexpr int kQMB = 128;   // tokens per Q smoothing block
constexpr int kF4Threads = 256;
constexpr float kF4Log2_448 = 8.807354922057604f;  // log2(448)
// Reference maximum of the online softmax (log2 units): it moves when a tile's maximum exceeds it
// by more than kF4Tau.  With kF4Tau = 0 it is the exact running maximum, so p = 2^(t - m) <= 1 and
// P = e4m3(448 * p).
constexpr int kF4Tau = 0;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v8f __attribute__((ext_vector_type(8)));

// e2m1 codes of y0 (low nibble) and y1 (high nibble) into byte `sel` of w: the nearest of the
// magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, saturating at 6, bit 3 = the
// sign bit (a negative value rounding to 0 gives -0).  gfx950's v_cvt_scalef32_pk_fp4_f32 with
// unit scale computes exactly this: checked on the GPU against the rule written out as threshold
// comparisons over every non-NaN fp32 bit pattern.
template <int SEL>
__device__ __forceinline__ unsigned e2m1_pair(unsigned w, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y0, y1, 1.0f, SEL);
}

// E8M0 byte X + 127 of an MX block with largest magnitude amax >= 0, X = floor(log2 amax) - 2
// clamped to [-127, 127] (a zero block, or one below 2^-125, takes -127); inv = 2^-X, a normal
// float, so x * inv is exact.
__device__ __forceinline__ unsigned mx_scale_byte(float amax, float& inv) {
  const int ef = (int)(__float_as_uint(amax) >> 23);  // biased exponent (amax >= 0)
  int X = ef - 129;                                   // floor(log2 amax) = ef - 127 for normal amax
  if (X < -127) X = -127;
  inv = __uint_as_float((unsigned)(127 - X) << 23);
  return (unsigned)(X + 127);
}

// MX-quantizes the 8 consecutive channels [8 cg, 8 cg + 8) of one token held by this thread.  The
// 4 threads holding one 32-channel block are lanes that differ in bits 0-1 (cg & 3).  Writes 4
// code bytes and, from the block's first thread, the scale byte in lane order (block 2 cs + g at
// byte g * (D/64) + cs).
template <int D>
__device__ __forceinline__ void mx_store8(const float (&x)[8], int cg, uint8_t* codes_row, uint8_t* sc_row) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  float inv;
  const unsigned e8 = mx_scale_byte(amax, inv);
  unsigned w = 0;
  w = e2m1_pair<0>(w, x[0] * inv, x[1] * inv);
  w = e2m1_pair<1>(w, x[2] * inv, x[3] * inv);
  w = e2m1_pair<2>(w, x[4] * inv, x[5] * inv);
  w = e2m1_pair<3>(w, x[6] * inv, x[7] * inv);
  *reinterpret_cast<unsigned*>(codes_row + cg * 4) = w;
  if ((cg & 3) == 0) {
    const int lb = cg >> 2;
    sc_row[(lb & 1) * (D / 64) + (lb >> 1)] = (uint8_t)e8;
  }
}

// ---------------------------------------------------------------------------------------------
// Q: block means (per_block) or the global mean from q_mean, smoothing, MX codes per 32 channels,
// and lse_corr[i] = sum_c fp64(Q[i,c]) * fp64(kmean[c]) of the query head's key head.
// grid = (Nq_pad / 128, B*H), block = 512: thread t holds channels [8 (t % (D/8)), +8) of the
// block's tokens t / (D/8) + i * (512 / (D/8)) -- four tokens a thread at d = 128, whose 72
// registers leave room for seven waves per SIMD.  Rows past Nq get zero codes and scale bytes.
// ---------------------------------------------------------------------------------------------
template <int D, int IN>
__global__ __launch_bounds__(2 * kF4Threads) void k_fp4_quant_q(Fp4QuantArgs a) {
  constexpr int CG = D / 8, RPI = 2 * kF4Threads / CG, TPT = kQMB / RPI;
  __shared__ double csum[RPI][D];
  __shared__ float qm_s[D];
  const int t = threadIdx.x, cg = t % CG, rs = t / CG;
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t bhk = b * a.Hkv + h / (a.H / a.Hkv);
  const int u = blockIdx.x;
  const int64_t t0 = (int64_t)u * kQMB;
  const unsigned short* src = a.q + b * a.q_sb + h * a.q_sh + cg * 8;
  float km[8];
  {
    const float4 k0 = *reinterpret_cast<const float4*>(a.k_mean + bhk * D + cg * 8);
    const float4 k1 = *reinterpret_cast<const float4*>(a.k_mean + bhk * D + cg * 8 + 4);
    km[0] = k0.x, km[1] = k0.y, km[2] = k0.z, km[3] = k0.w, km[4] = k1.x, km[5] = k1.y, km[6] = k1.z, km[7] = k1.w;
  }
  // all loads first (kept as raw 16-bit values); then one pass over them: this thread's column
  // sums (fp64, exact for any realistic spread of magnitudes) and each token's partial lse_corr
  // over its 8 channels (exact fp64 products), a token at a time
  u16x8 raw[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t tok = t0 + rs + i * RPI;
    raw[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (tok < a.Nq) raw[i] = *reinterpret_cast<const u16x8*>(src + tok * a.q_sn);
  }
  double cs[8], ls[TPT];
#pragma unroll
  for (int j = 0; j < 8; ++j) cs[j] = 0.0;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    ls[i] = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double xd = (double)in_to_f32<IN>(raw[i][j]);
      cs[j] += xd;
      ls[i] += xd * (double)km[j];
    }
    asm volatile("" : "+v"(cs[0]), "+v"(cs[1]), "+v"(cs[2]), "+v"(cs[3]), "+v"(cs[4]), "+v"(cs[5]), "+v"(cs[6]),
                 "+v"(cs[7]), "+v"(ls[i]));
  }
  // The empty asm statements (no code) pin the sums token by token and hide the raw values from
  // the compiler: otherwise it sinks the sums past this loop and converts the raw values once for
  // both loops, keeping 64 fp64 values live across the barrier; the loop below converts again.
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    unsigned w4[4];
    __builtin_memcpy(w4, &raw[i], 16);
    asm volatile("" : "+v"(w4[0]), "+v"(w4[1]), "+v"(w4[2]), "+v"(w4[3]));
    __builtin_memcpy(&raw[i], w4, 16);
  }
  if (a.per_block) {  // the block's column sums combined in a fixed order
#pragma unroll
    for (int j = 0; j < 8; ++j) csum[rs][cg * 8 + j] = cs[j];
    __syncthreads();
    if (t < D) {
      double s = 0.0;
      for (int r = 0; r < RPI; ++r) s += csum[r][t];
      const int64_t nv = a.Nq - t0 < kQMB ? a.Nq - t0 : kQMB;
      const float m = nv > 0 ? (float)(s / (double)nv) : 0.f;
      qm_s[t] = m;
      if (u < a.nqm) a.q_mean[(bh * a.nqm + u) * D + t] = m;
    }
  } else if (t < D) {
    qm_s[t] = a.q_mean[bh * D + t];
  }
  __syncthreads();
  float qm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qm[j] = qm_s[cg * 8 + j];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t tok = t0 + rs + i * RPI;
    const bool valid = tok < a.Nq;
    double s = ls[i];
#pragma unroll
    for (int o = 1; o < CG; o <<= 1) s += __shfl_xor(s, o);
    if (cg == 0 && valid) a.lse_corr[bh * a.Nq + tok] = (float)s;
    float xs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[j] = valid ? in_to_f32<IN>(raw[i][j]) - qm[j] : 0.f;  // one fp32 rounding
    const int64_t row = bh * a.Nq_pad + tok;
    mx_store8<D>(xs, cg, a.q4 + row * (D / 2), a.q_sc + row * (D / kMX));
  }
}

// K smoothed by its global mean and MX-quantized per 32 channels.  grid = (Nk_pad / 64, B*Hkv),
// block = 256 (thread layout as k_fp4_quant_q over 64 tokens).
template <int D, int IN>
__global__ __launch_bounds__(kF4Threads) void k_fp4_quant_k(Fp4QuantArgs a) {
  constexpr int CG = D / 8, RPI = kF4Threads / CG, TPT = 64 / RPI;
  __shared__ float km_s[D];
  const int t = threadIdx.x, cg = t % CG, rs = t / CG;
  const int64_t bhk = blockIdx.y, b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  if (t < D) km_s[t] = a.k_mean[bhk * D + t];
  __syncthreads();
  const unsigned short* src = a.k + b * a.k_sb + hk * a.k_sh + cg * 8;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t tok = t0 + rs + i * RPI;
    float xs[8];
    if (tok < a.Nk) {
      const u16x8 v = *reinterpret_cast<const u16x8*>(src + tok * a.k_sn);
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = in_to_f32<IN>(v[j]) - km_s[cg * 8 + j];  // one fp32 rounding
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = 0.f;
    }
    const int64_t row = bhk * a.Nk_pad + tok;
    mx_store8<D>(xs, cg, a.k4 + row * (D / 2), a.k_sc + row * (D / kMX));
  }
}

// V: per channel and 32-token block, MX codes along the tokens, written transposed.  grid =
// (Nk_pad / 64, B*Hkv), block = 256: the 64 x D tile goes through LDS as its raw 16-bit inputs
// (half the bytes of fp32, so twice the workgroups per CU hide the loads); thread t < 2D then
// quantizes channel t % D over the tile's 32-token block t / D.  Tokens past Nk count as zero.
template <int D, int IN>
__global__ __launch_bounds__(kF4Threads) void k_fp4_prep_v(Fp4QuantArgs a) {
  constexpr int CG = D / 8, RPI = kF4Threads / CG, TPT = 64 / RPI;
  __shared__ unsigned short sv[64][D + 2];  // raw inputs (17 KB: eight workgroups per CU)
  const int t = threadIdx.x, cg = t % CG, rs = t / CG;
  const int64_t bhk = blockIdx.y, b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const unsigned short* src = a.v + b * a.v_sb + hk * a.v_sh + cg * 8;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int r = rs + i * RPI;
    const int64_t tok = t0 + r;
    if (tok < a.Nk) {
      const u16x8 v = *reinterpret_cast<const u16x8*>(src + tok * a.v_sn);
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[r][cg * 8 + j] = v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[r][cg * 8 + j] = 0;
    }
  }
  __syncthreads();
  if (t < 2 * D) {
    const int c = t % D, blk = t / D;
    float amax = 0.f;
#pragma unroll 8
    for (int k = 0; k < kMX; ++k) amax = fmaxf(amax, fabsf(in_to_f32<IN>(sv[kMX * blk + k][c])));
    float inv;
    const unsigned e8 = mx_scale_byte(amax, inv);
    unsigned w[4] = {0u, 0u, 0u, 0u};
    auto x = [&](int k) { return in_to_f32<IN>(sv[kMX * blk + k][c]) * inv; };
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // tokens 8 q .. 8 q + 7 into word q
      w[q] = e2m1_pair<0>(w[q], x(8 * q), x(8 * q + 1));
      w[q] = e2m1_pair<1>(w[q], x(8 * q + 2), x(8 * q + 3));
      w[q] = e2m1_pair<2>(w[q], x(8 * q + 4), x(8 * q + 5));
      w[q] = e2m1_pair<3>(w[q], x(8 * q + 6), x(8 * q + 7));
    }
    uint8_t* dst = a.v4t + (bhk * D + c) * (a.Nk_pad / 2) + blockIdx.x * 32 + blk * 16;
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    a.v_sc[(bhk * (a.Nk_pad / kMX) + blockIdx.x * 2 + blk) * D + (c % 32) * (D / 32) + c / 32] = (uint8_t)e8;
  }
}

// x = p[0] + p[1] + p[2] exactly: three bf16 parts of fp32 values (each residue is exact in fp32
// and at most 16, then 8, significant bits long)
__device__ __forceinline__ void split3(v8f x, v8bf (&p)[3]) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    p[k] = __builtin_convertvector(x, v8bf);  // round to nearest even
    x = x - __builtin_convertvector(p[k], v8f);
  }
}

// qk_corr[b,h,u,j] = qmean[b,h,u,:] . (K[b,hk,j,:] - kmean) for keys j < Nk (zero for j < Nk_pad
// past Nk), as qmean . K_j - qmean . kmean: D (32 Q blocks x 32 keys) += qmean (32 x 16) K^T
// (16 x 32) per 16 channels on the bf16 MFMA, starting from D = -(qmean . kmean) (summed in fp64,
// rounded once).  qmean enters in three exact bf16 parts; a bf16 K is its own single part, an fp16
// K splits into two exact bf16 parts (its 11 significant bits) and the product of the two smallest
// parts, below 2^-24 of |qmean_c K_jc|, is dropped.  Every product is exact, so the only error is
// the fp32 accumulation; it scales with |qmean| |K| -- far below K's own input rounding relative
// to K - kmean, however large K's mean.
// A wave splits the means of one group of 32 Q blocks once, keeps the parts in registers and
// streams up to kpw blocks of 32 keys past them.  Work item c = (b*H + h) * nchunk + chunk covers
// 4 * kpw key blocks (wave w takes blocks 4 i + w of the chunk).  The ngroups workgroups of one
// item sit 8 apart in launch order: workgroups are dealt to the 8 XCDs in turn, so all groups of
// an item run on one XCD and read its K through one L2.
// Workgroup ids per launch of k_fp4_corr, whose id count grows with Nq * Nk: larger problems take
// several launches, each from an offset wg0 that is a multiple of 8 (the id's XCD is kept).
constexpr int64_t kF4MaxCorrLaunch = (int64_t)1 << 20;

__host__ __device__ constexpr int64_t f4corr_chunks(int64_t Nk_pad, int kpw) {
  return (Nk_pad / 32 + 4 * kpw - 1) / (4 * kpw);
}

template <int D, int IN>
__global__ __launch_bounds__(kF4Threads) __attribute__((amdgpu_waves_per_eu(2))) void k_fp4_corr(Fp4QuantArgs a,
                                                                                                  int ngroups, int kpw,
                                                                                                  int64_t wg0) {
  __shared__ float km_s[D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 31, g = lane >> 5;
  const int64_t nchunk = f4corr_chunks(a.Nk_pad, kpw), nkb = a.Nk_pad / 32;
  const int64_t wg = wg0 + blockIdx.x, grp = (wg >> 3) % ngroups, c = (wg & 7) + 8 * ((wg >> 3) / ngroups);
  if (c >= a.B * a.H * nchunk) return;  // the whole workgroup, before the barrier
  const int64_t bh = c / nchunk, b = bh / a.H, h = bh % a.H;
  const int64_t hk = h / (a.H / a.Hkv), bhk = b * a.Hkv + hk;
  const int64_t kb0 = (c % nchunk) * 4 * kpw + w;
  int64_t nb = (nkb - kb0 + 3) / 4;
  nb = nb < kpw ? nb : kpw;  // blocks kb0, kb0 + 4, ... of this wave (none in a ragged last chunk)
  const unsigned short* kh = a.k + b * a.k_sb + hk * a.k_sh + 8 * g;
  // B operand column: key 32 kb + lr, channels 16 kk + 8 g .. + 8.  The loads carry no branch (a
  // key past Nk reads row Nk - 1; its D column is independent of the others and stored as zero).
  auto load_k = [&](int64_t kb, u16x8(&r)[D / 16]) {
    const int64_t key = 32 * kb + lr;
    const unsigned short* src = kh + (key < a.Nk ? key : a.Nk - 1) * a.k_sn;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) r[kk] = *reinterpret_cast<const u16x8*>(src + 16 * kk);
  };
  auto kb_of = [&](int64_t i) { return kb0 + 4 * (i < nb ? i : (nb > 0 ? nb - 1 : 0)); };
  // the first two key blocks, the means and K's mean are all requested before anything waits
  u16x8 ka[D / 16], kz[D / 16];
  if (nb > 0) {
    load_k(kb_of(0), ka);
    load_k(kb_of(1), kz);
  }
  const int u = 32 * (int)grp + lr;  // A operand row: Q block u, channels 16 kk + 8 g .. + 8
  const bool uv = u < a.nqm;
  const float* qm = a.q_mean + (bh * a.nqm + (uv ? u : 0)) * D + 8 * g;
  v8f y[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    y[kk] = v8f{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (uv) {
      const float4 lo = *reinterpret_cast<const float4*>(qm + 16 * kk);
      const float4 hi = *reinterpret_cast<const float4*>(qm + 16 * kk + 4);
      y[kk] = v8f{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }
  if (threadIdx.x < D) km_s[threadIdx.x] = a.k_mean[bhk * D + threadIdx.x];
  __syncthreads();
  if (nb <= 0) return;
  v8bf ap[D / 16][3];
  double qk = 0.0;  // qmean_u . kmean over this lane's channels
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    split3(y[kk], ap[kk]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qk += (double)y[kk][e] * (double)km_s[16 * kk + 8 * g + e];
  }
  qk += __shfl_xor(qk, 32);
  const float qkf = (float)qk;
  v16f c0;  // D row 8 rq + 4 g + e is Q block 32 grp + 8 rq + 4 g + e, whose qmean . kmean lane 8 rq + 4 g + e holds
#pragma unroll
  for (int rq = 0; rq < 4; ++rq)
#pragma unroll
    for (int e = 0; e < 4; ++e) c0[4 * rq + e] = -__shfl(qkf, 8 * rq + 4 * g + e);
  // this head's correction rows (nqm * Nk_pad * 4 < 2^31 bytes, host-checked); the stores of rows
  // past nqm (in the last group) go to an offset past the range, which the hardware drops, so they
  // need no branch
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.qk_corr + bh * a.nqm * a.Nk_pad), (short)0, (int)(a.nqm * a.Nk_pad * 4), kBufferWord3);
  constexpr int kOutOfRange = 0x7ffffffc;
  auto block = [&](int64_t kb, const u16x8(&kr)[D / 16]) {
    v16f acc = c0;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if constexpr (IN == 0) {
        const v8bf kp = __builtin_bit_cast(v8bf, kr[kk]);
#pragma unroll
        for (int p = 2; p >= 0; --p) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][p], kp, acc, 0, 0, 0);
      } else {
        v8f x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = in_to_f32<IN>(kr[kk][e]);
        const v8bf k0 = __builtin_convertvector(x, v8bf);  // round to nearest even
        const v8bf k1 = __builtin_convertvector(x - __builtin_convertvector(k0, v8f), v8bf);  // exact residue
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][2], k0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][1], k1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][1], k0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][0], k1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][0], k0, acc, 0, 0, 0);
      }
    }
    const bool kv = 32 * kb + lr < a.Nk;  // D column lr is key 32 kb + lr
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int uu = 32 * (int)grp + 8 * rq + 4 * g + e;
        const int off = uu < a.nqm ? (int)(((int64_t)uu * a.Nk_pad + 32 * kb + lr) * 4) : kOutOfRange;
        // a scalar first: hipcc compiles __builtin_bit_cast of a vector element as element 0
        const float x = kv ? acc[4 * rq + e] : 0.f;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), crs, off, 0, 0);
      }
  };
  // Two register buffers: the next block's loads are issued before the current block's products
  // (past the end, a block reloads itself).  The first block is peeled off so that the loop is
  // entered, as it repeats, with one block's stores in flight between the two buffers' loads: the
  // compiler's wait for a buffer then lets those stores retire in the background.
  __builtin_amdgcn_sched_barrier(0);
  block(kb_of(0), ka);
  for (int64_t i = 1; i < nb; i += 2) {
    load_k(kb_of(i + 1), ka);
    __builtin_amdgcn_sched_barrier(0);
    block(kb_of(i), kz);
    if (i + 1 >= nb) break;
    load_k(kb_of(i + 2), kz);
    __builtin_amdgcn_sched_barrier(0);
    block(kb_of(i + 1), ka);
  }
}

// ---------------------------------------------------------------------------------------------
// Attention (head dimension 128).
// ---------------------------------------------------------------------------------------------
constexpr int kF4Waves = kBlockM / 32;           // 8 waves x 32 query rows
constexpr int kF4AttnThreads = kF4Waves * 64;
constexpr int kF4NS = 4;                         // ring stages
constexpr int kF4KB = kBlockN * 64;              // K tile: 64 keys x 64 bytes
constexpr int kF4VB = 128 * kBlockN / 2;         // V^T tile: 128 channels x 32 bytes (64 rows of 64)
constexpr int kF4CB = 2 * kBlockN * 4;           // correction values of the workgroup's two Q blocks
constexpr int kF4SB = 256;                       // K scales (64 keys x 4) or V scales (2 x 128) of a tile
constexpr int kF4Ring = kF4NS * (kF4KB + kF4VB + kF4CB + 2 * kF4SB);
constexpr int kF4OStage = (kF4AttnThreads / 64) * 32 * 256;  // the epilogue's output staging: 32 rows of 256 bytes a wave
constexpr int kF4Smem = kF4Ring > kF4OStage ? kF4Ring : kF4OStage;

// Chunk swizzle of the FP4 tiles' 64-byte LDS rows (64 rows per tile).  In one 16-lane LDS phase
// the K fragment reads take rows 32 kb + 16 (l bit 2) + 4 (l >> 3) + (l & 3) and the V fragment
// reads rows 16 db + (l >> 1) with chunk 2 (l & 1) + g; XORing the chunk with
// (row bit 2) | (row bit 4) << 1 sends each phase to 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_f4(int row) { return ((row >> 2) & 1) | (((row >> 4) & 1) << 1); }
// LDS row of the K tile that MFMA row r of key block kb reads (its key within the tile)
__device__ __forceinline__ int f4_krow(int kb, int r) { return 32 * kb + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }
// Key of the tile held in accumulator register r of key block kb by lane group g
__device__ __forceinline__ int f4_key(int kb, int r, int g) { return 32 * kb + 16 * g + 4 * (r >> 2) + (r & 3); }

// Per-lane LDS offsets of a lane's fragments inside a tile buffer.
struct F4Lanes {
  int k[2];   // K codes, chunk 2 cs + g of row f4_krow(0, lr); key block 1 is 32 rows (2 KiB) on
  int v[4];   // V codes of channel block db: row 16 db + (lr >> 1), chunk 2 (lr & 1) + g
  int ks[2];  // K scale bytes (u16 at 2 g) of the key block's row
  int c;      // correction values: the wave's Q block, keys 16 g ..
  int vs;     // V scale word: 32-token block g, channel lr
  __device__ __forceinline__ void init(int lr, int g, int sel) {
    const int r0 = f4_krow(0, lr);
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) k[cs] = r0 * 64 + (((2 * cs + g) ^ swz_f4(r0)) << 4);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int r = 16 * db + (lr >> 1);
      v[db] = r * 64 + (((2 * (lr & 1) + g) ^ swz_f4(r)) << 4);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ks[kb] = f4_krow(kb, lr) * 4 + 2 * g;
    c = sel * 256 + 16 * g * 4;
    vs = g * 128 + lr * 4;
  }
};

__device__ __forceinline__ v8i widen(v4i x) { return v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }

// O^T[db] += V^T P^T for channel block db: A = e2m1 V codes (scale byte db of the lane's word vs),
// B = e4m3 P (unit scale 2^0).  The scale byte select is an immediate, hence the switch.
__device__ __forceinline__ void f4_pv(v16f (&o)[4], int db, v4i vf, const v8i& P, int vs) {
  switch (db) {
    case 0: o[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(vf), P, o[0], 4, 0, 0, vs, 0, 127); break;
    case 1: o[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(vf), P, o[1], 4, 0, 1, vs, 0, 127); break;
    case 2: o[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(vf), P, o[2], 4, 0, 2, vs, 0, 127); break;
    default: o[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(vf), P, o[3], 4, 0, 3, vs, 0, 127); break;
  }
}

// S^T of one tile for the wave: acc[kb][r] = S of query lr and key f4_key(kb, r, g), started from
// the correction values.  sK / sC / sKS: the tile's K codes, correction values and K scales.
__device__ __forceinline__ void f4_qk_tile(const char* sK, const char* sC, const char* sKS, const v8i (&qf)[2],
                                           int qsc, const F4Lanes& lb, v16f (&acc)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float* cp = reinterpret_cast<const float*>(sC + lb.c) + 32 * kb;
    v16f c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(cp + 4 * q);
      c[4 * q] = f.x;
      c[4 * q + 1] = f.y;
      c[4 * q + 2] = f.z;
      c[4 * q + 3] = f.w;
    }
    const int ks = *reinterpret_cast<const unsigned short*>(sKS + lb.ks[kb]);
    const v4i k0 = *reinterpret_cast<const v4i*>(sK + lb.k[0] + 2048 * kb);
    const v4i k1 = *reinterpret_cast<const v4i*>(sK + lb.k[1] + 2048 * kb);
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(k0), qf[0], c, 4, 4, 0, ks, 0, qsc);
    acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(k1), qf[1], c, 4, 4, 1, ks, 1, qsc);
  }
}

// Scores of keys past lim (tile-relative) become -inf.
__device__ __forceinline__ void f4_mask(v16f (&acc)[2], int g, int lim) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (f4_key(kb, r, g) > lim) acc[kb][r] = -INFINITY;
}

// Row maximum of a tile in four chains of eight scores; piece p (0..7) advances chain p/2 (pieces
// 0-3 cover key block 0, 4-7 key block 1).
__device__ __forceinline__ float f4_at(const v16f (&s)[2], int i) { return s[i >> 4][i & 15]; }
__device__ __forceinline__ void f4_max_piece(const v16f (&s)[2], float (&ch)[4], int p) {
  const int c = p >> 1, e = 8 * c;
  if ((p & 1) == 0) {
    ch[c] = fmaxf(fmaxf(f4_at(s, e), f4_at(s, e + 1)), f4_at(s, e + 2));
    ch[c] = fmaxf(fmaxf(ch[c], f4_at(s, e + 3)), f4_at(s, e + 4));
  } else {
    ch[c] = fmaxf(fmaxf(ch[c], f4_at(s, e + 5)), f4_at(s, e + 6));
    ch[c] = fmaxf(ch[c], f4_at(s, e + 7));
  }
}

struct F4Row {
  float m;   // reference maximum (log2 units)
  float pm;  // exponent offset: m - log2(448) + kF4Tau
  float l;   // partial denominator (sum of P's unrounded values over this lane group's keys)
};

// Combines the chains over the row (lanes l and l ^ 32) and moves the reference maximum when the
// tile's maximum exceeds it by more than kF4Tau; returns 2^(m_old - m_new).
// c = sm_scale * log2(e) > 0.
__device__ __forceinline__ float f4_finish_max(const float (&ch)[4], float c, F4Row& rs) {
  float im = fmaxf(fmaxf(ch[0], ch[1]), fmaxf(ch[2], ch[3]));
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(im), __float_as_int(im), false, false);
  im = fmaxf(__int_as_float((int)sw[0]), __int_as_float((int)sw[1]));
  const float mt = im * c;  // -inf if nothing of the tile is visible
  const float m_new = mt > rs.m + (float)kF4Tau ? mt : rs.m;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(rs.m - m_use);
  rs.m = m_new;
  rs.pm = m_use - kF4Log2_448 + (float)kF4Tau;
  return alpha;
}

// One software-pipelined tile step of a wave.  At step n T[n] has been scored (acc) and the row
// maxima of its key block 0 are in ch; P holds T[n-1]'s probabilities.  MFMA stream: PV of T[n-1]
// (V from sVp, first operand in vpre, scale word vsc) into O, then QK of T[n+1] (K, correction
// values and K scales from sKn / sCn / sKSn) into acc.  VALU: T[n]'s key-block-1 maxima (slot 0),
// its running maximum (slot 1), its exponentials (key block 0 in slots 2-3, before the QK of slot
// 4 overwrites acc[0]; key block 1 in slots 4-5, before slot 6), and T[n+1]'s key-block-0 maxima
// (slots 6-7).  SLOW: T[n+1] is masked by lim after the stream, then its maxima are taken.
// At the end vpre / vsc receive the next step's first PV operand and scale word (sVn / sVSn).
// Returns 2^(m_{n-1} - m_n), the factor O takes after the PV of T[n-1].
template <bool SLOW>
__device__ __forceinline__ float f4_step(v16f (&acc)[2], float (&ch)[4], v8i& P, v4i& vpre, int& vsc,
                                         const char* sVp, const char* sVn, const char* sVSn, const char* sKn,
                                         const char* sCn, const char* sKSn, const v8i (&qf)[2], int qsc,
                                         v16f (&o)[4], float c, F4Row& rs, const F4Lanes& lb, int g, int lim) {
  const v16f sc[2] = {acc[0], acc[1]};  // scores of T[n]
  const v8i pin = P;                    // probabilities of T[n-1]
  v4i vf[4], kf[4];
  v16f cv[2];
  int ks[2];
  vf[0] = vpre;
  auto read = [&](int r) {  // operands of MFMA r
    if (r < 4) {
      vf[r] = *reinterpret_cast<const v4i*>(sVp + lb.v[r]);
    } else {
      const int q = r - 4, kb = q >> 1, cs = q & 1;
      kf[q] = *reinterpret_cast<const v4i*>(sKn + lb.k[cs] + 2048 * kb);
    }
  };
  auto read_c = [&](int kb) {  // correction values and K scales of key block kb of T[n+1]
    const float* cp = reinterpret_cast<const float*>(sCn + lb.c) + 32 * kb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(cp + 4 * q);
      cv[kb][4 * q] = f.x;
      cv[kb][4 * q + 1] = f.y;
      cv[kb][4 * q + 2] = f.z;
      cv[kb][4 * q + 3] = f.w;
    }
    ks[kb] = *reinterpret_cast<const unsigned short*>(sKSn + lb.ks[kb]);
  };
  float psum = 0.f, alpha = 1.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k + 1 < 8) read(k + 1);
    if (k == 2) read_c(0);
    if (k == 4) read_c(1);
    if (k < 4) {
      f4_pv(o, k, vf[k], pin, vsc);
    } else {
      const int q = k - 4, kb = q >> 1, cs = q & 1;
      if (cs == 0)
        acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(kf[q]), qf[0], cv[kb], 4, 4, 0, ks[kb], 0, qsc);
      else
        acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(kf[q]), qf[1], acc[kb], 4, 4, 1, ks[kb], 1, qsc);
    }
    if (k == 0) {
#pragma unroll
      for (int p = 4; p < 8; ++p) f4_max_piece(sc, ch, p);
    }
    if (k == 1) alpha = f4_finish_max(ch, c, rs);
    if (k >= 2 && k < 6) {  // exponential groups 2 (k - 2) and 2 (k - 2) + 1: four scores each
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int gi = 2 * (k - 2) + gg;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * gi + e;
          float s = sc[idx >> 4][idx & 15];
          asm volatile("" : "+v"(s));  // keeps the exponential in its slot
          x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s, c, -rs.pm));  // -inf gives 0
        }
        psum += (x[0] + x[1]) + (x[2] + x[3]);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        P[gi] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);  // byte e: key f4_key(gi / 4, 4 (gi % 4) + e, g)
      }
    }
    if (!SLOW && k >= 6) {
#pragma unroll
      for (int p = 2 * (k - 6); p < 2 * (k - 6) + 2; ++p) f4_max_piece(acc, ch, p);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (SLOW) {
    f4_mask(acc, g, lim);
#pragma unroll
    for (int p = 0; p < 4; ++p) f4_max_piece(acc, ch, p);
  }
  rs.l = alpha * rs.l + psum;
  vpre = *reinterpret_cast<const v4i*>(sVn + lb.v[0]);
  vsc = *reinterpret_cast<const int*>(sVSn + lb.vs);
  return alpha;
}

// Phase-split form of the step (the INT8 kernel's phase-split schedule): waves 0-3 take a tile's
// softmax and then the MFMA phase, waves 4-7 the MFMA phase and then the next tile's softmax, so
// the two waves of a SIMD overlap one's exponentials with the other's MFMAs.
// Softmax of the tile whose scores are in acc (SLOW: keys past lim masked): row maxima, reference
// maximum, P = e4m3(448 * p) and the row sums.  Returns 2^(m_old - m_new), O's factor before this
// tile's PV.
template <bool SLOW>
__device__ __forceinline__ float f4_softmax(v16f (&acc)[2], v8i& P, float c, F4Row& rs, int g, int lim) {
  if constexpr (SLOW) f4_mask(acc, g, lim);
  float ch[4];
#pragma unroll
  for (int p = 0; p < 8; ++p) f4_max_piece(acc, ch, p);
  const float alpha = f4_finish_max(ch, c, rs);
  float psum = 0.f;
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = 4 * gi + e;
      x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[idx >> 4][idx & 15], c, -rs.pm));  // -inf gives 0
    }
    psum += (x[0] + x[1]) + (x[2] + x[3]);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    P[gi] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);  // byte e: key f4_key(gi / 4, 4 (gi % 4) + e, g)
  }
  rs.l = alpha * rs.l + psum;
  return alpha;
}

// MFMA phase: the QK of the next tile (K codes, correction values and K scales from sK / sC / sKS;
// its first K fragment arrives in k0) into acc, then the PV of the current tile (V codes and scale
// word from sV / sVS) from P into O.  Operands are read from LDS two MFMAs ahead.
__device__ __forceinline__ void f4_mfma(v4i k0, const char* sK, const char* sC, const char* sKS, const char* sV,
                                        const char* sVS, const v8i (&qf)[2], int qsc, const v8i& P, v16f (&o)[4],
                                        v16f (&acc)[2], const F4Lanes& lb) {
  v4i kf[4], vf[4];
  v16f cv[2];
  int ks[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float* cp = reinterpret_cast<const float*>(sC + lb.c) + 32 * kb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(cp + 4 * q);
      cv[kb][4 * q] = f.x;
      cv[kb][4 * q + 1] = f.y;
      cv[kb][4 * q + 2] = f.z;
      cv[kb][4 * q + 3] = f.w;
    }
    ks[kb] = *reinterpret_cast<const unsigned short*>(sKS + lb.ks[kb]);
  }
  const int vsc = *reinterpret_cast<const int*>(sVS + lb.vs);
  kf[0] = k0;
  auto read = [&](int r) {
    if (r < 4) {
      const int kb = r >> 1, cs = r & 1;
      kf[r] = *reinterpret_cast<const v4i*>(sK + lb.k[cs] + 2048 * kb);
    } else {
      vf[r - 4] = *reinterpret_cast<const v4i*>(sV + lb.v[r - 4]);
    }
  };
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k == 0) read(1);  // operands two MFMAs ahead (k0 arrives read)
    if (k + 2 < 8) read(k + 2);
    if (k < 4) {
      const int kb = k >> 1, cs = k & 1;
      if (cs == 0)
        acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(kf[k]), qf[0], cv[kb], 4, 4, 0, ks[kb], 0, qsc);
      else
        acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(kf[k]), qf[1], acc[kb], 4, 4, 1, ks[kb], 1, qsc);
    } else {
      f4_pv(o, k - 4, vf[k - 4], P, vsc);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The workgroup's tile loads.  Waves 0-3 each fill one 1 KiB segment of a K tile (wave 3 also the
// two correction rows with lanes 0-31, wave 2 the K scale bytes with lanes 0-15); waves 4-7 one
// segment of a V tile (wave 7 also the V scale bytes with lanes 0-15).  A lane fetches the global
// 16-byte chunk that belongs at its swizzled LDS position.
struct F4Stager {
  __amdgpu_buffer_rsrc_t rs, xs;
  int off, xoff;  // per-lane source offsets
  int w, lane;
  __device__ __forceinline__ void init(const Fp4AttnArgs& a, int64_t bh, int64_t bhk, int qt, int wave, int ln) {
    w = __builtin_amdgcn_readfirstlane(wave);
    lane = ln;
    const int r = 16 * (w & 3) + (lane >> 2);  // LDS row of this lane's chunk
    const int lc = (lane & 3) ^ swz_f4(r);     // the logical chunk that belongs there
    const int vrow = (int)(a.Nk_pad / 2);      // bytes per channel row of V^T
    if (w < 4) {
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k4 + bhk * a.Nk_pad * 64), (short)0, (int)(a.Nk_pad * 64),
                                             kBufferWord3);
      off = r * 64 + lc * 16;
    } else {
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v4t + bhk * 128 * (int64_t)vrow), (short)0, 128 * vrow,
                                             kBufferWord3);
      off = (2 * r + (lc >> 1)) * vrow + (lc & 1) * 16;
    }
    xoff = 0;
    if (w == 3) {  // correction rows of the workgroup's Q blocks 2 qt and 2 qt + 1
      int row = a.per_block ? 2 * qt + (lane >> 4) : 0;
      row = row < a.nqm ? row : a.nqm - 1;
      xs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.qk_corr + bh * a.nqm * a.Nk_pad), (short)0,
                                             (int)(a.nqm * a.Nk_pad * 4), kBufferWord3);
      xoff = row * (int)a.Nk_pad * 4 + (lane & 15) * 16;
    } else if (w == 2) {
      xs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_sc + bhk * a.Nk_pad * 4), (short)0, (int)(a.Nk_pad * 4),
                                             kBufferWord3);
      xoff = lane * 16;
    } else if (w == 7) {
      xs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v_sc + bhk * (a.Nk_pad / kMX) * 128), (short)0,
                                             (int)(a.Nk_pad / kMX * 128), kBufferWord3);
      xoff = lane * 16;
    }
  }
  // loads issued per step by this wave (for the vmcnt waits)
  __device__ __forceinline__ int nload() const { return (w == 2 || w == 3 || w == 7) ? 2 : 1; }
  __device__ __forceinline__ void load_k(int kt, char* sK, char* sC, char* sKS) const {
    if (w < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(sK + w * 1024), 16, off, kt * kF4KB, 0, 0);
      if (w == 3 && lane < 32)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t*)sC, 16, xoff, kt * 256, 0, 0);
      if (w == 2 && lane < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t*)sKS, 16, xoff, kt * 256, 0, 0);
    }
  }
  __device__ __forceinline__ void load_v(int kt, char* sV, char* sVS) const {
    if (w >= 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(sV + (w - 4) * 1024), 16, off, kt * 32, 0, 0);
      if (w == 7 && lane < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t*)sVS, 16, xoff, kt * 256, 0, 0);
    }
  }
};

// PP: the phase-split schedule (f4_softmax / f4_mfma) instead of f4_step.
template <int PP>
__global__ __launch_bounds__(kF4AttnThreads) void k_fp4_attn(Fp4AttnArgs a) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) char smem[kF4Smem];
  char* const kring = smem;
  char* const vring = kring + kF4NS * kF4KB;
  char* const cring = vring + kF4NS * kF4VB;
  char* const ksring = cring + kF4NS * kF4CB;
  char* const vsring = ksring + kF4NS * kF4SB;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int w = tid >> 6;
  // PP: waves 4-7 run their MFMA phase first; waves w and w + 4 share a SIMD
  const int grp1 = __builtin_amdgcn_readfirstlane(w >= 4 ? 1 : 0);

  int64_t bh;
  int qt;
  map_workgroup(a.B, a.H, a.Hkv, a.nQT, a.causal, bh, qt);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t bhk = b * a.Hkv + h / (a.H / a.Hkv);
  const int q0 = qt * kBlockM;
  const int r0w = q0 + w * 32;
  const int row = r0w + lr;
  const int nk = (int)a.Nk, nq = (int)a.Nq;
  if (q0 >= nq) return;

  int kt_end = (nk + kBlockN - 1) / kBlockN;
  if (a.causal) {
    const int lim = (q0 + kBlockM + kBlockN - 1) / kBlockN;
    if (lim < kt_end) kt_end = lim;
  }

  v16f o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // The first step multiplies a zero P by the V slot of "T[-1]": clear its codes and scale bytes so
  // uninitialized LDS (a NaN scale) cannot leak in.
  for (int i = tid; i < kF4VB / 16; i += kF4AttnThreads)
    *reinterpret_cast<v4i*>(vring + (kF4NS - 1) * kF4VB + i * 16) = v4i{0, 0, 0, 0};
  for (int i = tid; i < kF4SB / 16; i += kF4AttnThreads)
    *reinterpret_cast<v4i*>(vsring + (kF4NS - 1) * kF4SB + i * 16) = v4i{0, 0, 0, 0};

  F4Stager st;
  st.init(a, bh, bhk, qt, w, lane);
  const int t0 = 0;
  auto clampt = [&](int t) { return t < kt_end ? t : 0; };
  if (kt_end > 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
      st.load_k(clampt(t0 + i), kring + i * kF4KB, cring + i * kF4CB, ksring + i * kF4SB);
#pragma unroll
    for (int i = 0; i < 2; ++i) st.load_v(clampt(t0 + i), vring + i * kF4VB, vsring + i * kF4SB);
  }
  // the wave's Q codes (B operand: row lr, channels 64 cs + 32 g ..) and scale bytes
  v8i qf[2];
  int qsc = 0;
  {
    const int64_t qrow = bh * a.Nq_pad + (row < a.Nq_pad ? row : 0);
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) qf[cs] = widen(*reinterpret_cast<const v4i*>(a.q4 + qrow * 64 + 32 * cs + 16 * g));
    qsc = *reinterpret_cast<const unsigned short*>(a.q_sc + qrow * 4 + 2 * g);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const float c = a.sm_scale * kLog2e;
  auto partial = [&](int t) {
    if (t >= kt_end) return true;
    const int j0 = __builtin_amdgcn_mbcnt_lo(0u, t) * kBlockN;  // per-lane copy: see the INT8 kernel
    return j0 + kBlockN > nk || (a.causal && j0 + kBlockN - 1 > r0w);
  };
  auto limit = [&](int t) {  // last visible tile-relative key of this lane's row
    if (t >= kt_end) return -1;
    const int j0 = t * kBlockN;
    int lim = j0 + kBlockN > nk ? nk - j0 - 1 : kBlockN - 1;
    if (a.causal) {
      const int dr = row - j0;
      lim = dr < lim ? (dr < -1 ? -1 : dr) : lim;
    }
    return lim;
  };

  F4Lanes lb;
  lb.init(lr, g, w >> 2);
  F4Row rs;
  rs.m = -INFINITY;
  rs.pm = 0.f;
  rs.l = 0.f;
  v16f acc[2];
  float ch[4];
  v8i P = {0, 0, 0, 0, 0, 0, 0, 0};
  v4i vpre;
  int vsc;
  bool part_cur = partial(t0);
  if constexpr (PP) {  // scores of T[0]; group 1 takes their softmax before its first step
    f4_qk_tile(kring, cring, ksring, qf, qsc, lb, acc);
    if (grp1) {
      if (part_cur)
        f4_softmax<true>(acc, P, c, rs, g, limit(t0));
      else
        f4_softmax<false>(acc, P, c, rs, g, kBlockN - 1);
      // O is still zero: the factor returned needs no application
    }
  } else {  // scores of T[0] and the row maxima of its key block 0; the first PV operands (T[-1])
    f4_qk_tile(kring, cring, ksring, qf, qsc, lb, acc);
    if (part_cur) f4_mask(acc, g, limit(t0));
#pragma unroll
    for (int p = 0; p < 4; ++p) f4_max_piece(acc, ch, p);
    vpre = *reinterpret_cast<const v4i*>(vring + (kF4NS - 1) * kF4VB + lb.v[0]);
    vsc = *reinterpret_cast<const int*>(vsring + (kF4NS - 1) * kF4SB + lb.vs);
  }
  const int nl = st.nload();

  int n = 0;
  int tc = t0, tn = t0 + 1, tnn = t0 + 2, tnnn = t0 + 3;  // T[n] .. T[n+3]
  auto step = [&](auto slot) -> bool {
    constexpr int Q = decltype(slot)::value;  // n % 4
    if (tc >= kt_end) return false;
    __syncthreads();
    st.load_v(clampt(tnn), vring + ((Q + 2) % kF4NS) * kF4VB, vsring + ((Q + 2) % kF4NS) * kF4SB);
    st.load_k(clampt(tnnn), kring + ((Q + 3) % kF4NS) * kF4KB, cring + ((Q + 3) % kF4NS) * kF4CB,
              ksring + ((Q + 3) % kF4NS) * kF4SB);
    const char* sVp = vring + ((Q + kF4NS - 1) % kF4NS) * kF4VB;  // V of T[n-1]
    const char* sVn = vring + Q * kF4VB;                          // V of T[n]
    const char* sVSn = vsring + Q * kF4SB;
    const int s1 = (Q + 1) % kF4NS;                               // K side of T[n+1]
    const bool part_nxt = partial(tn);
    float alpha;
    if (part_cur || part_nxt)
      alpha = f4_step<true>(acc, ch, P, vpre, vsc, sVp, sVn, sVSn, kring + s1 * kF4KB, cring + s1 * kF4CB,
                            ksring + s1 * kF4SB, qf, qsc, o, c, rs, lb, g, limit(tn));
    else
      alpha = f4_step<false>(acc, ch, P, vpre, vsc, sVp, sVn, sVSn, kring + s1 * kF4KB, cring + s1 * kF4CB,
                             ksring + s1 * kF4SB, qf, qsc, o, c, rs, lb, g, kBlockN - 1);
    if (__ballot(alpha != 1.f)) {  // O moves to T[n]'s maximum after the PV of T[n-1]
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    part_cur = part_nxt;
    if (nl == 1)
      wait_vmcnt<1>();
    else
      wait_vmcnt<2>();
    tc = tn;
    tn = tnn;
    tnn = tnnn;
    tnnn = tnnn + 1;
    ++n;
    return true;
  };
  // Phase-split step n: both groups read K of T[n+1] and V of T[n]; group 0 takes T[n]'s softmax
  // and then the MFMA phase, group 1 the MFMA phase and then T[n+1]'s softmax (past the last tile
  // every score is masked: P = 0, factor 1).
  auto pstep = [&](auto slot) -> bool {
    constexpr int Q = decltype(slot)::value;  // n % 4
    if (tc >= kt_end) return false;
    __syncthreads();
    auto stage = [&] {
      st.load_v(clampt(tnn), vring + ((Q + 2) % kF4NS) * kF4VB, vsring + ((Q + 2) % kF4NS) * kF4SB);
      st.load_k(clampt(tnnn), kring + ((Q + 3) % kF4NS) * kF4KB, cring + ((Q + 3) % kF4NS) * kF4CB,
                ksring + ((Q + 3) % kF4NS) * kF4SB);
    };
    const char* sV = vring + Q * kF4VB;  // V of T[n]
    const char* sVS = vsring + Q * kF4SB;
    const int s1 = (Q + 1) % kF4NS;      // K side of T[n+1]
    const char* sK = kring + s1 * kF4KB;
    // group 1 streams its MFMAs right after the barrier and stages the loads after them; group 0
    // stages first and reads its operands after its softmax
    if (grp1) {
      f4_mfma(*reinterpret_cast<const v4i*>(sK + lb.k[0]), sK, cring + s1 * kF4CB, ksring + s1 * kF4SB, sV, sVS, qf,
              qsc, P, o, acc, lb);
      stage();
    } else {
      stage();
    }
    const int ts = grp1 ? tn : tc;
    float alpha;
    if (partial(ts))
      alpha = f4_softmax<true>(acc, P, c, rs, g, limit(ts));
    else
      alpha = f4_softmax<false>(acc, P, c, rs, g, kBlockN - 1);
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    if (!grp1)
      f4_mfma(*reinterpret_cast<const v4i*>(sK + lb.k[0]), sK, cring + s1 * kF4CB, ksring + s1 * kF4SB, sV, sVS, qf,
              qsc, P, o, acc, lb);
    if (nl == 1)
      wait_vmcnt<1>();
    else
      wait_vmcnt<2>();
    tc = tn;
    tn = tnn;
    tnn = tnnn;
    tnnn = tnnn + 1;
    ++n;
    return true;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if constexpr (PP) {
    while (pstep(I0{}) && pstep(I1{}) && pstep(I2{}) && pstep(I3{})) {
    }
  } else {
    while (step(I0{}) && step(I1{}) && step(I2{}) && step(I3{})) {
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (!PP && n > 0) {  // PV of the last tile
    const int sl = (n - 1) % kF4NS;
    const char* sV = vring + sl * kF4VB;
    const int vs = *reinterpret_cast<const int*>(vsring + sl * kF4SB + lb.vs);
#pragma unroll
    for (int db = 0; db < 4; ++db) f4_pv(o, db, *reinterpret_cast<const v4i*>(sV + lb.v[db]), P, vs);
  }

  // epilogue: normalize, store O (bf16, fp16 or fp32) and the LSE.  O leaves through LDS: each wave
  // writes its 32 rows into its own region (rows of 256 bytes, 16-byte chunks XOR-swizzled by the
  // row) and reads them back so that consecutive lanes store consecutive 16-byte chunks of one row;
  // fp32 output takes two passes of 64 channels.
  const float l_tot = rs.l + __shfl_xor(rs.l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int RB = 2 * D, CPR = RB / 16;  // region row bytes, chunks per row
  __syncthreads();                          // every wave's last reads of the ring are done
  char* const so = smem + w * (32 * RB);
  const int64_t orow0 = b * a.o_sb + h * a.o_sh + (int64_t)r0w * a.o_sn;  // elements
  auto store_region = [&](char* outp, int osz, int ch0) {
    __syncthreads();  // the region is written
#pragma unroll
    for (int it = 0; it < CPR / 2; ++it) {
      const int r = it * (64 / CPR) + lane / CPR, c = lane % CPR;
      const v4i val = *reinterpret_cast<const v4i*>(so + r * RB + ((c ^ (r & (CPR - 1))) * 16));
      if (r0w + r < nq)
        *reinterpret_cast<v4i*>(outp + (orow0 + r * a.o_sn + ch0) * osz + c * 16) = val;
    }
  };
  if (a.out_kind == 2) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (pass) __syncthreads();  // the previous pass's reads of the region are done
#pragma unroll
      for (int db = 2 * pass; db < 2 * pass + 2; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int c = (db - 2 * pass) * 8 + rq * 2 + g;
          *reinterpret_cast<float4*>(so + lr * RB + ((c ^ (lr & (CPR - 1))) * 16)) =
              make_float4(o[db][rq * 4] * inv, o[db][rq * 4 + 1] * inv, o[db][rq * 4 + 2] * inv, o[db][rq * 4 + 3] * inv);
        }
      store_region(static_cast<char*>(a.out), 4, pass * 64);
    }
  } else {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = o[db][rq * 4 + e] * inv;
        uint2 pk;
        if (a.out_kind == 1) {
          pk.x = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[0], f[1]}), v2h));  // RNE
          pk.y = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[2], f[3]}), v2h));
        } else {
          pk.x = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[0], f[1]}), v2bf));  // RNE
          pk.y = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[2], f[3]}), v2bf));
        }
        const int c = db * 4 + rq;
        *reinterpret_cast<uint2*>(so + lr * RB + ((c ^ (lr & (CPR - 1))) * 16) + g * 8) = pk;
      }
    store_region(static_cast<char*>(a.out), 2, 0);
  }
  if (row < nq && g == 0 && a.lse) {
    float v = -INFINITY;
    if (l_tot > 0.f) v = (rs.pm + log2f(l_tot)) * kLn2 + a.sm_scale * a.lse_corr[bh * a.Nq + row];
    a.lse[bh * a.Nq + row] = v;
  }
}

// Raw scores S (before sm_scale) of a window of query head (b, h), by the attention kernel's tile
// code: grid = (32-row blocks, 64-key tiles) of the window, block = one wave.  The tile's K codes,
// the row block's correction row and the K scales are copied into the same LDS layout.
__global__ __launch_bounds__(64) void k_fp4_debug(Fp4DebugArgs d) {
  const Fp4AttnArgs& a = d.a;
  __shared__ __attribute__((aligned(16))) char sK[kF4KB];
  __shared__ __attribute__((aligned(16))) char sC[kF4CB];
  __shared__ __attribute__((aligned(16))) char sKS[kF4SB];
  const int lane = threadIdx.x, lr = lane & 31, g = lane >> 5;
  const int64_t bh = d.b * a.H + d.h, bhk = d.b * a.Hkv + d.h / (a.H / a.Hkv);
  const int64_t r0 = (d.row0 / 32 + blockIdx.x) * 32;
  const int64_t kt = d.col0 / kBlockN + blockIdx.y;
  const uint8_t* k4t = a.k4 + (bhk * a.Nk_pad + kt * kBlockN) * 64;
  for (int i = lane; i < kF4KB / 16; i += 64) {  // chunk i: tile row i / 4, logical chunk i % 4
    const int r = i >> 2, lc = i & 3;
    *reinterpret_cast<v4i*>(sK + r * 64 + ((lc ^ swz_f4(r)) << 4)) = *reinterpret_cast<const v4i*>(k4t + r * 64 + lc * 16);
  }
  const int64_t u = a.per_block ? r0 / kQMB : 0;
  const float* crow = a.qk_corr + (bh * a.nqm + (u < a.nqm ? u : a.nqm - 1)) * a.Nk_pad + kt * kBlockN;
  reinterpret_cast<float*>(sC)[lane] = crow[lane];  // the wave's Q block sits in row 0 of the tile buffer
  reinterpret_cast<int*>(sKS)[lane] = reinterpret_cast<const int*>(a.k_sc + (bhk * a.Nk_pad + kt * kBlockN) * 4)[lane];
  __syncthreads();
  F4Lanes lb;
  lb.init(lr, g, 0);
  v8i qf[2];
  const int64_t qrow = bh * a.Nq_pad + r0 + lr;
#pragma unroll
  for (int cs = 0; cs < 2; ++cs) qf[cs] = widen(*reinterpret_cast<const v4i*>(a.q4 + qrow * 64 + 32 * cs + 16 * g));
  const int qsc = *reinterpret_cast<const unsigned short*>(a.q_sc + qrow * 4 + 2 * g);
  v16f acc[2];
  f4_qk_tile(sK, sC, sKS, qf, qsc, lb, acc);
  const int64_t row = r0 + lr;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = kt * kBlockN + f4_key(kb, r, g);
      if (row >= d.row0 && row < d.row0 + d.nrows && j >= d.col0 && j < d.col0 + d.ncols)
        d.out[(row - d.row0) * d.ncols + (j - d.col0)] = acc[kb][r];
    }
}

// ---------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------
int64_t fp4_mean_partial_doubles(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  const int64_t kq = token_mean_partial_doubles(B, H, Nq, d), kk = token_mean_partial_doubles(B, Hkv, Nk, d);
  return kq > kk ? kq : kk;
}

// Key blocks per wave of k_fp4_corr for a total of wave_blocks (Q-block group, key block) pairs:
// about 768 waves (three per CU), at least 1 and at most 16 blocks each.  A wave's set-up (loading
// and splitting the means, its first loads) costs as much as several key blocks, so fewer, longer
// waves measure faster even below one wave per SIMD (on 24 heads x 4096 keys: 4 blocks per wave
// 14 us, 1 block 20 us; on 64 heads x 8192 keys x 2 groups: 16 blocks 63 us, 4 blocks 80 us).
static int fp4_corr_blocks_per_wave(int64_t wave_blocks) {
  const int64_t k = wave_blocks / 768;
  return (int)(k < 1 ? 1 : (k > 16 ? 16 : k));
}

template <int D, int IN>
static void launch_fp4_quant_t(const Fp4QuantArgs& a, hipStream_t s) {
  k_fp4_quant_q<D, IN><<<dim3((unsigned)(a.Nq_pad / kQMB), (unsigned)(a.B * a.H)), 2 * kF4Threads, 0, s>>>(a);
  k_fp4_quant_k<D, IN><<<dim3((unsigned)(a.Nk_pad / 64), (unsigned)(a.B * a.Hkv)), kF4Threads, 0, s>>>(a);
  k_fp4_prep_v<D, IN><<<dim3((unsigned)(a.Nk_pad / 64), (unsigned)(a.B * a.Hkv)), kF4Threads, 0, s>>>(a);
  const int64_t ngroups = (a.nqm + 31) / 32;
  const int kpw = fp4_corr_blocks_per_wave(a.B * a.H * ngroups * (a.Nk_pad / 32));
  const int64_t items = a.B * a.H * f4corr_chunks(a.Nk_pad, kpw);
  const int64_t nwg = (items + 7) / 8 * 8 * ngroups;
  for (int64_t wg0 = 0; wg0 < nwg; wg0 += kF4MaxCorrLaunch) {
    const unsigned g = (unsigned)(nwg - wg0 < kF4MaxCorrLaunch ? nwg - wg0 : kF4MaxCorrLaunch);
    k_fp4_corr<D, IN><<<g, kF4Threads, 0, s>>>(a, (int)ngroups, kpw, wg0);
  }
}

// K mean; the global Q mean (not per_block) into q_mean; then Q, K, V and the correction rows.
hipError_t launch_fp4_quant(const Fp4QuantArgs& a, double* partial, hipStream_t s) {
  hipError_t e = launch_token_mean(a.k, a.in_fp16, (int)a.d, a.B, a.Hkv, a.Nk, a.k_sb, a.k_sh, a.k_sn, partial,
                                   a.k_mean, s);
  if (e != hipSuccess) return e;
  if (!a.per_block) {
    e = launch_token_mean(a.q, a.in_fp16, (int)a.d, a.B, a.H, a.Nq, a.q_sb, a.q_sh, a.q_sn, partial, a.q_mean, s);
    if (e != hipSuccess) return e;
  }
  a.in_fp16 ? launch_fp4_quant_t<128, 1>(a, s) : launch_fp4_quant_t<128, 0>(a, s);  // d = 128 (host-checked)
  return hipGetLastError();
}

// The attention kernel runs the phase-split schedule (build with -DSAGE_PHASE_SPLIT=0 for the
// interleaved f4_step schedule, e.g. to compare the two).
#ifndef SAGE_PHASE_SPLIT
#define SAGE_PHASE_SPLIT 1
#endif
constexpr bool kPhaseSplitF4 = SAGE_PHASE_SPLIT;

hipError_t launch_fp4_attn(const Fp4AttnArgs& a, hipStream_t s) {
  if (kPhaseSplitF4)
    k_fp4_attn<1><<<(unsigned)(a.nQT * a.B * a.H), kF4AttnThreads, 0, s>>>(a);
  else
    k_fp4_attn<0><<<(unsigned)(a.nQT * a.B * a.H), kF4AttnThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp4_debug(const Fp4DebugArgs& d, hipStream_t s) {
  const int64_t rb0 = d.row0 / 32, rb1 = (d.row0 + d.nrows + 31) / 32;
  const int64_t kt0 = d.col0 / kBlockN, kt1 = (d.col0 + d.ncols + kBlockN - 1) / kBlockN;
  k_fp4_debug<<<dim3((unsigned)(rb1 - rb0), (unsigned)(kt1 - kt0)), 64, 0, s>>>(d);
  return hipGetLastError();
}

}  // namespace sage

namespace sage {
int fp4_softmax_tau() { return kF4Tau; }
}  // namespace sage
