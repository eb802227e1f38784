// sage_prep.hip -- HBM-streaming preparation kernels for the quantized attention forward (gfx950).
//
//   k_colred_partial  per-(b,h,256-token chunk) column sums of K in fp64 (K mean) or column
//                     maxima of |V| (fp8 V scale); fixed summation order, no atomics
//   k_kmean_final     k_mean[b,h,c] = fp32(sum over chunks / Nk)
//   k_quant_qk        per-64-token-block INT8 quantization of Q and of the smoothed K, their
//                     scales, and the LSE shift sum_c Q[i,c]*k_mean[c]
//   k_prep_v16        V (or, with smooth_v, fp32(V - mean)) -> fp16 (round to nearest even),
//                     transposed to [d][Nk_pad] in the key order the PV MFMA consumes
//   k_prep_v8         V -> e4m3 with per-channel scale 448/max|V|, transposed likewise
//   k_mask_tiles      classifies each (256-row x 64-key) tile of a boolean or fp32 additive mask
//                     as all-masked, all-visible (fp32: all exactly 0) or mixed, so the attention
//                     kernel skips a tile or reads no mask for it
//   k_mask_walk       adds to each tile's state the next tile of its row block that is not skipped
//
// Non-finite inputs: every maximum that sets a scale keeps NaN (mag_max), so a Q or K block or an
// FP8 V channel holding a NaN gets a NaN scale, and a NaN or +inf scale gives every code of its
// group the value 0; the means are plain sums.  The NaN then reaches the outputs through the
// scales and means instead of turning into finite codes.
//
// Method sources (page title, section): SageAttention docs digest (context7 llms.txt) --
// "sageattn_qk_int8_pv_fp16_triton" (per-block INT8 Q/K, smooth_k), "sageattn3_blackwell" usage
// (smoothing by the global token mean), "sageattn_qk_int8_pv_fp8_cuda" (per-channel FP8 V).
#include <limits.h>

#include <type_traits>

#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kChunk = 256;  // tokens per column-reduction chunk
constexpr int kPrepThreads = 256;
constexpr int kColredThreads = 512;

// ---------------------------------------------------------------------------------------------
// Column reductions over token chunks.  MODE 0: fp64 sums of x; MODE 1: fp32 maxima of |x|.
// x is bf16 (IN = 0) or fp16 (IN = 1).
// grid = (nchunk, B*H), block = 512.  Thread t covers channels [8*(t % (D/8)), +8) of the rows
// t / (D/8) + i * (512 / (D/8)) of the chunk; all of its loads are issued before the first is used.
// ---------------------------------------------------------------------------------------------
template <int D, int MODE, int IN>
__global__ __launch_bounds__(kColredThreads) void k_colred_partial(const unsigned short* __restrict__ x, int64_t H,
                                                                 int64_t Nmax, int64_t sb, int64_t sh, int64_t sn,
                                                                 void* __restrict__ partial, int nchunk,
                                                                 const int* __restrict__ cu, int64_t total) {
  constexpr int CG = D / 8;               // threads per row
  constexpr int RPI = kColredThreads / CG;  // rows per iteration
  const int t = threadIdx.x, cg = t % CG, rs = t / CG;
  const int64_t bh = blockIdx.y, b = bh / H, h = bh % H;
  const SeqSpan sp = seq_span(cu, b, Nmax, total);
  const int64_t N = sp.len;
  const int64_t t0 = (int64_t)blockIdx.x * kChunk;
  const unsigned short* base = x + b * sb + h * sh + sp.off * sn + cg * 8;
  double sum[8];
  float mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sum[j] = 0.0;
    mx[j] = 0.f;
  }
  // all of the chunk's loads are issued before the first is used (zero rows past N add nothing)
  constexpr int TPT = kChunk / RPI;
  u16x8 v[TPT];
  const int64_t nlast = N > 0 ? N - 1 : 0;  // rows past N read row N - 1 and count as zero; no loads if N = 0
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t tok = t0 + rs + i * RPI;
    v[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (N > 0) v[i] = *reinterpret_cast<const u16x8*>(base + (tok < N ? tok : nlast) * sn);
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t tok = t0 + rs + i * RPI;
      const float f = tok < N ? in_to_f32<IN>(v[i][j]) : 0.f;
      if constexpr (MODE == 0)
        sum[j] += (double)f;
      else
        mx[j] = mag_max(mx[j], fabsf(f));
    }
  // combine the RPI row-slices in a fixed order
  if constexpr (MODE == 0) {
    __shared__ double red[RPI][D];
#pragma unroll
    for (int j = 0; j < 8; ++j) red[rs][cg * 8 + j] = sum[j];
    __syncthreads();
    if (t < D) {
      double s = 0.0;
      for (int r = 0; r < RPI; ++r) s += red[r][t];
      static_cast<double*>(partial)[(bh * nchunk + blockIdx.x) * D + t] = s;
    }
  } else {
    __shared__ float red[RPI][D];
#pragma unroll
    for (int j = 0; j < 8; ++j) red[rs][cg * 8 + j] = mx[j];
    __syncthreads();
    if (t < D) {
      float m = 0.f;
      for (int r = 0; r < RPI; ++r) m = mag_max(m, red[r][t]);
      static_cast<float*>(partial)[(bh * nchunk + blockIdx.x) * D + t] = m;
    }
  }
}

// k_mean = fp32(sum_chunks partial / Nk); grid = B*H, block = D.  A sequence without keys gets 0.
template <int D>
__global__ __launch_bounds__(D) void k_kmean_final(const double* __restrict__ partial, int nchunk, int64_t H,
                                                   int64_t Nmax, const int* __restrict__ cu, int64_t total,
                                                   float* __restrict__ kmean) {
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  const int64_t N = seq_span(cu, bh / H, Nmax, total).len;
  double s = 0.0;
  int i = 0;
  for (; i + 8 <= nchunk; i += 8) {  // eight loads in flight, added in chunk order
    double p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = partial[(bh * nchunk + i + k) * D + c];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += p[k];
  }
  for (; i < nchunk; ++i) s += partial[(bh * nchunk + i) * D + c];
  kmean[bh * D + c] = N > 0 ? (float)(s / (double)N) : 0.f;
}

// block-wide maximum of a magnitude, NaN kept (256 threads)
__device__ __forceinline__ float block_max256(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = mag_max(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = mag_max(mag_max(red[0], red[1]), mag_max(red[2], red[3]));
  return r;
}

// ---------------------------------------------------------------------------------------------
// Per-block INT8 quantization.  grid = (Nq_pad/64 + Nk_pad/64, B*H), block = 256.
// Block x < Nq_pad/64 handles Q rows [64x, 64x+64) of query head y; the others handle K rows of
// key head y (only y < B*Hkv: the key heads of group-query attention).  Blocks past the last valid
// block only write zero pad rows.  Each thread holds 8 channels of RPB rows.  A query head's LSE
// shift uses the K mean of its key head h / (H / Hkv).  per_block_mean (kbmean set): a key block
// is smoothed by its own column means (fp64 sums of its valid rows, combined in a fixed order, one
// rounding), which it also writes out; the global K mean is then zero.
// ---------------------------------------------------------------------------------------------
template <int D, int IN>
__global__ __launch_bounds__(kPrepThreads) void k_quant_qk(QuantArgs a) {
  constexpr int CG = D / 8;
  constexpr int RPI = kPrepThreads / CG;  // 16 (D=128) or 32 (D=64)
  constexpr int RPB = kQuantBlock / RPI;  // rows per thread: 4 or 2
  __shared__ float red[4];
  __shared__ float km_s[D];
  const int t = threadIdx.x, cg = t % CG, rs = t / CG;
  const int nqb_pad = (int)(a.Nq_pad / kQuantBlock);
  const bool isq = (int)blockIdx.x < nqb_pad;
  // query blocks: bh indexes B*H query heads; key blocks: bh indexes B*Hkv key heads
  const int64_t nh = isq ? a.H : a.Hkv;
  const int64_t bh = blockIdx.y;
  if (bh >= a.B * nh) return;  // key blocks of the grid rows past the key heads
  const int64_t b = bh / nh, h = bh % nh;
  const int64_t bhk = isq ? b * a.Hkv + h / (a.H / a.Hkv) : bh;  // head of the K mean
  const int u = isq ? (int)blockIdx.x : (int)blockIdx.x - nqb_pad;
  const SeqSpan sp = isq ? seq_span(a.cu_q, b, a.Nq, a.total_q) : seq_span(a.cu_k, b, a.Nk, a.total_k);
  const int64_t N = sp.len;  // this sequence's tokens (dense: Nq or Nk)
  const int64_t Npad = isq ? a.Nq_pad : a.Nk_pad;
  int8_t* x8 = (isq ? a.q8 : a.k8) + (bh * Npad + (int64_t)u * kQuantBlock) * D;
  const int64_t r0 = (int64_t)u * kQuantBlock;

  if (r0 >= N) {  // pure pad block: zero codes, and a zero scale where the scale array has a slot
#pragma unroll
    for (int i = 0; i < RPB; ++i) {
      int r = rs + i * RPI;
      *reinterpret_cast<uint2*>(x8 + (int64_t)r * D + cg * 8) = make_uint2(0u, 0u);
    }
    if (t == 0 && u < (isq ? a.nbq : a.nbk)) (isq ? a.qs : a.ks)[bh * (isq ? a.nbq : a.nbk) + u] = 0.f;
    if (!isq && a.kbmean != nullptr && u < a.nbk && t < D) a.kbmean[(bh * a.nbk + u) * D + t] = 0.f;
    return;
  }

  if (t < D) km_s[t] = a.kmean[bhk * D + t];
  __syncthreads();

  const int64_t sn = isq ? a.q_sn : a.k_sn;
  const unsigned short* src =
      (isq ? a.q + b * a.q_sb + h * a.q_sh : a.k + b * a.k_sb + h * a.k_sh) + sp.off * sn + cg * 8;
  const bool pbm = !isq && a.kbmean != nullptr;  // uniform
  float x[RPB][8];
  float amax = 0.f;
  u16x8 raw[RPB];
#pragma unroll
  for (int i = 0; i < RPB; ++i) {  // every load in flight first; rows past N read row N - 1 (N > r0)
    const int64_t tok = r0 + rs + i * RPI;
    raw[i] = *reinterpret_cast<const u16x8*>(src + (tok < N ? tok : N - 1) * sn);
  }
  float kmr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kmr[j] = km_s[cg * 8 + j];
#pragma unroll
  for (int i = 0; i < RPB; ++i) {
    const bool valid = r0 + rs + i * RPI < N;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f = in_to_f32<IN>(raw[i][j]);
      if (!isq && !pbm) f = f - kmr[j];  // one fp32 rounding
      f = valid ? f : 0.f;
      x[i][j] = f;
      amax = mag_max(amax, fabsf(f));
    }
  }
  if (pbm) {  // the block's own column means, then the smoothed values and their amax
    __shared__ double colsum[RPI][D];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < RPB; ++i) s += (double)x[i][j];  // rows past N hold 0
      colsum[rs][cg * 8 + j] = s;
    }
    __syncthreads();
    if (t < D) {
      double s = 0.0;
      for (int r = 0; r < RPI; ++r) s += colsum[r][t];
      const int64_t nv = N - r0 < kQuantBlock ? N - r0 : kQuantBlock;
      const float m = (float)(s / (double)nv);
      km_s[t] = m;
      a.kbmean[(bh * a.nbk + u) * D + t] = m;
    }
    __syncthreads();
    amax = 0.f;
#pragma unroll
    for (int i = 0; i < RPB; ++i) {
      const bool valid = r0 + rs + i * RPI < N;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = valid ? x[i][j] - km_s[cg * 8 + j] : 0.f;  // one fp32 rounding
        x[i][j] = f;
        amax = mag_max(amax, fabsf(f));
      }
    }
  }
  amax = block_max256(amax, red);
  float scale = 0.f, inv = 0.f;
  if (amax != 0.f) {  // a NaN or +inf block too: scale NaN / +inf, inverse NaN / 0
    scale = amax / 127.0f;  // IEEE-correct binary32 division
    inv = 127.0f / amax;
  }
  if (t == 0) (isq ? a.qs : a.ks)[bh * (isq ? a.nbq : a.nbk) + u] = scale;
#pragma unroll
  for (int i = 0; i < RPB; ++i) {
    unsigned lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = x[i][j] * inv;
      float q = __builtin_rintf(y);  // round to nearest even
      q = y != y ? 0.f : fminf(fmaxf(q, -127.f), 127.f);  // NaN (a NaN or +inf block) codes 0
      unsigned byte = (unsigned)((int)q) & 0xffu;
      if (j < 4)
        lo |= byte << (8 * j);
      else
        hi |= byte << (8 * (j - 4));
    }
    int r = rs + i * RPI;
    *reinterpret_cast<uint2*>(x8 + (int64_t)r * D + cg * 8) = make_uint2(lo, hi);
  }
  if (isq) {
    // LSE shift: sum_c fp64(Q[i,c]) * fp64(k_mean[c]); the CG threads of a row are adjacent lanes
#pragma unroll
    for (int i = 0; i < RPB; ++i) {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) s += (double)x[i][j] * (double)kmr[j];
#pragma unroll
      for (int o = 1; o < CG; o <<= 1) s += __shfl_xor(s, o);
      int64_t tok = r0 + rs + i * RPI;
      if (cg == 0 && tok < N) a.corr[bh * a.Nq + tok] = (float)s;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// per_block_mean score terms: blk_corr[b,h,u,i] = sum_c Q[i,c] * kbmean[b,hk,u,c] for the valid key
// blocks u and query rows i of the sequence, on the matrix cores: D (32 blocks x 32 query rows) +=
// M (32 x 16) Q^T (16 x 32) per 16 channels.  Q enters exactly (it is bf16 / fp16 already); each
// fp32 block mean is split into a sum of input-format parts (bf16: three parts, 24 significant
// bits; fp16: two parts, 22 bits) -- the rounding residue of a part is exact in fp32 -- so the
// products are exact and only the fp32 accumulation rounds.
// A wave splits the means of one group of 32 key blocks once, keeps the parts in registers and
// streams up to kpw blocks of 32 query rows past them.  Work item c = (b*H + h) * nchunk + chunk
// covers 4 * kpw row blocks (wave w takes blocks 4 i + w of the chunk); the ngroups workgroups of
// one item sit 8 apart in launch order, so they run on one XCD (workgroups are dealt to the 8 XCDs
// in turn) and read its Q rows through one L2.  Stores outside the sequence's rows and key blocks
// go to an offset past the head's buffer range, which the hardware drops.
// ---------------------------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v8f __attribute__((ext_vector_type(8)));

// Workgroup ids per launch of k_block_corr, whose id count grows with Nq * Nk: larger problems
// take several launches, each from an offset wg0 that is a multiple of 8 (the id's XCD is kept).
constexpr int64_t kMaxCorrLaunch = (int64_t)1 << 20;

__host__ __device__ constexpr int64_t block_corr_chunks(int64_t Nq, int kpw) {
  return ((Nq + 31) / 32 + 4 * kpw - 1) / (4 * kpw);
}

template <int D, int IN>
__global__ __launch_bounds__(kPrepThreads) void k_block_corr(QuantArgs a, int ngroups, int kpw, int64_t wg0) {
  using V8 = typename std::conditional<IN == 0, v8bf, v8h>::type;
  constexpr int NP = IN == 0 ? 3 : 2;  // parts of a mean
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 31, g = lane >> 5;
  const int64_t nchunk = block_corr_chunks(a.Nq, kpw);
  const int64_t wg = wg0 + blockIdx.x, grp = (wg >> 3) % ngroups, c = (wg & 7) + 8 * ((wg >> 3) / ngroups);
  if (c >= a.B * a.H * nchunk) return;
  const int64_t bh = c / nchunk, b = bh / a.H, h = bh % a.H;
  const int64_t bhk = b * a.Hkv + h / (a.H / a.Hkv);
  const SeqSpan sp = seq_span(a.cu_q, b, a.Nq, a.total_q);
  const SeqSpan sk = seq_span(a.cu_k, b, a.Nk, a.total_k);
  const int nbk_b = (int)((sk.len + kQuantBlock - 1) / kQuantBlock);
  if (32 * grp >= nbk_b || sp.len <= 0) return;
  const int64_t nrb = (sp.len + 31) / 32;
  const int64_t rb0 = (c % nchunk) * 4 * kpw + w;
  int64_t nb = (nrb - rb0 + 3) / 4;
  nb = nb < kpw ? nb : kpw;  // row blocks rb0, rb0 + 4, ... of this wave
  if (nb <= 0) return;
  // A operand: key block u = 32 grp + lr, channels 16 kk + 8 g .. + 8, as NP exact parts
  const int u = 32 * (int)grp + lr;
  const float* mp = a.kbmean + (bhk * a.nbk + (u < nbk_b ? u : 0)) * D + 8 * g;
  V8 ap[D / 16][NP];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    v8f m = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (u < nbk_b) {
      const float4 lo = *reinterpret_cast<const float4*>(mp + 16 * kk);
      const float4 hi = *reinterpret_cast<const float4*>(mp + 16 * kk + 4);
      m = v8f{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {  // m = part[0] + part[1] (+ part[2]), residues exact in fp32
      ap[kk][p] = __builtin_convertvector(m, V8);  // round to nearest even
      m = m - __builtin_convertvector(ap[kk][p], v8f);
    }
  }
  // B operand: query row 32 rb + lr, channels 16 kk + 8 g .. + 8 (a row past the sequence reads
  // its last row; its column is not stored)
  const unsigned short* qh = a.q + b * a.q_sb + h * a.q_sh + sp.off * a.q_sn + 8 * g;
  auto load_q = [&](int64_t rb, u16x8(&r)[D / 16]) {
    const int64_t row = 32 * rb + lr;
    const unsigned short* src = qh + (row < sp.len ? row : sp.len - 1) * a.q_sn;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) r[kk] = *reinterpret_cast<const u16x8*>(src + 16 * kk);
  };
  // this head's terms, nbk * Nq * 4 < 2^31 bytes (host-checked)
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.blk_corr + bh * a.nbk * a.Nq), (short)0, (int)(a.nbk * a.Nq * 4), kBufferWord3);
  constexpr int kOutOfRange = 0x7ffffffc;
  auto block = [&](int64_t rb, const u16x8(&qr)[D / 16]) {
    v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const V8 qb = __builtin_bit_cast(V8, qr[kk]);
#pragma unroll
      for (int p = NP - 1; p >= 0; --p) {  // smallest part first
        if constexpr (IN == 0)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[kk][p], qb, acc, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[kk][p], qb, acc, 0, 0, 0);
      }
    }
    const int64_t row = 32 * rb + lr;  // D column lr
#pragma unroll
    for (int r = 0; r < 16; ++r) {  // D row (r/4)*8 + 4g + r%4 is key block 32 grp + that
      const int ub = 32 * (int)grp + (r >> 2) * 8 + g * 4 + (r & 3);
      const int off = (ub < nbk_b && row < sp.len) ? (int)(((int64_t)ub * a.Nq + row) * 4) : kOutOfRange;
      // copied to a scalar first: hipcc compiles __builtin_bit_cast of a vector element (acc[r])
      // as element 0 for every r
      const float x = acc[r];
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), crs, off, 0, 0);
    }
  };
  // Two register buffers: the next block's loads are issued before the current block's products
  // (past the end, a block reloads itself).
  auto rb_of = [&](int64_t i) { return rb0 + 4 * (i < nb ? i : nb - 1); };
  u16x8 qa[D / 16], qz[D / 16];
  load_q(rb_of(0), qa);
  for (int64_t i = 0; i < nb; i += 2) {
    load_q(rb_of(i + 1), qz);
    __builtin_amdgcn_sched_barrier(0);
    block(rb_of(i), qa);
    if (i + 1 >= nb) break;
    load_q(rb_of(i + 2), qa);
    __builtin_amdgcn_sched_barrier(0);
    block(rb_of(i + 1), qz);
  }
}

// ---------------------------------------------------------------------------------------------
// V preparation.  Each 64-token x D tile is converted and written transposed: row c of v_t holds
// the tile's 64 keys of channel c, in the MFMA key order.
// ---------------------------------------------------------------------------------------------
// position p (0..15) inside a 16-key group holds key ((p & 7) >> 2) * 8 + (p >> 3) * 4 + (p & 3)
__device__ __forceinline__ int fp16_pos_to_key(int p) { return ((p & 7) >> 2) * 8 + (p >> 3) * 4 + (p & 3); }
// position p (0..63) inside a 64-key group: g = p/32, kb = (p/16)%2, r = p%16;
// key = kb*32 + (r/4)*8 + g*4 + r%4
__device__ __forceinline__ int fp8_pos_to_key(int p) {
  int g = p >> 5, kb = (p >> 4) & 1, r = p & 15;
  return kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
}

// Each thread converts 8 keys x 8 channels with no LDS: it loads the 8 keys that fill positions
// [8 pg, 8 pg + 8) of the tile (keys 16 (pg / 2) + pos_to_key(8 (pg % 2) + e), e = 0..7), 16 bytes
// of each key's row, and writes, per channel, the 16 bytes of those positions.  Two neighbouring
// positions of one channel come out of one v_cvt_pk_f16_f32, which also transposes.  A workgroup
// covers 256 / (8 * D/8) tiles of 64 keys; grid = (ceil(Nk_pad / 64 / tiles per workgroup), B*H).
template <int D, int IN>
__global__ __launch_bounds__(kPrepThreads) void k_prep_v16(PrepVArgs a) {
  constexpr int CG = D / 8;
  constexpr int TT = 8 * CG;                // threads per 64-key tile
  constexpr int TPW = kPrepThreads / TT;    // tiles per workgroup
  // lanes next to each other take neighbouring position groups of one channel group, so a store
  // instruction writes 128 contiguous bytes of each of 8 channel rows
  const int t = threadIdx.x, tt = t % TT, pg = tt % 8, cg = tt / 8;
  const int64_t kt = (int64_t)blockIdx.x * TPW + t / TT;
  if (kt * 64 >= a.Nk_pad) return;
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t k0 = kt * 64;
  const SeqSpan sp = seq_span(a.cu_k, b, a.Nk, a.total_k);
  const unsigned short* src = a.v + b * a.v_sb + h * a.v_sh + sp.off * a.v_sn + cg * 8;
  const int64_t nlast = sp.len > 0 ? sp.len - 1 : 0;
  u16x8 raw[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // every load in flight first; keys past the sequence read its last key
    const int64_t tok = k0 + 16 * (pg >> 1) + fp16_pos_to_key(8 * (pg & 1) + e);
    raw[e] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (sp.len > 0) raw[e] = *reinterpret_cast<const u16x8*>(src + (tok < sp.len ? tok : nlast) * a.v_sn);
  }
  float vm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vm[j] = a.vmean ? a.vmean[bh * D + cg * 8 + j] : 0.f;  // smooth_v
  unsigned short* dst = static_cast<unsigned short*>(a.vt) + (bh * D + cg * 8) * a.Nk_pad + k0 + 8 * pg;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v4i o;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float x2[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * m + q;
        const int64_t tok = k0 + 16 * (pg >> 1) + fp16_pos_to_key(8 * (pg & 1) + e);
        float x = in_to_f32<IN>(raw[e][j]);
        if (a.vmean) x = x - vm[j];  // one fp32 rounding
        x2[q] = tok < sp.len ? x : 0.f;  // pad keys 0
      }
      // round to nearest even (exact for fp16 V)
      o[m] = __builtin_bit_cast(int, __builtin_convertvector((v2f{x2[0], x2[1]}), v2h));
    }
    *reinterpret_cast<v4i*>(dst + (int64_t)j * a.Nk_pad) = o;
  }
}

// max over chunks of the column maxima of k_colred_partial<MODE 1>, written over the first chunk's
// entry (grid = B*H, block = D; eight loads in flight per step)
template <int D>
__global__ __launch_bounds__(D) void k_vmax_final(float* __restrict__ partial, int nchunk) {
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  float m = 0.f;
  int i = 0;
  for (; i + 8 <= nchunk; i += 8) {
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = partial[(bh * nchunk + i + k) * D + c];
#pragma unroll
    for (int k = 0; k < 8; ++k) m = mag_max(m, p[k]);
  }
  for (; i < nchunk; ++i) m = mag_max(m, partial[(bh * nchunk + i) * D + c]);
  partial[(bh * nchunk) * D + c] = m;
}

// V -> e4m3.  The per-channel maxima come from k_colred_partial<MODE 1> and k_vmax_final.  The
// tile goes through LDS as its raw 16-bit inputs (half the bytes of fp32: twice the workgroups per
// CU to hide the loads); the scaling and saturation follow the LDS read.
template <int D, int IN>
__global__ __launch_bounds__(kPrepThreads) void k_prep_v8(PrepVArgs a) {
  constexpr int CG = D / 8;
  constexpr int RPI = kPrepThreads / CG;
  __shared__ unsigned short tile[64][D + 2];
  __shared__ float inv_s[D];
  const int t = threadIdx.x, cg = t % CG, rs = t / CG;
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  if (t < D) {
    const float m = a.vmax_partial[(bh * a.nchunk) * D + t];  // max over chunks (k_vmax_final)
    float sc = 0.f, inv = 0.f;
    if (m != 0.f) {  // NaN and +inf included, as for the INT8 blocks
      sc = m / 448.0f;
      inv = 448.0f / m;
    }
    inv_s[t] = inv;
    if (blockIdx.x == 0) a.vscale[bh * D + t] = sc;
  }
  __syncthreads();
  const SeqSpan sp = seq_span(a.cu_k, b, a.Nk, a.total_k);
  const unsigned short* src = a.v + b * a.v_sb + h * a.v_sh + sp.off * a.v_sn + cg * 8;
  for (int r = rs; r < 64; r += RPI) {
    int64_t tok = k0 + r;
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (tok < sp.len) v = *reinterpret_cast<const u16x8*>(src + tok * a.v_sn);
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[r][cg * 8 + j] = v[j];
  }
  __syncthreads();
  // D rows x 4 chunks of 16 bytes; chunk q holds positions [16q, 16q+16)
  uint8_t* dst = static_cast<uint8_t*>(a.vt) + (bh * D) * a.Nk_pad + k0;
  for (int i = t; i < D * 4; i += kPrepThreads) {
    int c = i / 4, q = i % 4;
    const float inv = inv_s[c];
    auto x = [&](int key) {
      float f = in_to_f32<IN>(tile[key][c]) * inv;
      f = f != f ? 0.f : f;                               // a NaN or +inf channel codes 0
      return fabsf(f) > 448.f ? copysignf(448.f, f) : f;  // saturate
    };
    v4i o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int p = q * 16 + w * 4;
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x(fp8_pos_to_key(p)), x(fp8_pos_to_key(p + 1)), 0, false);
      o[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x(fp8_pos_to_key(p + 2)), x(fp8_pos_to_key(p + 3)), lo, true);
    }
    *reinterpret_cast<v4i*>(dst + (int64_t)c * a.Nk_pad + q * 16) = o;
  }
}

// ---------------------------------------------------------------------------------------------
// Mask tile classification.  grid = (nKT, nQT, B*Hm), block = 256.
// state: 0 = every (valid) entry masked, 1 = every valid entry visible with nothing added (boolean:
// nonzero; fp32: exactly +-0), 2 = anything else.  Entries beyond Nq / Nk do not count.  F32: the
// mask is fp32 and additive, -inf masks.  A whole 16-byte-aligned tile is read in 16-byte chunks,
// consecutive lanes along a row (4 lanes a row for a boolean tile row of 64 bytes, 16 for fp32's
// 256 bytes), every load issued before the first is classified; a ragged or unaligned tile is read
// one row per thread.
// ---------------------------------------------------------------------------------------------
// key tiles per classification workgroup: a boolean workgroup reads whole 128-byte lines of its rows
template <bool F32>
constexpr int kMaskTilesPerGroup = F32 ? 1 : 2;

template <bool F32>
__device__ __forceinline__ void mask_classify16(uint4 w, int& any0, int& any1, int& anyx) {
  const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (F32) {
      const float v = __uint_as_float(ws[e]);
      any0 |= v == -INFINITY;
      any1 |= v == 0.f;
      anyx |= v != -INFINITY && v != 0.f;
    } else {
      const unsigned v = ws[e];
      // per byte: zero -> any0, nonzero -> any1
      const unsigned nz = ((v & 0x7f7f7f7fu) + 0x7f7f7f7fu | v) & 0x80808080u;
      any1 |= nz != 0u;
      any0 |= nz != 0x80808080u;
    }
  }
}

template <bool F32>
__global__ __launch_bounds__(kPrepThreads) void k_mask_tiles(MaskTileArgs a) {
  constexpr int ESZ = F32 ? 4 : 1;
  constexpr int TPW = kMaskTilesPerGroup<F32>;  // key tiles per workgroup
  const int kt0 = (int)blockIdx.x * TPW, qt = blockIdx.y;
  const int64_t bm = blockIdx.z, b = bm / a.Hm, hm = bm % a.Hm;
  const int64_t i0 = (int64_t)qt * kMaskTileRows;
  const int64_t j0 = (int64_t)kt0 * kBlockN;
  const char* head = static_cast<const char*>(a.mask) + (b * a.sb + hm * a.sh) * ESZ;
  unsigned flags = 0;  // for tile kt0 + t, bit 3t: a masked entry, 3t + 1: a plainly visible one, 3t + 2: other
  if (a.vec16 && a.Nk - j0 >= (int64_t)TPW * kBlockN) {
    constexpr int CPR = TPW * kBlockN * ESZ / 16;  // 16-byte chunks per row of the group's tiles
    constexpr int RPP = kPrepThreads / CPR;        // rows per pass
    constexpr int NP = kMaskTileRows / RPP;        // passes
    const int c = threadIdx.x % CPR, r = threadIdx.x / CPR;
    uint4 w[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t i = i0 + r + p * RPP;
      w[p] = make_uint4(0u, 0u, 0u, 0u);
      if (i < a.Nq) w[p] = *reinterpret_cast<const uint4*>(head + (i * a.sq + j0) * ESZ + c * 16);
    }
    int any0 = 0, any1 = 0, anyx = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (i0 + r + p * RPP < a.Nq) mask_classify16<F32>(w[p], any0, any1, anyx);
    const int t = c / (CPR / TPW);
    flags = (unsigned)(any0 | any1 << 1 | anyx << 2) << (3 * t);
  } else {
    const int64_t i = i0 + threadIdx.x;
    for (int t = 0; t < TPW && kt0 + t < a.nKT; ++t) {
      const int64_t jt = j0 + (int64_t)t * kBlockN;
      const int64_t jn = a.Nk - jt < kBlockN ? a.Nk - jt : kBlockN;
      int any0 = 0, any1 = 0, anyx = 0;
      if (i < a.Nq) {
        if constexpr (F32) {
          const float* row = reinterpret_cast<const float*>(head) + i * a.sq + jt;
          for (int64_t j = 0; j < jn; ++j) {
            const float v = row[j];
            any0 |= v == -INFINITY;
            any1 |= v == 0.f;
            anyx |= v != -INFINITY && v != 0.f;
          }
        } else {
          const uint8_t* row = reinterpret_cast<const uint8_t*>(head) + i * a.sq + jt;
          for (int64_t j = 0; j < jn; ++j) {
            const uint8_t v = row[j];
            any1 |= v != 0;
            any0 |= v == 0;
          }
        }
      }
      flags |= (unsigned)(any0 | any1 << 1 | anyx << 2) << (3 * t);
    }
  }
  // OR of the flags over the workgroup
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) flags |= __shfl_xor(flags, o);
  __shared__ unsigned wflags[kPrepThreads / 64];
  if ((threadIdx.x & 63) == 0) wflags[threadIdx.x >> 6] = flags;
  __syncthreads();
  if (threadIdx.x < TPW && kt0 + (int)threadIdx.x < a.nKT) {
    unsigned f = 0;
#pragma unroll
    for (int wv = 0; wv < kPrepThreads / 64; ++wv) f |= wflags[wv];
    f >>= 3 * threadIdx.x;
    const bool z = f & 1u, o = f & 2u, x = f & 4u;
    a.state[(bm * a.nQT + qt) * a.nKT + kt0 + threadIdx.x] = x || (z && o) ? 2 : (o ? 1 : 0);
  }
}

// The walk over a row block's key tiles: each entry of the state table gets, above its state (bits
// 0-1), the index of the next tile after it that is not all-masked (nKT if there is none), so the
// attention kernel steps from tile to tile with one load instead of a loop over dropped tiles.  One
// wave per (mask batch, head, row block) row of the table takes it 64 entries at a time from the
// end: a suffix minimum across the lanes gives each entry the first kept tile at or after it, and
// the chunk's minimum carries over to the chunk before it.
__global__ __launch_bounds__(64) void k_mask_walk(int* __restrict__ state, int nKT) {
  int* row = state + (int64_t)blockIdx.x * nKT;
  const int lane = threadIdx.x;
  int carry = nKT;  // the first kept tile after this chunk
  for (int base = ((nKT - 1) / 64) * 64; base >= 0; base -= 64) {
    const int kt = base + lane;
    const int st = kt < nKT ? row[kt] & 3 : 0;
    int v = st != 0 ? kt : INT_MAX;  // (entries past nKT have st = 0)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_down(v, off);
      if (lane + off < 64) v = v < o ? v : o;  // minimum over lanes [lane, 63] of this chunk
    }
    int nxt = __shfl_down(v, 1);
    if (lane == 63) nxt = INT_MAX;
    nxt = nxt < carry ? nxt : carry;
    if (kt < nKT) row[kt] = st | (nxt << 2);
    const int cmin = __shfl(v, 0);
    carry = cmin < carry ? cmin : carry;
  }
}

// ---------------------------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------------------------
template <int D, int IN>
static void launch_kmean_t(const QuantArgs& a, double* partial, int nchunk, hipStream_t s) {
  if (a.kbmean) {  // per_block_mean: the global mean is zero (no chunks summed)
    k_kmean_final<D><<<(unsigned)(a.B * a.Hkv), D, 0, s>>>(partial, 0, a.Hkv, a.Nk, a.cu_k, a.total_k, a.kmean);
    return;
  }
  dim3 g(nchunk, (unsigned)(a.B * a.Hkv));
  k_colred_partial<D, 0, IN><<<g, kColredThreads, 0, s>>>(a.k, a.Hkv, a.Nk, a.k_sb, a.k_sh, a.k_sn, partial, nchunk,
                                                        a.cu_k, a.total_k);
  k_kmean_final<D><<<(unsigned)(a.B * a.Hkv), D, 0, s>>>(partial, nchunk, a.Hkv, a.Nk, a.cu_k, a.total_k, a.kmean);
}

hipError_t launch_kmean(const QuantArgs& a, double* partial, int nchunk, hipStream_t s) {
  if (a.d == 128)
    a.in_fp16 ? launch_kmean_t<128, 1>(a, partial, nchunk, s) : launch_kmean_t<128, 0>(a, partial, nchunk, s);
  else
    a.in_fp16 ? launch_kmean_t<64, 1>(a, partial, nchunk, s) : launch_kmean_t<64, 0>(a, partial, nchunk, s);
  return hipGetLastError();
}

// Per-(b,h,channel) token mean of x [B][H][N][d] (fp64 chunk sums, one rounding to fp32), the same
// reduction as the K mean; partial holds token_mean_partial_doubles() doubles.
int64_t token_mean_partial_doubles(int64_t B, int64_t H, int64_t N, int64_t d) {
  return B * H * ((N + kChunk - 1) / kChunk) * d;
}

template <int D, int IN>
static void launch_token_mean_t(const unsigned short* x, int64_t B, int64_t H, int64_t N, int64_t sb, int64_t sh,
                                int64_t sn, double* partial, float* mean, hipStream_t s) {
  const int nchunk = (int)((N + kChunk - 1) / kChunk);
  dim3 g(nchunk, (unsigned)(B * H));
  k_colred_partial<D, 0, IN><<<g, kColredThreads, 0, s>>>(x, H, N, sb, sh, sn, partial, nchunk, nullptr, 0);
  k_kmean_final<D><<<(unsigned)(B * H), D, 0, s>>>(partial, nchunk, H, N, nullptr, 0, mean);
}

hipError_t launch_token_mean(const unsigned short* x, int in_fp16, int d, int64_t B, int64_t H, int64_t N, int64_t sb,
                             int64_t sh, int64_t sn, double* partial, float* mean, hipStream_t s) {
  if (d == 128)
    in_fp16 ? launch_token_mean_t<128, 1>(x, B, H, N, sb, sh, sn, partial, mean, s)
            : launch_token_mean_t<128, 0>(x, B, H, N, sb, sh, sn, partial, mean, s);
  else
    in_fp16 ? launch_token_mean_t<64, 1>(x, B, H, N, sb, sh, sn, partial, mean, s)
            : launch_token_mean_t<64, 0>(x, B, H, N, sb, sh, sn, partial, mean, s);
  return hipGetLastError();
}

// Row blocks per wave of k_block_corr for wave_blocks (key-block group, row block) pairs in all:
// about 768 waves (three per CU), 1 to 16 blocks each -- a wave's set-up (loading and splitting its
// means) costs several blocks, so fewer, longer waves are faster.
static int block_corr_rows_per_wave(int64_t wave_blocks) {
  const int64_t k = wave_blocks / 768;
  return (int)(k < 1 ? 1 : (k > 16 ? 16 : k));
}

hipError_t launch_block_corr(const QuantArgs& a, hipStream_t s) {
  const int64_t ngroups = (a.nbk + 31) / 32;
  const int kpw = block_corr_rows_per_wave(a.B * a.H * ngroups * ((a.Nq + 31) / 32));
  const int64_t items = a.B * a.H * block_corr_chunks(a.Nq, kpw);
  const int64_t nwg = (items + 7) / 8 * 8 * ngroups;
  const int ng = (int)ngroups;
  for (int64_t wg0 = 0; wg0 < nwg; wg0 += kMaxCorrLaunch) {
    const unsigned g = (unsigned)(nwg - wg0 < kMaxCorrLaunch ? nwg - wg0 : kMaxCorrLaunch);
    if (a.d == 128)
      a.in_fp16 ? k_block_corr<128, 1><<<g, kPrepThreads, 0, s>>>(a, ng, kpw, wg0)
                : k_block_corr<128, 0><<<g, kPrepThreads, 0, s>>>(a, ng, kpw, wg0);
    else
      a.in_fp16 ? k_block_corr<64, 1><<<g, kPrepThreads, 0, s>>>(a, ng, kpw, wg0)
                : k_block_corr<64, 0><<<g, kPrepThreads, 0, s>>>(a, ng, kpw, wg0);
  }
  return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t s) {
  dim3 g((unsigned)(a.Nq_pad / kQuantBlock + a.Nk_pad / kQuantBlock), (unsigned)(a.B * a.H));
  if (a.d == 128)
    a.in_fp16 ? k_quant_qk<128, 1><<<g, kPrepThreads, 0, s>>>(a) : k_quant_qk<128, 0><<<g, kPrepThreads, 0, s>>>(a);
  else
    a.in_fp16 ? k_quant_qk<64, 1><<<g, kPrepThreads, 0, s>>>(a) : k_quant_qk<64, 0><<<g, kPrepThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, int IN>
static void launch_prep_v_t(const PrepVArgs& a, int pv_fp8, hipStream_t s) {
  if (!pv_fp8) {
    constexpr int tpw = kPrepThreads / D;  // 64-key tiles per workgroup of k_prep_v16
    const dim3 g16((unsigned)((a.Nk_pad / 64 + tpw - 1) / tpw), (unsigned)(a.B * a.H));
    if (a.vmean) {  // smooth_v: V's channel means first, exactly as K's
      dim3 gr(a.nchunk, (unsigned)(a.B * a.H));
      k_colred_partial<D, 0, IN><<<gr, kColredThreads, 0, s>>>(a.v, a.H, a.Nk, a.v_sb, a.v_sh, a.v_sn, a.vsum_partial,
                                                            a.nchunk, a.cu_k, a.total_k);
      k_kmean_final<D><<<(unsigned)(a.B * a.H), D, 0, s>>>(a.vsum_partial, a.nchunk, a.H, a.Nk, a.cu_k, a.total_k,
                                                          a.vmean);
    }
    k_prep_v16<D, IN><<<g16, kPrepThreads, 0, s>>>(a);
  } else {
    dim3 gr(a.nchunk, (unsigned)(a.B * a.H));
    k_colred_partial<D, 1, IN><<<gr, kColredThreads, 0, s>>>(a.v, a.H, a.Nk, a.v_sb, a.v_sh, a.v_sn, a.vmax_partial,
                                                          a.nchunk, a.cu_k, a.total_k);
    k_vmax_final<D><<<(unsigned)(a.B * a.H), D, 0, s>>>(a.vmax_partial, a.nchunk);
    const dim3 g8((unsigned)(a.Nk_pad / 64), (unsigned)(a.B * a.H));
    k_prep_v8<D, IN><<<g8, kPrepThreads, 0, s>>>(a);
  }
}

hipError_t launch_prep_v(const PrepVArgs& a, int pv_fp8, hipStream_t s) {
  if (a.d == 128)
    a.in_fp16 ? launch_prep_v_t<128, 1>(a, pv_fp8, s) : launch_prep_v_t<128, 0>(a, pv_fp8, s);
  else
    a.in_fp16 ? launch_prep_v_t<64, 1>(a, pv_fp8, s) : launch_prep_v_t<64, 0>(a, pv_fp8, s);
  return hipGetLastError();
}

hipError_t launch_mask_tiles(const MaskTileArgs& a, hipStream_t s) {
  const unsigned gq = (unsigned)a.nQT, gb = (unsigned)(a.B * a.Hm);
  if (a.f32) {
    constexpr int T = kMaskTilesPerGroup<true>;
    k_mask_tiles<true><<<dim3((unsigned)((a.nKT + T - 1) / T), gq, gb), kPrepThreads, 0, s>>>(a);
  } else {
    constexpr int T = kMaskTilesPerGroup<false>;
    k_mask_tiles<false><<<dim3((unsigned)((a.nKT + T - 1) / T), gq, gb), kPrepThreads, 0, s>>>(a);
  }
  const int64_t rows = a.B * a.Hm * a.nQT;  // one wave per row of the table
  k_mask_walk<<<(unsigned)rows, 64, 0, s>>>(a.state, a.nKT);
  return hipGetLastError();
}

}  // namespace sage
