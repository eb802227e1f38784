// sage_attn.hip -- the quantized attention forward kernel for gfx950, and the debug kernel that
// exposes its int32 QK^T scores.
//
// Method (SageAttention docs digest, context7 llms.txt): per-block INT8 Q and smoothed K, INT8
// Q K^T with int32 accumulation, dequantization by q_scale * k_scale * sm_scale, online softmax,
// P V in FP16 ("sageattn_qk_int8_pv_fp16_triton", "SageAttention CUDA INT8/FP16 Kernel (Ampere
// sm80)", pv_accum_dtype="fp32") or with per-channel FP8 V ("sageattn_qk_int8_pv_fp8_cuda");
// keys at or beyond the logical length are masked before the softmax (FlashInfer API doc
// "flashinfer.nvfp4_attention_sm120_fwd", parameter unpadded_k_len).
//
// Design (MI355X / CDNA4):
//  * One workgroup = 8 waves = 256 query rows of one (b,h); each wave owns 32 rows.  Two waves
//    share a SIMD, so one wave's MFMAs overlap the other's softmax VALU work.
//  * S^T = K8 . Q8^T on v_mfma_i32_32x32x32_i8: the K tile (A operand) comes from LDS, the
//    wave's Q8 rows (B operand) stay in registers for the whole key loop.  In the 32x32 output
//    layout each lane holds one query row and 16 of every 32 keys, so the row max and row sum are
//    in-lane except for one exchange with lane ^ 32.
//  * O^T += V^T . P^T on v_mfma_f32_32x32x16_f16 (or the 32x32x64 f8f6f4 MFMA with unit scales
//    for e4m3): P goes from the QK accumulator registers straight into the B operand.  The
//    prepared V is stored transposed with its keys permuted to match that register layout, so
//    each A-operand fetch is one 16-byte LDS read.
//  * K and V tiles (64 keys) are double-buffered in LDS through registers with one barrier per
//    tile; 16-byte chunks are XOR-swizzled so ds_read_b128 phases are bank-conflict free.
//  * Workgroup ids are remapped so each XCD (own L2) works through whole heads; causal q-tiles
//    run longest first.  Fully masked key tiles (causal or mask classification) are skipped;
//    only diagonal, tail and mixed-mask tiles evaluate per-element predicates.
#include <limits.h>

#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kAttnThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;

template <int D, int PV>
struct TileGeom {
  static constexpr int K_BYTES = kBlockN * D;                   // K8 tile: 64 key rows x D bytes
  static constexpr int V_ROW = PV == 0 ? kBlockN * 2 : kBlockN;  // bytes per channel row of V tile
  static constexpr int V_BYTES = D * V_ROW;
  static constexpr int K_CHUNKS = K_BYTES / 16;
  static constexpr int V_CHUNKS = V_BYTES / 16;
  static constexpr int K_CPR = D / 16;
  static constexpr int V_CPR = V_ROW / 16;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int V_ESZ = PV == 0 ? 2 : 1;
};

// Cooperative global -> register -> LDS staging of one key tile by NT threads.
template <int D, int PV, int NT>
struct Stager {
  using G = TileGeom<D, PV>;
  static constexpr int KN = (G::K_CHUNKS + NT - 1) / NT;
  static constexpr int VN = (G::V_CHUNKS + NT - 1) / NT;
  v4i kreg[KN];
  v4i vreg[VN];

  __device__ __forceinline__ void load_k(const int8_t* k8h, int kt, int tid) {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      int c = tid + i * NT;
      if (c < G::K_CHUNKS) {
        int row = c / G::K_CPR, ch = c % G::K_CPR;
        kreg[i] = *reinterpret_cast<const v4i*>(k8h + ((int64_t)kt * kBlockN + row) * D + ch * 16);
      }
    }
  }
  __device__ __forceinline__ void store_k(char* sK, int tid) {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      int c = tid + i * NT;
      if (c < G::K_CHUNKS) {
        int row = c / G::K_CPR, ch = c % G::K_CPR;
        *reinterpret_cast<v4i*>(sK + lds_chunk_offset<D>(row, ch)) = kreg[i];
      }
    }
  }
  __device__ __forceinline__ void load_v(const uint8_t* vth, int64_t Nk_pad, int kt, int tid) {
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      int c = tid + i * NT;
      if (c < G::V_CHUNKS) {
        int row = c / G::V_CPR, ch = c % G::V_CPR;
        vreg[i] = *reinterpret_cast<const v4i*>(vth + ((int64_t)row * Nk_pad + (int64_t)kt * kBlockN) * G::V_ESZ +
                                                ch * 16);
      }
    }
  }
  __device__ __forceinline__ void store_v(char* sV, int tid) {
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      int c = tid + i * NT;
      if (c < G::V_CHUNKS) {
        int row = c / G::V_CPR, ch = c % G::V_CPR;
        *reinterpret_cast<v4i*>(sV + lds_chunk_offset<G::V_ROW>(row, ch)) = vreg[i];
      }
    }
  }
};

// B operand of S^T = K Q^T for one wave: lane (lr, g) holds bytes [32*cs + 16*g, +16) of its row.
template <int D>
__device__ __forceinline__ void load_q_frags(const int8_t* q8h, int64_t row, int64_t Nq_pad, int g,
                                             v4i (&qf)[D / 32]) {
#pragma unroll
  for (int cs = 0; cs < D / 32; ++cs) {
    if (row < Nq_pad)
      qf[cs] = *reinterpret_cast<const v4i*>(q8h + row * D + cs * 32 + g * 16);
    else
      qf[cs] = v4i{0, 0, 0, 0};
  }
}

// S^T for 64 keys x the wave's 32 queries.  acc[kb][r] = score of query lr and key
// kb*32 + (r/4)*8 + g*4 + r%4 of the tile.
template <int D>
__device__ __forceinline__ void qk_tile(const char* sK, const v4i (&qf)[D / 32], int lr, int g, v16i (&acc)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[kb][r] = 0;
#pragma unroll
  for (int cs = 0; cs < D / 32; ++cs) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      v4i a = *reinterpret_cast<const v4i*>(sK + lds_chunk_offset<D>(kb * 32 + lr, 2 * cs + g));
      acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[cs], acc[kb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ int key_of(int kb, int r, int g) { return kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3); }

template <int D, int PV>
__global__ __launch_bounds__(kAttnThreads) void k_attn_fwd(AttnArgs a) {
  using G = TileGeom<D, PV>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 31, g = lane >> 5;

  // workgroup -> (head, q-tile); consecutive logical ids land on the same XCD
  const int total = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, jx = bid >> 3, per = total >> 3, rem = total & 7;
  const int L = xcd < rem ? xcd * (per + 1) + jx : rem * (per + 1) + (xcd - rem) * per + jx;
  const int64_t bh = L / a.nQT;
  int qt = L % a.nQT;
  if (a.causal) qt = a.nQT - 1 - qt;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t q0 = (int64_t)qt * kBlockM;
  const int64_t r0w = q0 + (int64_t)w * kWaveRows;
  const int64_t row = r0w + lr;

  int kt_end = a.nKT;
  if (a.causal) {
    int64_t lim = (q0 + kBlockM + kBlockN - 1) / kBlockN;
    if (lim < kt_end) kt_end = (int)lim;
  }
  const uint8_t* mt = a.mtiles ? a.mtiles + ((b * a.Hm + (a.Hm == 1 ? 0 : h)) * a.nQT + qt) * a.nKT : nullptr;
  const uint8_t* mrow = nullptr;
  if (a.mask && row < a.Nq) mrow = a.mask + b * a.m_sb + (a.Hm == 1 ? 0 : h) * a.m_sh + row * a.m_sq;

  const int8_t* q8h = a.q8 + bh * a.Nq_pad * D;
  const int8_t* k8h = a.k8 + bh * a.Nk_pad * D;
  const uint8_t* vth = static_cast<const uint8_t*>(a.vt) + bh * D * a.Nk_pad * G::V_ESZ;
  v4i qf[D / 32];
  load_q_frags<D>(q8h, row, a.Nq_pad, g, qf);
  const int qblk = (int)(r0w / kQuantBlock);
  const float qsw = qblk < a.nbq ? a.qs[bh * a.nbq + qblk] : 0.f;
  const float* ksh = a.ks + bh * a.nbk;

  v16f o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_state = -INFINITY, l_lane = 0.f;

  Stager<D, PV, kAttnThreads> st;
  int kt = 0;
  while (kt < kt_end && mt && mt[kt] == 0) ++kt;
  if (kt < kt_end) {
    st.load_k(k8h, kt, tid);
    st.load_v(vth, a.Nk_pad, kt, tid);
    st.store_k(smem, tid);
    st.store_v(smem + G::K_BYTES, tid);
  }
  __syncthreads();
  int buf = 0;
  while (kt < kt_end) {
    int ktn = kt + 1;
    while (ktn < kt_end && mt && mt[ktn] == 0) ++ktn;
    if (ktn < kt_end) {
      st.load_k(k8h, ktn, tid);
      st.load_v(vth, a.Nk_pad, ktn, tid);
    }
    const char* sK = smem + buf * G::STAGE_BYTES;
    const char* sV = sK + G::K_BYTES;
    const int64_t j0 = (int64_t)kt * kBlockN;
    const bool wave_skip = a.causal && j0 > r0w + kWaveRows - 1;
    if (!wave_skip) {
      const bool mixed = mt && mt[kt] == 2;
      const bool partial = (j0 + kBlockN > a.Nk) || (a.causal && j0 + kBlockN - 1 > r0w) || mixed;
      v16i acc[2];
      qk_tile<D>(sK, qf, lr, g, acc);
      const float c = ((qsw * ksh[kt]) * a.sm_scale) * kLog2e;
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t j = j0 + key_of(kb, r, g);
            bool valid = j < a.Nk;
            if (a.causal) valid = valid && j <= row;
            if (mixed && mrow && valid) valid = mrow[j] != 0;
            if (!valid) acc[kb][r] = INT_MIN;
          }
      }
      int imax = INT_MIN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) imax = max(imax, acc[kb][r]);
      imax = max(imax, __shfl_xor(imax, 32));
      const float mt_ = imax == INT_MIN ? -INFINITY : (float)imax * c;
      const float m_new = fmaxf(m_state, mt_);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_state - m_use);
      const float pm = PV == 1 ? m_use - kLog2_448 : m_use;  // e4m3 path carries P as 448 * p
      float p[2][16];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)acc[kb][r], c, -pm));
          if (partial) e = acc[kb][r] == INT_MIN ? 0.f : e;
          p[kb][r] = e;
          psum += e;
        }
      l_lane = alpha * l_lane + psum;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      m_state = m_new;

      if constexpr (PV == 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kb = s >> 1, rb = (s & 1) * 8;
          v8h pf;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            v2f two = {p[kb][rb + 2 * jj], p[kb][rb + 2 * jj + 1]};
            v2h hh = __builtin_convertvector(two, v2h);  // round to nearest even
            pf[2 * jj] = hh[0];
            pf[2 * jj + 1] = hh[1];
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            v8h vf = *reinterpret_cast<const v8h*>(sV + lds_chunk_offset<128>(db * 32 + lr, 2 * s + g));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o[db], 0, 0, 0);
          }
        }
      } else {
        v8i pf;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int kb = q >> 2, r0 = (q & 3) * 4;
          int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r0], p[kb][r0 + 1], 0, false);
          pf[q] = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r0 + 2], p[kb][r0 + 3], lo, true);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          v4i v0 = *reinterpret_cast<const v4i*>(sV + lds_chunk_offset<64>(db * 32 + lr, 2 * g));
          v4i v1 = *reinterpret_cast<const v4i*>(sV + lds_chunk_offset<64>(db * 32 + lr, 2 * g + 1));
          v8i vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[db], 0, 0, 0, 127, 0, 127);
        }
      }
    }
    if (ktn < kt_end) {
      char* nK = smem + (buf ^ 1) * G::STAGE_BYTES;
      st.store_k(nK, tid);
      st.store_v(nK + G::K_BYTES, tid);
    }
    __syncthreads();
    buf ^= 1;
    kt = ktn;
  }

  // epilogue: normalize, store bf16 O and the LSE
  const float l_tot = l_lane + __shfl_xor(l_lane, 32);
  if (row < a.Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned short* orow = a.out + b * a.o_sb + h * a.o_sh + row * a.o_sn;
    const float* vsh = PV == 1 ? a.vscale + bh * D : nullptr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + rq * 8 + g * 4;
        unsigned short hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float f = o[db][rq * 4 + e] * inv;
          if constexpr (PV == 1) f = o[db][rq * 4 + e] * (vsh[d0 + e] * inv);
          hv[e] = f32_to_bf16(f);
        }
        uint2 pk = make_uint2((unsigned)hv[0] | ((unsigned)hv[1] << 16), (unsigned)hv[2] | ((unsigned)hv[3] << 16));
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
    if (g == 0 && a.lse) {
      float v = -INFINITY;
      if (l_tot > 0.f) {
        float m2 = PV == 1 ? m_state - kLog2_448 : m_state;
        v = (m2 + log2f(l_tot)) * kLn2 + a.sm_scale * a.corr[bh * a.Nq + row];
      }
      a.lse[bh * a.Nq + row] = v;
    }
  }
}

// Raw int32 scores of a window of one head, via the same staging and tile code as k_attn_fwd.
// grid = (32-row blocks, 64-key tiles) covering the window; block = one wave.
template <int D>
__global__ __launch_bounds__(64) void k_debug_qk(DebugQKArgs a, int64_t Nq_pad) {
  __shared__ __attribute__((aligned(16))) char sK[kBlockN * D];
  const int lane = threadIdx.x, lr = lane & 31, g = lane >> 5;
  const int64_t rb = a.row0 / kWaveRows + blockIdx.x;
  const int kt = (int)(a.col0 / kBlockN) + (int)blockIdx.y;
  Stager<D, 0, 64> st;
  st.load_k(a.k8h, kt, lane);
  st.store_k(sK, lane);
  __syncthreads();
  v4i qf[D / 32];
  const int64_t row = rb * kWaveRows + lr;
  load_q_frags<D>(a.q8h, row, Nq_pad, g, qf);
  v16i acc[2];
  qk_tile<D>(sK, qf, lr, g, acc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = (int64_t)kt * kBlockN + key_of(kb, r, g);
      if (row >= a.row0 && row < a.row0 + a.nrows && j >= a.col0 && j < a.col0 + a.ncols)
        a.out[(row - a.row0) * a.ncols + (j - a.col0)] = acc[kb][r];
    }
}

hipError_t launch_attn(const AttnArgs& a, int d, int pv_fp8, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nQT * a.B * a.H);
  if (d == 128) {
    if (pv_fp8)
      k_attn_fwd<128, 1><<<grid, kAttnThreads, 0, s>>>(a);
    else
      k_attn_fwd<128, 0><<<grid, kAttnThreads, 0, s>>>(a);
  } else {
    if (pv_fp8)
      k_attn_fwd<64, 1><<<grid, kAttnThreads, 0, s>>>(a);
    else
      k_attn_fwd<64, 0><<<grid, kAttnThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_debug_qk(const DebugQKArgs& a, int d, int64_t Nq_pad, hipStream_t s) {
  const int64_t rb0 = a.row0 / kWaveRows, rb1 = (a.row0 + a.nrows + kWaveRows - 1) / kWaveRows;
  const int64_t kt0 = a.col0 / kBlockN, kt1 = (a.col0 + a.ncols + kBlockN - 1) / kBlockN;
  dim3 grid((unsigned)(rb1 - rb0), (unsigned)(kt1 - kt0));
  if (d == 128)
    k_debug_qk<128><<<grid, 64, 0, s>>>(a, Nq_pad);
  else
    k_debug_qk<64><<<grid, 64, 0, s>>>(a, Nq_pad);
  return hipGetLastError();
}

}  // namespace sage
