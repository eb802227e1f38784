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
//  * One workgroup = 8 waves = 256 query rows of one (b,h), two waves per SIMD; each wave owns one
//    32-row MFMA block, and all eight read the K and V tiles the workgroup stages in LDS.  At
//    d = 128 (no float mask) each step is split into a softmax phase and an
//    MFMA phase, run in opposite orders by the two waves of a SIMD, so one wave's exponentials
//    overlap the other's MFMA stream.  The other launches software-pipeline the key loop inside
//    each wave instead (QK of the next tile, softmax of this tile and PV of the previous tile
//    interleaved).
//  * S^T = K8 . Q8^T on v_mfma_i32_32x32x32_i8: the K tile (A operand) comes from LDS, the
//    wave's Q8 rows (B operand) stay in registers for the whole key loop.  In the 32x32 output
//    layout each lane holds one query row and 16 of every 32 keys, so the row max and row sum are
//    in-lane except for one exchange with lane ^ 32.
//  * O^T += V^T . P^T on v_mfma_f32_32x32x16_f16 (or the 32x32x64 f8f6f4 MFMA with unit scales
//    for e4m3): P goes from the QK accumulator registers straight into the B operand.  The
//    prepared V is stored transposed with its keys permuted to match that register layout, so
//    each A-operand fetch is one 16-byte LDS read.
//  * K and V tiles (64 keys) stream into a four-stage LDS ring by direct buffer-to-LDS loads issued
//    two tiles ahead, one barrier per tile; 16-byte chunks are XOR-swizzled so ds_read_b128
//    phases are bank-conflict free.
//  * Workgroup ids are remapped so each XCD (own L2) works through whole heads; causal q-tiles
//    run longest first.  Fully masked key tiles (causal or mask classification) are skipped;
//    only diagonal, tail and mixed-mask tiles evaluate per-element predicates.
#include <limits.h>

#include <type_traits>

#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kWaves = kBlockM / 32;  // waves per attention workgroup, 32 query rows each
constexpr int kAttnThreads = kWaves * 64;
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
  static constexpr int K_SEGS_ALL = K_BYTES / 1024;
  static constexpr int V_SEGS_ALL = V_BYTES / 1024;
};

// Direct global -> LDS staging of key tiles with buffer loads (buffer_load_dwordx4 ... lds: lane l
// of a wave writes the 16 bytes at LDS base + 16*l).  Each wave fills whole 1 KiB segments of the
// tile buffer; a lane fetches the global chunk that belongs at its swizzled LDS position.  The
// per-head tensors are addressed through buffer resources (SGPRs).  The swizzle depends on the row
// modulo 16 only, so a lane's offset inside a segment depends on the segment's parity alone: one
// per-lane offset register serves every segment of a wave, and the segment and tile offsets are
// wave-uniform (SGPR soffset).

// Offset (relative to its segment's first row) of the global chunk that lane `lane` stores, for a
// segment of parity `par` of a buffer with ROW_BYTES-byte LDS rows and global row stride gstride.
template <int ROW_BYTES>
__device__ __forceinline__ int lds_lane_source(int par, int lane, int gstride) {
  constexpr int CPR = ROW_BYTES / 16, RPS = 1024 / ROW_BYTES;
  const int r = lane / CPR;                // row inside the segment
  const int row16 = (r + RPS * par) & 15;  // row of the buffer modulo 16
  const int lc = (lane % CPR) ^ (ROW_BYTES == 128 ? swz128(row16) : swz64(row16));
  return r * gstride + lc * 16;
}

template <int D, int PV, int NW>
struct Stager {
  using G = TileGeom<D, PV>;
  static constexpr int K_SEGS = G::K_BYTES / 1024;
  static constexpr int V_SEGS = G::V_BYTES / 1024;
  static constexpr int KN = (K_SEGS + NW - 1) / NW;
  static constexpr int VN = (V_SEGS + NW - 1) / NW;
  static constexpr int NP = NW % 2 == 0 ? 1 : 2;  // segment parities one wave sees
  __amdgpu_buffer_rsrc_t krs, vrs;
  int kx[NP], vx[NP];  // per-lane source offsets by segment parity
  int wu;              // wave index (SGPR)
  int vseg;            // global bytes between V segments (SGPR)

  // k8h: K8 rows of one head ([Nk_pad][D] bytes); vth: prepared V of one head ([D][Nk_pad])
  __device__ __forceinline__ void init(const int8_t* k8h, const uint8_t* vth, int64_t Nk_pad, int wave, int lane) {
    wu = __builtin_amdgcn_readfirstlane(wave);
    const int vrow = (int)Nk_pad * G::V_ESZ;
    vseg = (1024 / G::V_ROW) * vrow;
    krs = __builtin_amdgcn_make_buffer_rsrc((void*)k8h, (short)0, (int)(Nk_pad * D), kBufferWord3);
    vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vth, (short)0, vrow * D, kBufferWord3);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int par = NP == 1 ? (wu & 1) : p;
      kx[p] = lds_lane_source<D>(par, lane, D);
      vx[p] = lds_lane_source<G::V_ROW>(par, lane, vrow);
    }
  }
  __device__ __forceinline__ int px(const int (&x)[NP], int i) const { return NP == 1 ? x[0] : x[(i * NW) & 1]; }
  // K tile kt into the LDS buffer sK
  __device__ __forceinline__ void load_k(int kt, char* sK) const {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int seg = wu + i * NW;
      if (K_SEGS % NW == 0 || seg < K_SEGS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_t*)(sK + seg * 1024), 16, px(kx, i),
                                                 kt * kBlockN * D + seg * 1024, 0, 0);
    }
  }
  // V tile kt (columns [64kt, 64kt+64) of every channel row) into sV
  __device__ __forceinline__ void load_v(int kt, char* sV) const {
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      const int seg = wu + i * NW;
      if (V_SEGS % NW == 0 || seg < V_SEGS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_t*)(sV + seg * 1024), 16, px(vx, i),
                                                 kt * kBlockN * G::V_ESZ + seg * vseg, 0, 0);
    }
  }
};

// loads one wave issues for a tile buffer of SEGS 1 KiB segments shared by NW waves
template <int SEGS, int NW>
__device__ __forceinline__ int segs_of_wave(int w) {
  return SEGS / NW + (w < SEGS % NW ? 1 : 0);
}

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

__device__ __forceinline__ int key_of(int kb, int r, int g) { return kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3); }


// P^T fragments of one tile in the PV MFMA's B-operand layout (one 32-row block).
template <int PV>
struct PFrag;
template <>
struct PFrag<0> {  // fp16: 4 steps of 16 keys, 8 halves per lane each
  v8h s[4];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) s[i][j] = (_Float16)0.f;
  }
};
template <>
struct PFrag<1> {  // e4m3: 64 keys, 32 bytes per lane
  v8i b;
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = 0;
  }
};

// Per-lane LDS address bases.  The swizzles depend on the row modulo 16 only, so the fragment at
// row 32*k + lr of a tile lies at  (per-lane base for its chunk) + k * 32 * ROW_BYTES.  Lane
// (lr, g) reads chunks 2*c + g of 128-byte rows (K with d = 128, FP16 V), chunks 2*c + g of
// 64-byte rows (K with d = 64) and chunks 2*g + h of 64-byte rows (e4m3 V); every base is a
// register of its own, so no fragment address indexes an array by lane.
struct LaneBases {
  int b128[4];  // 128-byte rows, chunk 2*c + g
  int k64[2];   // 64-byte rows, chunk 2*c + g
  int v64[2];   // 64-byte rows, chunk 2*g + h
  __device__ __forceinline__ void init(int lr, int g) {
    const int x = g ^ swz128(lr);
#pragma unroll
    for (int c = 0; c < 4; ++c) b128[c] = lr * 128 + ((x ^ (2 * c)) << 4);
    const int y = swz64(lr);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      k64[c] = lr * 64 + (((2 * c + g) ^ y) << 4);
      v64[c] = lr * 64 + (((2 * g + c) ^ y) << 4);
    }
  }
};
// fragment at row 32*k + lr, chunk 2*c + g of a 128-byte-row tile starting at base
__device__ __forceinline__ v4i frag128(const char* base, const LaneBases& lb, int k, int c) {
  return *reinterpret_cast<const v4i*>(base + lb.b128[c] + 4096 * k);
}
// fragment at row 32*k + lr of a 64-byte-row tile: chunk 2*c + g (K) or 2*g + c (e4m3 V)
__device__ __forceinline__ v4i frag64k(const char* base, const LaneBases& lb, int k, int c) {
  return *reinterpret_cast<const v4i*>(base + lb.k64[c] + 2048 * k);
}
__device__ __forceinline__ v4i frag64v(const char* base, const LaneBases& lb, int k, int c) {
  return *reinterpret_cast<const v4i*>(base + lb.v64[c] + 2048 * k);
}

// A operand of QK MFMA q of a tile (key block q / (D/32), chunk step q % (D/32)): K rows
// 32*kb + lr, chunk 2*cs + g of the K tile at sK.  Every K tile of the attention kernel, and the
// debug scores, are read through this.
template <int D>
__device__ __forceinline__ v4i kfrag(const char* sK, const LaneBases& lb, int q) {
  constexpr int NB = D / 32;
  const int kb = q / NB, cs = q % NB;
  if constexpr (D == 128)
    return frag128(sK, lb, kb, cs);
  else
    return frag64k(sK, lb, kb, cs);
}

// QK MFMA q of S^T = K8 . Q8^T: starts key block q / (D/32)'s int32 accumulator at its first chunk
// step, accumulates the later ones.  acc[kb][r] = score of query lr and key kb*32 + (r/4)*8 + g*4 + r%4.
template <int D, bool MG = false>
__device__ __forceinline__ void qk_mfma(v4i kf, const v4i (&qf)[D / 32], int q, v16i (&acc)[2],
                                        const v16i& magic = v16i{}) {
  constexpr int NB = D / 32;
  const int kb = q / NB, cs = q % NB;
  if (cs == 0) {
    const v16i z = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[cs], MG ? magic : z, 0, 0, 0);
  } else {
    acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[cs], acc[kb], 0, 0, 0);
  }
}

// S^T for 64 keys x the wave's 32 queries, by the same operand reads and MFMA sequence as the
// QK half of every tile step.
template <int D, bool MG = false>
__device__ __forceinline__ void qk_tile(const char* sK, const v4i (&qf)[D / 32], const LaneBases& lb, v16i (&acc)[2],
                                        const v16i& magic = v16i{}) {
#pragma unroll
  for (int q = 0; q < 2 * (D / 32); ++q) qk_mfma<D, MG>(kfrag<D>(sK, lb, q), qf, q, acc, magic);
}

// Softmax state of a wave's rows.  Lane (lr, g) holds row lr; both halves of the wave carry the
// same reference maximum, and each holds the partial denominator of its half of the keys.
struct RowState {
  float m;      // reference maximum (log2 units) of the newest scored tile
  float pm;     // exponent offset of the tile being exponentiated (m, or m - log2(448) + tau for e4m3 P)
  float l;      // partial denominator
  float alpha;  // 2^(previous m - m) for the tile being exponentiated; O takes it after the
                // previous tile's PV
};

// Scores of a tile that fall outside the visible region become INT_MIN: key jr of the tile is
// visible iff jr <= lim and (mtile == nullptr or mtile[jr] != 0).
__device__ __forceinline__ void mask_scores(v16i (&acc)[2], int g, int lim, const uint8_t* mtile, bool mvec4) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int j4 = kb * 32 + rq * 8 + g * 4;
      unsigned mb = 0x01010101u;
      if (mtile) {
        if (mvec4 && j4 + 3 <= lim) {
          mb = *reinterpret_cast<const unsigned*>(mtile + j4);
        } else {
          mb = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j4 + e <= lim) mb |= (unsigned)mtile[j4 + e] << (8 * e);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = (j4 + e <= lim) && ((mb >> (8 * e)) & 0xffu) != 0;
        if (!valid) acc[kb][rq * 4 + e] = INT_MIN;
      }
    }
}

// Float-mask form: every score of a tile becomes the fp32 bit pattern of its log2-unit value
// acc * c + log2(e) * M[j] (M = 0 where mtile is null), and -inf outside the visible keys
// (j > lim) or where M is -inf.  mtile is the row's mask at the tile's first key, read only if
// has_m (the same for the whole wave); full4: the tile's 64 keys all exist and the row is 16-byte
// aligned, so it is read 16 bytes at a time; otherwise one element at a time at indices clamped
// to the visible range (j <= max(lim, 0) < Nk - j0: always inside the row).  No per-lane branches.
// GUARD (a NaN or infinite scale c, where acc * c - inf is NaN): entries whose M is -inf are set
// to -inf explicitly, so a masked key stays out of the row even then.
template <bool GUARD>
__device__ __forceinline__ void mask_scores_f32(v16i (&acc)[2], int g, int lim, const float* mtile, bool has_m,
                                                bool full4, float c) {
  const int jmax = lim > 0 ? lim : 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int j4 = kb * 32 + rq * 8 + g * 4;
      float mv[4] = {0.f, 0.f, 0.f, 0.f};
      if (has_m) {
        if (full4) {
          const float4 m4 = *reinterpret_cast<const float4*>(mtile + j4);
          mv[0] = m4.x;
          mv[1] = m4.y;
          mv[2] = m4.z;
          mv[3] = m4.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[e] = mtile[j4 + e < jmax ? j4 + e : jmax];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = __builtin_fmaf((float)acc[kb][rq * 4 + e], c, mv[e] * kLog2e);
        const bool vis = j4 + e <= lim && (!GUARD || mv[e] != -INFINITY);
        acc[kb][rq * 4 + e] = __float_as_int(vis ? t : -INFINITY);
      }
    }
}

// Row maximum of a tile's scores in four independent chains of eight: piece p (0..7) advances
// chain p/2 by two max3/max steps.  The scores are int32 (MF = false) or fp32 bit patterns (MF).
template <bool MF>
__device__ __forceinline__ int smax(int x, int y) {
  if constexpr (MF)
    return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y)));
  else
    return max(x, y);
}
__device__ __forceinline__ int score_at(const v16i (&acc)[2], int i) { return acc[i >> 4][i & 15]; }
template <bool MF = false>
__device__ __forceinline__ void max_piece(const v16i (&acc)[2], int (&ch)[4], int p) {
  const int c = p >> 1, e = 8 * c;
  if ((p & 1) == 0) {
    ch[c] = smax<MF>(smax<MF>(score_at(acc, e), score_at(acc, e + 1)), score_at(acc, e + 2));
    ch[c] = smax<MF>(smax<MF>(ch[c], score_at(acc, e + 3)), score_at(acc, e + 4));
  } else {
    ch[c] = smax<MF>(smax<MF>(ch[c], score_at(acc, e + 5)), score_at(acc, e + 6));
    ch[c] = smax<MF>(ch[c], score_at(acc, e + 7));
  }
}
// Combines the chains across the wave's halves and moves the reference maximum (lazy by
// kSoftmaxTau[PV] log2 units).  Returns 2^(m_old - m_new); the new exponent offset goes to pm_new.
template <int PV, bool MASKED, bool MF = false, bool BM = false, bool MG = false>
__device__ __forceinline__ float finish_max(const int (&ch)[4], float c, RowState& rs, float& pm_new, float cb = 0.f) {
  constexpr float kTau = kSoftmaxTau[PV];
  int im = smax<MF>(smax<MF>(ch[0], ch[1]), smax<MF>(ch[2], ch[3]));
  const auto sw = __builtin_amdgcn_permlane32_swap(im, im, false, false);  // lanes l and l ^ 32
  im = smax<MF>((int)sw[0], (int)sw[1]);
  if constexpr (MG) im = (MASKED && im == INT_MIN) ? INT_MIN : im - kMagicBits;  // the biased accumulator
  float mt;
  if constexpr (MF)
    mt = __int_as_float(im);  // already log2-unit fp32, -inf if nothing is visible
  else if constexpr (BM && MASKED)  // with the row's per-block score term cb (per_block_mean)
    mt = im == INT_MIN ? -INFINITY : __builtin_fmaf((float)im, c, cb);
  else if constexpr (BM)
    mt = __builtin_fmaf((float)im, c, cb);
  else if constexpr (MASKED)
    mt = im == INT_MIN ? -INFINITY : (float)im * c;
  else
    mt = (float)im * c;
  const float m_new = (mt > rs.m + kTau) ? mt : rs.m;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(rs.m - m_use);
  rs.m = m_new;
  pm_new = PV == 1 ? m_use - (kLog2_448 - kTau) : m_use;  // the e4m3 path carries P as 448 * 2^-tau * p
  return alpha;
}

// MFMA operand geometry of one tile step.
template <int D, int PV>
struct StepGeom {
  static constexpr int NB = D / 32;                   // 32-wide blocks of the head dimension
  static constexpr int NQ = 2 * NB;                   // QK MFMAs: key block q / NB, chunk step q % NB
  static constexpr int NPV = PV == 0 ? 4 * NB : NB;  // PV MFMAs
  static constexpr int NM = NPV + NQ;                 // MFMA k < NPV is PV MFMA k, else QK MFMA k - NPV
  static constexpr int LA = PV == 0 ? 3 : 1;          // operands read from LDS ahead of the MFMA stream
  using VFrag = typename std::conditional<PV == 0, v4i, v8i>::type;
};

// A operand of PV MFMA j from the V tile at sV: fp16 -- channels 32*(j % NB) + lr, keys of step
// j / NB; e4m3 -- channel block j, the lane's 32 keys (two 16-byte chunks)
template <int D, int PV>
__device__ __forceinline__ typename StepGeom<D, PV>::VFrag vfrag(const char* sV, const LaneBases& lb, int g, int j) {
  constexpr int NB = D / 32;
  if constexpr (PV == 0) {
    return frag128(sV, lb, j % NB, j / NB);
  } else {
    const v4i v0 = frag64v(sV, lb, j, 0), v1 = frag64v(sV, lb, j, 1);
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// One software-pipelined tile step of a wave.  At step n the tile T[n] has been scored (acc) and
// the row maxima of its first key block are in ch[0..1]; T[n-1]'s probabilities are in P; T[n+1]
// is to be scored.  The step interleaves three independent streams:
//   MFMA: PV of T[n-1] (P, V from sVp; its first LA operands arrive in vpre) into O first, then QK
//         of T[n+1] (K from sKn) into acc;
//   VALU: the rest of T[n]'s row maxima and its reference maximum (first slots), the
//         exponentials of T[n] into P -- each group once the MFMAs reading its registers have been
//         issued -- with the row sums, and the row maxima of T[n+1]'s first key block.
// Ordered this way, P and the scores are overwritten in place and no VALU work waits for a
// just-issued MFMA.  Every MFMA is issued with a slice of VALU work and the LDS reads LA operands
// ahead; sched_barrier fences keep that order.  At the end vpre receives the first operands of the
// next step's PV (V tile sVn).  With SLOW, T[n]'s scores may be masked (INT_MIN) and T[n+1] is
// masked by lim / mtile (mask_scores).  With MF (float mask; implies SLOW) T[n]'s raw scores are
// converted at the start of the step to log2-unit fp32 with the mask added (mask_scores_f32, with
// lim / mtile / has_m / mvec4 describing T[n] and scale c_cur), all its row maxima follow, and the
// exponentials take the converted scores as they are.  Returns 2^(m_{n-1} - m_n), the factor O
// takes after the PV of T[n-1].
template <int D, int PV, bool SLOW, bool MF = false, bool BM = false>
__device__ __forceinline__ float tile_step(v16i (&acc)[2], int (&ch)[4], PFrag<PV>& P,
                                           typename StepGeom<D, PV>::VFrag (&vpre)[StepGeom<D, PV>::LA],
                                           const char* sKn, const char* sVp, const char* sVn, const v4i (&qf)[D / 32],
                                           v16f (&o)[D / 32], float c_cur, RowState& rs, const LaneBases& lb, int g,
                                           int lim, const void* mtile, bool mvec4, bool has_m = false,
                                           float cb_cur = 0.f, const v16i& magic = v16i{}) {
  static_assert(SLOW || !MF, "the float-mask step is a masked step");
  static_assert(!(MF && BM), "per_block_mean is not combined with a float mask");
  using SG = StepGeom<D, PV>;
  constexpr int NB = SG::NB, NQ = SG::NQ, NPV = SG::NPV, NM = SG::NM, LA = SG::LA;
  // FP16 P without a float mask: the QK accumulators start at the bit pattern of 1.5 * 2^23, so each
  // score arrives as the float 1.5 * 2^23 + s and enters the exponent with one FMA
  constexpr bool MG = PV == 0 && !MF;
  constexpr int NG = 8;                 // exponential groups of 4 scores
  constexpr int FIN = 1;                // slot of the reference-maximum update (pieces 4-7 in slot 0)
  using VFrag = typename SG::VFrag;

  // Slot of exponential group gi, after the reference maximum.  FP16: after the PV MFMAs that
  // read the P registers it overwrites, spread so that each key block's scores are consumed
  // before the QK of T[n+1] overwrites them.  e4m3: every PV MFMA reads all of P, so P is written
  // into fresh registers, spread over the slots before the second key block's QK.
  auto exp_slot = [](int gi) {
    if (PV == 1) return FIN + 1 + gi * (NPV + NB - FIN - 1) / NG;
    // group gi writes P fragment gi / 2, which PV MFMAs (gi / 2) * NB .. (gi / 2) * NB + NB - 1 read
    const int first = ((gi >> 1) + 1) * NB > FIN + 1 ? ((gi >> 1) + 1) * NB : FIN + 1;
    const int s = NB + gi * NPV / NG;
    return s > first ? s : first;
  };
  // slot of row-max piece p < 4 of T[n+1] (key block 0): two MFMAs after that block's last QK
  auto max_slot = [](int p) { return NPV + NB + 1 + p / 2 < NM - 1 ? NPV + NB + 1 + p / 2 : NM - 1; };

  v16i sc[2] = {acc[0], acc[1]};  // scores of T[n]
  if constexpr (MF) {
    // T[n]'s scores to log2-unit fp32 with its mask (lim / mtile / has_m / mvec4 describe T[n]),
    // and all eight row-maximum pieces, before the MFMA stream
    const float* mt4 = static_cast<const float*>(mtile);
    const int cbits = __builtin_amdgcn_readfirstlane(__float_as_int(c_cur));  // the same in every lane
    if ((cbits & 0x7f800000) != 0x7f800000)
      mask_scores_f32<false>(sc, g, lim, mt4, has_m, mvec4, c_cur);
    else
      mask_scores_f32<true>(sc, g, lim, mt4, has_m, mvec4, c_cur);
#pragma unroll
    for (int p = 0; p < 8; ++p) max_piece<true>(sc, ch, p);
  }
  const PFrag<PV> pin = P;              // probabilities of T[n-1]
  VFrag vf[NPV];
  v4i kf[NQ];
#pragma unroll
  for (int r = 0; r < LA; ++r) vf[r] = vpre[r];
  auto read = [&](int r) {  // operand r of the MFMA stream
    if (r < NPV)
      vf[r] = vfrag<D, PV>(sVp, lb, g, r);
    else
      kf[r - NPV] = kfrag<D>(sKn, lb, r - NPV);
  };
  float psum = 0.f, alpha = 1.f;
  float nb = 0.f;  // per_block_mean: T[n]'s row term minus the exponent offset
  float kk = 0.f;  // MG: the exponent's constant term, -(1.5 * 2^23) * c - pm (+ the row term)

#pragma unroll
  for (int k = 0; k < NM; ++k) {
    if (k + LA < NM) read(k + LA);  // LDS reads for a later MFMA
    if (k < NPV) {
      if constexpr (PV == 0)
        o[k % NB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, vf[k]), pin.s[k / NB], o[k % NB], 0,
                                                          0, 0);
      else
        o[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[k], pin.b, o[k], 0, 0, 0, 127, 0, 127);
    } else {
      qk_mfma<D, MG>(kf[k - NPV], qf, k - NPV, acc, magic);
    }
    // T[n]'s row maxima over its second key block, then its reference maximum
    if (!MF && k == 0) {
#pragma unroll
      for (int p = 4; p < 8; ++p) max_piece(sc, ch, p);
    }
    if (k == FIN) {
      float pm_new;
      alpha = finish_max<PV, SLOW, MF, BM, MG>(ch, c_cur, rs, pm_new, cb_cur);
      rs.pm = pm_new;
      if constexpr (BM) nb = cb_cur - pm_new;
      if constexpr (MG) kk = __builtin_fmaf(-kMagic, c_cur, BM ? nb : -pm_new);
    }
    // exponentials of T[n] assigned to slot k
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (exp_slot(gi) != k) continue;
      constexpr int GS = 32 / NG;
      float x[GS];
#pragma unroll
      for (int e = 0; e < GS; ++e) {
        const int idx = gi * GS + e, kb = idx >> 4, r = idx & 15;
        // The empty asm pins the score to this slot: without it the compiler converts all 32 scores
        // at the top of the step, where no MFMA overlaps them.
        int si = sc[kb][r];
        asm volatile("" : "+v"(si));
        float t;
        if constexpr (MF) {
          t = __builtin_amdgcn_exp2f(__int_as_float(si) - rs.pm);  // -inf gives 0
        } else if constexpr (MG) {
          t = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(si), c_cur, kk));
          if constexpr (SLOW) t = si == INT_MIN ? 0.f : t;
        } else {
          t = __builtin_amdgcn_exp2f(__builtin_fmaf((float)si, c_cur, BM ? nb : -rs.pm));
          if constexpr (SLOW) t = si == INT_MIN ? 0.f : t;
        }
        x[e] = t;
      }
      // the row sum takes the fp32 probabilities (before P's rounding)
      psum += (x[0] + x[1]) + (x[2] + x[3]);
      if constexpr (PV == 0) {
        const int idx = gi * 4, kb = idx >> 4, r = idx & 15;
        const int s2 = kb * 2 + (r >> 3), jj = (r & 7) >> 1;  // jj = 0 or 2
        const v2h h0 = __builtin_convertvector((v2f{x[0], x[1]}), v2h);  // round to nearest even
        const v2h h1 = __builtin_convertvector((v2f{x[2], x[3]}), v2h);
        P.s[s2][2 * jj] = h0[0];
        P.s[s2][2 * jj + 1] = h0[1];
        P.s[s2][2 * jj + 2] = h1[0];
        P.s[s2][2 * jj + 3] = h1[1];
      } else {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        P.b[gi] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
      }
    }
    // row maxima of T[n+1]'s first key block (a tile that needs masking takes them after the slots)
    if constexpr (!SLOW) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (max_slot(p) == k) max_piece(acc, ch, p);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!MF && SLOW) {
    mask_scores(acc, g, lim, static_cast<const uint8_t*>(mtile), mvec4);
#pragma unroll
    for (int p = 0; p < 4; ++p) max_piece(acc, ch, p);
  }
  rs.l = alpha * rs.l + psum;
#pragma unroll
  for (int r = 0; r < LA; ++r) vpre[r] = vfrag<D, PV>(sVn, lb, g, r);
  return alpha;
}

// O^T += V^T P^T for one tile (V tile from LDS); used for the last tile after the loop.
template <int D, int PV>
__device__ __forceinline__ void pv_tile(const char* sV, const PFrag<PV>& pf, const LaneBases& lb, int g,
                                        v16f (&o)[D / 32]) {
  if constexpr (PV == 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, frag128(sV, lb, db, s)), pf.s[s], o[db],
                                                      0, 0, 0);
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const v4i v0 = frag64v(sV, lb, db, 0), v1 = frag64v(sV, lb, db, 1);
      const v8i vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf.b, o[db], 0, 0, 0, 127, 0, 127);
    }
  }
}

template <int D>
__device__ __forceinline__ void scale_acc(v16f (&o)[D / 32], float alpha) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
}

// Phase-split schedule (PP) for launches without a mask table, float mask or per-block means.
// The waves of a workgroup form two groups, one wave of each on every SIMD (waves 0-3 and 4-7).
// Every step holds one softmax phase (VALU: a tile's row maxima, exponentials, row sums and
// P) and one MFMA phase (QK of the next tile into the score registers, PV of the current tile
// from P), in opposite orders in the two groups: group 0 runs softmax then MFMA, group 1 runs
// MFMA then the softmax of the next tile.  So while one wave of a SIMD streams its MFMAs, the
// other runs its softmax on the vector unit, and a wave holds one set of score registers, not two.

// Softmax of one tile whose scores are in acc (BM: plus the row's per_block_mean term cb, log2
// units): masks them (SLOW; lim and the boolean mask row mtile as in mask_scores), takes the row maxima, moves the
// reference maximum, and writes P = exp2(s*c - pm) (fp16, or e4m3 of 448*2^-tau*p) with the row
// sums.  Returns 2^(m_old - m_new), the factor O takes before this tile's PV.
template <int D, int PV, bool SLOW, bool BM = false>
__device__ __forceinline__ float softmax_phase(v16i (&acc)[2], PFrag<PV>& P, float c, RowState& rs, int g, int lim,
                                               const uint8_t* mtile, bool mvec4, float cb = 0.f) {
  constexpr bool MG = PV == 0;  // FP16 P: the QK accumulators start at the biased value (see tile_step)
  c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)));  // the same in every lane: an SGPR operand
  if constexpr (SLOW) mask_scores(acc, g, lim, mtile, mvec4);
  int ch[4];
#pragma unroll
  for (int p = 0; p < 8; ++p) max_piece(acc, ch, p);
  float pm_new;
  const float alpha = finish_max<PV, SLOW, false, BM, MG>(ch, c, rs, pm_new, cb);
  rs.pm = pm_new;
  const float nb = BM ? cb - pm_new : -pm_new;  // per_block_mean: the row's term of this key block
  const float kk = MG ? __builtin_fmaf(-kMagic, c, nb) : nb;
  float psum = 0.f;
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = gi * 4 + e;
      const int si = acc[idx >> 4][idx & 15];
      float t;
      if constexpr (MG)
        t = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(si), c, kk));
      else
        t = __builtin_amdgcn_exp2f(__builtin_fmaf((float)si, c, kk));
      if constexpr (SLOW) t = si == INT_MIN ? 0.f : t;
      x[e] = t;
    }
    psum += (x[0] + x[1]) + (x[2] + x[3]);  // the fp32 probabilities, before P's rounding
    if constexpr (PV == 0) {
      const int idx = gi * 4, kb = idx >> 4, r = idx & 15;
      const int s2 = kb * 2 + (r >> 3), jj = (r & 7) >> 1;
      const v2h h0 = __builtin_convertvector((v2f{x[0], x[1]}), v2h);  // round to nearest even
      const v2h h1 = __builtin_convertvector((v2f{x[2], x[3]}), v2h);
      P.s[s2][2 * jj] = h0[0];
      P.s[s2][2 * jj + 1] = h0[1];
      P.s[s2][2 * jj + 2] = h1[0];
      P.s[s2][2 * jj + 3] = h1[1];
    } else {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      P.b[gi] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    }
  }
  rs.l = alpha * rs.l + psum;
  return alpha;
}

// Operands of the MFMA phase read from LDS ahead of its MFMA stream.
constexpr int kPhaseLA = 3;

// MFMA phase: the QK MFMAs of the next tile (K from sK) into acc, then the PV MFMAs of the
// current tile (V from sV, P) into O.  Operand r < NQ is K fragment r, else V fragment r - NQ;
// the first kPhaseLA K fragments arrive in pre, the rest are read kPhaseLA MFMAs ahead.
template <int D, int PV>
__device__ __forceinline__ void mfma_phase(const v4i (&pre)[kPhaseLA], const char* sK, const char* sV,
                                           const PFrag<PV>& P, const v4i (&qf)[D / 32], v16f (&o)[D / 32],
                                           v16i (&acc)[2], const LaneBases& lb, int g, const v16i& magic) {
  using SG = StepGeom<D, PV>;
  constexpr int NB = SG::NB, NQ = SG::NQ, NPV = SG::NPV, NM = NQ + NPV;
  static_assert(NQ > kPhaseLA, "the preloaded operands are K fragments");
  v4i kf[NQ];
  typename SG::VFrag vf[NPV];
#pragma unroll
  for (int r = 0; r < kPhaseLA; ++r) kf[r] = pre[r];
  auto read = [&](int r) {
    if (r < NQ)
      kf[r] = kfrag<D>(sK, lb, r);
    else
      vf[r - NQ] = vfrag<D, PV>(sV, lb, g, r - NQ);
  };
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    if (k + kPhaseLA < NM) read(k + kPhaseLA);
    if (k < NQ) {
      qk_mfma<D, PV == 0>(kf[k], qf, k, acc, magic);
    } else {
      const int j = k - NQ;
      if constexpr (PV == 0)
        o[j % NB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, vf[j]), P.s[j / NB], o[j % NB], 0,
                                                          0, 0);
      else
        o[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[j], P.b, o[j], 0, 0, 0, 127, 0, 127);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Main loop, software-pipelined inside each wave (see tile_step).  One workgroup = 8 waves = 256
// query rows; wave w owns rows 32w..32w+31.  LDS holds a four-stage ring of K tiles and one of V
// tiles; processed tiles are numbered T[0], T[1], ...: K of T[i] lives in kslot i%4, V of T[i] in
// vslot i%4.  Step n consumes K of T[n+1] and V of T[n-1], issues the loads of V of T[n+2] and K
// of T[n+3] into slots freed two steps earlier, and waits at its end only for the loads of the
// previous step.  The loop is unrolled four times so every slot is a compile-time offset.  One
// barrier per tile.  MF: the mask is fp32 and additive, and every tile takes the masked step.
// BM: per_block_mean -- every score of key tile t gets the row's term blk_corr[t][row] (loaded a
// step ahead, before the step's staging loads, so the vmcnt waits below cover it).
// The kernel's argument block, read through an opaque copy of its address: loads through it are
// issued where they appear instead of being hoisted into SGPRs held across the loop.
template <typename T>
__device__ __forceinline__ const T* kernarg_reload() {
  const T* p = (const T*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// TT: the launch has a mask-tile table (a boolean or float mask; MF implies TT).  Without one the
// tile walk is plain arithmetic: no tile is dropped and only the causal diagonal and ragged tail
// take the per-element step.
// PP: the phase-split schedule (softmax_phase / mfma_phase) instead of tile_step; not with a float
// mask.
template <int D, int PV, int MF, int BM, int TT, int PP = 0>
__global__ __launch_bounds__(kAttnThreads) void k_attn_fwd(AttnArgs a) {
  static_assert(TT || !MF, "a float mask comes with its tile table");
  static_assert(!PP || !MF, "the phase-split schedule takes no float mask");
  using G = TileGeom<D, PV>;
  constexpr int kNS = 4;
  // PP with per_block_mean: a third ring holds each key tile's per-row score terms (4 B x 256 rows)
  constexpr int kCB = PP && BM ? kBlockM * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem[kNS * G::K_BYTES + kNS * G::V_BYTES + kNS * kCB];
  // V ring first: with at most 64 KiB of V slots every V fragment read is a lane base plus an
  // immediate ds_read offset
  char* const vring = smem;
  char* const kring = smem + kNS * G::V_BYTES;
  char* const cbring = kring + kNS * G::K_BYTES;  // PP && BM only
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int w = tid >> 6;
  // PP: waves 4-7 run their MFMA phase first.  Waves w and w + 4 share a SIMD (waves go round-robin
  // over the four SIMDs), so every SIMD holds one wave of each group.
  const int grp1 = __builtin_amdgcn_readfirstlane(w >= kWaves / 2 ? 1 : 0);

  int64_t bh;
  int qt;
  map_workgroup(a.B, a.H, a.Hkv, a.nQT, a.causal, bh, qt);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int q0 = qt * kBlockM;
  const int r0w = q0 + w * 32;  // first row of this wave (token counts are < 2^30)
  const int row = r0w + lr;
  // this batch entry's query and key counts (a packed variable-length batch: its sequence's)
  const SeqSpan sq = seq_span(a.cu_q, b, a.Nq, a.total_q), sk = seq_span(a.cu_k, b, a.Nk, a.total_k);
  const int nk = (int)sk.len, nq = (int)sq.len;
  if (q0 >= nq) return;  // a query tile past the end of a shorter sequence: the whole workgroup leaves

  int kt_end = (nk + kBlockN - 1) / kBlockN;
  if (a.causal) {
    const int lim = (q0 + kBlockM + kBlockN - 1) / kBlockN;
    if (lim < kt_end) kt_end = lim;
  }
  const int* mt = TT ? a.mtiles + ((b * a.Hm + (a.Hm == 1 ? 0 : h)) * a.nQT + qt) * a.nKT : nullptr;
  constexpr int kMaskBytes = MF ? 4 : 1;  // bytes per mask element
  // the float-mask step reads rows past Nq at row Nq - 1 (never stored), so a tile's mask pointer
  // is null or not for the whole wave
  const int mrow_i = MF && row >= nq ? nq - 1 : row;
  const char* mrow = (a.mask && mrow_i < nq) ? static_cast<const char*>(a.mask) +
                                                   (b * a.m_sb + (a.Hm == 1 ? 0 : h) * a.m_sh +
                                                    (int64_t)mrow_i * a.m_sq) * kMaskBytes
                                             : nullptr;

  const int64_t bhk = b * a.Hkv + h / (a.H / a.Hkv);  // key/value head (group-query attention)
  const int8_t* q8h = a.q8 + bh * a.Nq_pad * D;
  const int8_t* k8h = a.k8 + bhk * a.Nk_pad * D;
  const uint8_t* vth = static_cast<const uint8_t*>(a.vt) + bhk * D * a.Nk_pad * G::V_ESZ;
  const int r0u = __builtin_amdgcn_readfirstlane(r0w);  // the same value, held in an SGPR
  const int qblk = r0u / kQuantBlock;                   // a wave's rows lie in one quantization block
  const float cq = qblk < a.nbq ? scalar_ld(a.qs + bh * a.nbq, qblk) : 0.f;
  const float* ksh = a.ks + bhk * a.nbk;

  v16f o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // The first step multiplies a zero P by the V slot of "T[-1]": clear it so uninitialized LDS
  // (possibly NaN patterns) cannot leak in through 0 * NaN.
  for (int i = tid; i < G::V_BYTES / 16; i += kAttnThreads)
    *reinterpret_cast<v4i*>(vring + (kNS - 1) * G::V_BYTES + i * 16) = v4i{0, 0, 0, 0};

  Stager<D, PV, kWaves> st;
  st.init(k8h, vth, a.Nk_pad, w, lane);
  // mask-tile table entry: state in bits 0-1 (0 all masked, 1 all visible, 2 mixed), above them the
  // next tile of this row block that is not all masked
  auto tstate = [&](int t) { return TT ? scalar_ld(mt, t) & 3 : 1; };
  auto dropped = [&](int t) { return tstate(t) == 0; };
  auto next_tile = [&](int t) {
    if constexpr (!TT) return t + 1 < kt_end ? t + 1 : kt_end;
    if (t >= kt_end) return kt_end;
    const int nx = scalar_ld(mt, t) >> 2;
    return nx < kt_end ? nx : kt_end;
  };
  int t0 = 0;
  if (TT && kt_end > 0 && dropped(0)) t0 = next_tile(0);
  const int t1 = next_tile(t0), t2 = next_tile(t1), t3 = next_tile(t2);
  const int tstand = t0 < kt_end ? t0 : 0;  // a valid tile to stand in for loads past the end
  auto clampt = [&](int t) { return t < kt_end ? t : tstand; };
  // PP with per_block_mean: key tile t's terms of the workgroup's 256 rows (blk_corr[t][q0 ..], 4 B
  // each) travel through their own ring slot beside its K tile.  Wave w loads the 64 rows of
  // quarter w % 4, one dword a lane (the rows start at any 4-byte boundary): waves w and w + 4 write
  // the same values to the same bytes, so every wave issues the same loads per step and the step's
  // wait stays one compile-time count (a wave-dependent wait made the compiler spill).  Rows past
  // the head's terms read 0.
  const __amdgpu_buffer_rsrc_t cbrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(PP && BM ? a.blk_corr + bh * a.nbk * a.Nq : nullptr), (short)0, PP && BM ? (int)(a.nbk * a.Nq * 4) : 0,
      kBufferWord3);
  const int wq = __builtin_amdgcn_readfirstlane(w % (kWaves / 2));  // quarter of the rows
  auto load_cb = [&](int t, int slot) {
    if constexpr (PP && BM)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cbrs, (lds_void_t*)(cbring + slot * kCB + wq * 256), 4, (int)(lane * 4),
                                               (int)(((int64_t)t * a.Nq + q0) * 4) + wq * 256, 0, 0);
  };
  if (t0 < kt_end) {
    st.load_k(t0, kring);
    st.load_k(clampt(t1), kring + G::K_BYTES);
    st.load_k(clampt(t2), kring + 2 * G::K_BYTES);
    load_cb(t0, 0);
    load_cb(clampt(t1), 1);
    load_cb(clampt(t2), 2);
    st.load_v(t0, vring);
    st.load_v(clampt(t1), vring + G::V_BYTES);
  }
  v4i qf[D / 32];
  load_q_frags<D>(q8h, row, a.Nq_pad, g, qf);
  LaneBases lb;
  lb.init(lr, g);
  __builtin_amdgcn_s_waitcnt(0);  // Q fragments and the prologue tiles resident
  __syncthreads();

  // per-tile scale, and whether a tile needs per-element visibility (past the end, ragged tail,
  // causal diagonal, mixed mask tile); lim / mtile describe the visible keys of such a tile
  auto scale_of = [&](int t) { return t < kt_end ? ((cq * scalar_ld(ksh, t)) * a.sm_scale) * kLog2e : 0.f; };
  // In the loop the k-scales arrive by vector loads a step ahead, counted by vmcnt with the staging
  // loads: a scalar load there would need lgkmcnt(0), which also drains the in-flight LDS reads.
  const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)ksh, (short)0, a.nbk * 4, kBufferWord3);
  const int vzero = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);  // 0 in a vector register: a vector load
  auto ks_load = [&](int t) {
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksrs, vzero, (t < kt_end ? t : 0) * 4, 0));
  };
  auto scale_from = [&](int t, float ks) { return t < kt_end ? ((cq * ks) * a.sm_scale) * kLog2e : 0.f; };
  // Tiles [0, first_part) are whole for every row of this wave: no ragged tail, and (causal) every
  // key at or before the wave's first row.  Tiles at or past it, and past kt_end, take the
  // per-element step.
  const int first_part = a.causal && (r0u + 1) / kBlockN < nk / kBlockN ? (r0u + 1) / kBlockN : nk / kBlockN;
  auto partial = [&](int t) {
    // The test runs on a vector-register copy of the tile index (v_mbcnt_lo with an empty mask
    // adds 0): the compiler then keeps the masked/unmasked step choice as a per-lane branch, which
    // it compiles without spills, and holds no row index in a vector register across the loop.
    return (int)__builtin_amdgcn_mbcnt_lo(0u, t) >= first_part || (TT && tstate(t) == 2);
  };
  auto visible = [&](int t, int& lim, const void*& mtile) {
    if (t >= kt_end) {
      lim = -1;
      mtile = nullptr;
      return;
    }
    const int j0 = t * kBlockN;
    lim = j0 + kBlockN > nk ? nk - j0 - 1 : kBlockN - 1;
    if (a.causal) {
      const int dr = row - j0;
      lim = dr < lim ? (dr < -1 ? -1 : dr) : lim;
    }
    mtile = (TT && tstate(t) == 2 && mrow) ? mrow + (int64_t)j0 * kMaskBytes : nullptr;
  };
  // float-mask step: whether tile t reads its mask (uniform), and whether it may read it 16 bytes
  // at a time; the mask pointer is then formed for every lane
  auto fmask_of = [&](int t, bool& has_m, bool& full4) -> const void* {
    has_m = t < kt_end && TT && tstate(t) == 2;
    full4 = a.mask_vec4 && (t + 1) * kBlockN <= nk;
    return mrow ? mrow + (int64_t)(t < kt_end ? t : 0) * kBlockN * kMaskBytes : nullptr;
  };

  // FP16 P: the QK accumulators' starting value (see tile_step), held in registers for the whole
  // loop -- the empty asm keeps the compiler from rebuilding the constant in every step
  v16i magic;
  if constexpr (PV == 0 && !MF) {
    int mb = kMagicBits;
    asm volatile("" : "+v"(mb));
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = mb;
  }
  RowState rs;
  rs.m = -INFINITY;
  rs.pm = 0.f;
  rs.l = 0.f;
  v16i acc[2];
  int ch[4];
  PFrag<PV> P;
  P.zero();
  typename StepGeom<D, PV>::VFrag vpre[StepGeom<D, PV>::LA];
  float c_cur = scale_of(t0);
  bool part_cur = partial(t0);
  // per_block_mean: the row's score term of a key tile, in log2 units (rows past Nq read row Nq-1)
  const float* cbh = BM ? a.blk_corr + (bh * a.nbk) * a.Nq + (row < a.Nq ? row : a.Nq - 1) : nullptr;
  const float cbs = a.sm_scale * kLog2e;
  auto cb_of = [&](int t) { return BM && t < kt_end ? cbh[(int64_t)t * a.Nq] * cbs : 0.f; };
  float cb_cur = cb_of(t0);
  // PP with per_block_mean: this lane's row term of the key tile in ring slot `slot`, log2 units
  auto cb_at = [&](int slot) -> float {
    if constexpr (PP && BM)
      return reinterpret_cast<const float*>(cbring + slot * kCB)[32 * w + lr] * cbs;
    else
      return 0.f;
  };
  if constexpr (PP) {  // scores of T[0]; group 1 takes their softmax before its first step
    qk_tile<D, PV == 0>(kring, qf, lb, acc, magic);
    if (grp1) {
      int lim;
      const void* mtile;
      visible(t0, lim, mtile);
      if (part_cur)
        softmax_phase<D, PV, true, BM>(acc, P, c_cur, rs, g, lim, static_cast<const uint8_t*>(mtile), a.mask_vec4,
                                       cb_at(0));
      else
        softmax_phase<D, PV, false, BM>(acc, P, c_cur, rs, g, kBlockN - 1, nullptr, false, cb_at(0));
      // O is still zero: the factor returned (0) needs no application
    }
  } else {  // scores of T[0] and the row maxima of its first key block; the first PV operands
    qk_tile<D, (PV == 0 && !MF)>(kring, qf, lb, acc, magic);
    int lim;
    const void* mtile;
    visible(t0, lim, mtile);
    if constexpr (!MF) {  // (the float-mask step takes T[n]'s masking and maxima itself)
      if (part_cur) mask_scores(acc, g, lim, static_cast<const uint8_t*>(mtile), a.mask_vec4);
#pragma unroll
      for (int p = 0; p < 4; ++p) max_piece(acc, ch, p);
    }
#pragma unroll
    for (int r = 0; r < StepGeom<D, PV>::LA; ++r) vpre[r] = vfrag<D, PV>(vring + (kNS - 1) * G::V_BYTES, lb, g, r);
  }
  // loads this wave issues per step (its share of one V and one K tile), for the vmcnt waits
  const int nload = segs_of_wave<G::V_SEGS_ALL, kWaves>(w) + segs_of_wave<G::K_SEGS_ALL, kWaves>(w);

  int n = 0;
  int tc = t0, tn = t1, tnn = t2, tnnn = t3;  // T[n] .. T[n+3]
  float ks_n1 = scalar_ld(ksh, t1 < kt_end ? t1 : 0);  // k-scale of T[n+1]
  // PP: the phase-split step takes T[n+1]'s scale at its start, where no LDS read is in flight, so
  // the k-scales come by scalar loads issued three tiles ahead into a ring indexed by the step's slot
  // (T[i]'s scale in ksr[i % 4]).  (A vector load there would be waited for by vmcnt, and the
  // compiler's wait would also drain the staging loads.)
  float ksr[4] = {0.f, ks_n1, PP ? scalar_ld(ksh, t2 < kt_end ? t2 : 0) : 0.f, 0.f};
  auto step = [&](auto slot) -> bool {
    constexpr int Q = decltype(slot)::value;  // n % kNS
    if (tc >= kt_end) return false;
    const float cb_nxt = cb_of(tn);  // before the staging loads (see above)
    // The barrier orders this step's staging writes after every wave's reads of the slots they
    // reuse (read and consumed in earlier steps), and makes the loads waited for at the end of the
    // previous step visible to all waves.  LDS reads still in flight (the next PV operands, of a
    // slot not rewritten here) may cross it.
    asm volatile("s_barrier" ::: "memory");
    st.load_v(clampt(tnn), vring + ((Q + 2) % kNS) * G::V_BYTES);
    st.load_k(clampt(tnnn), kring + ((Q + 3) % kNS) * G::K_BYTES);
    const float ks_n2 = ks_load(tnn);  // k-scale of T[n+2], after the staging loads
    const char* sVp = vring + ((Q + kNS - 1) % kNS) * G::V_BYTES;  // V of T[n-1]
    const char* sVn = vring + Q * G::V_BYTES;                      // V of T[n]
    const char* sKn = kring + ((Q + 1) % kNS) * G::K_BYTES;        // K of T[n+1]
    const bool part_nxt = partial(tn);
    float alpha;
    if constexpr (MF) {
      int lim;
      const void* mtile;
      visible(tc, lim, mtile);
      bool has_m, full4;
      const void* mf = fmask_of(tc, has_m, full4);
      // a per-lane test of a wave-uniform condition (as in partial()): two specialised steps
      if (__builtin_amdgcn_mbcnt_lo(0u, has_m ? 1u : 0u) != 0u)
        alpha = tile_step<D, PV, true, true>(acc, ch, P, vpre, sKn, sVp, sVn, qf, o, c_cur, rs, lb, g, lim, mf, full4,
                                             true);
      else
        alpha = tile_step<D, PV, true, true>(acc, ch, P, vpre, sKn, sVp, sVn, qf, o, c_cur, rs, lb, g, lim, mf, full4,
                                             false);
    } else if (part_cur || part_nxt) {
      int lim;
      const void* mtile;
      visible(tn, lim, mtile);
      alpha = tile_step<D, PV, true, false, BM>(acc, ch, P, vpre, sKn, sVp, sVn, qf, o, c_cur, rs, lb, g, lim, mtile,
                                                a.mask_vec4, false, cb_cur, magic);
    } else {
      alpha = tile_step<D, PV, false, false, BM>(acc, ch, P, vpre, sKn, sVp, sVn, qf, o, c_cur, rs, lb, g,
                                                 kBlockN - 1, nullptr, false, false, cb_cur, magic);
    }
    // O moves to T[n]'s reference maximum after the PV of T[n-1] (rare under the lazy maximum)
    if (__ballot(alpha != 1.f)) scale_acc<D>(o, alpha);
    cb_cur = cb_nxt;
    part_cur = part_nxt;
    // the loads of the previous steps (and the k-scale of T[n+1]) must have landed before the next
    // barrier; this step's staging loads and k-scale load stay in flight
    switch (nload) {
      case 0: wait_vmcnt<1>(); break;
      case 1: wait_vmcnt<2>(); break;
      case 2: wait_vmcnt<3>(); break;
      case 3: wait_vmcnt<4>(); break;
      case 4: wait_vmcnt<5>(); break;
      case 5: wait_vmcnt<6>(); break;
      default: wait_vmcnt<7>(); break;
    }
    c_cur = scale_from(tn, ks_n1);
    ks_n1 = ks_n2;
    tc = tn;
    tn = tnn;
    tnn = tnnn;
    tnnn = next_tile(tnnn);
    ++n;
    return true;
  };
  // Phase-split step n: both groups read K of T[n+1] and V of T[n] (slots (n+1)%4 and n%4), and
  // issue the loads of V of T[n+2] and K of T[n+3] into slots last read two steps earlier.  Group
  // 0: softmax of T[n], then QK of T[n+1] and PV of T[n].  Group 1 (T[n]'s softmax done a step
  // earlier): QK of T[n+1] and PV of T[n], then the softmax of T[n+1].  The softmax past the last
  // tile sees only masked scores (P = 0, factor 1).
  auto pstep = [&](auto slot) -> bool {
    constexpr int Q = decltype(slot)::value;
    if (tc >= kt_end) return false;
    asm volatile("s_barrier" ::: "memory");
    const char* sV = vring + Q * G::V_BYTES;                // V of T[n]
    const char* sK = kring + ((Q + 1) % kNS) * G::K_BYTES;  // K of T[n+1]
    auto stage = [&] {  // this step's staging loads and the k-scale of T[n+3]
      st.load_v(clampt(tnn), vring + ((Q + 2) % kNS) * G::V_BYTES);
      st.load_k(clampt(tnnn), kring + ((Q + 3) % kNS) * G::K_BYTES);
      load_cb(clampt(tnnn), (Q + 3) % kNS);
      ksr[(Q + 3) % kNS] = scalar_ld(ksh, tnnn < kt_end ? tnnn : 0);
    };
    v4i pre[kPhaseLA];
    auto preload = [&] {
#pragma unroll
      for (int r = 0; r < kPhaseLA; ++r) pre[r] = kfrag<D>(sK, lb, r);
    };
    const float c_nxt = scale_from(tn, ksr[(Q + 1) % kNS]);
    // Group 1 reads its first operands and streams its MFMAs right after the barrier, and issues the
    // loads after them; group 0 starts its softmax at once and issues the loads and its operand reads
    // after it, so group 1's reads are served first.
    if (grp1) {
      preload();
      mfma_phase<D, PV>(pre, sK, sV, P, qf, o, acc, lb, g, magic);
      stage();
    }
    const int ts = grp1 ? tn : tc;
    const float cs = grp1 ? c_nxt : c_cur;
    int lim;
    const void* mtile;
    visible(ts, lim, mtile);
    float alpha;
    const float cb = cb_at(grp1 ? (Q + 1) % kNS : Q);  // per_block_mean: T[n+1]'s or T[n]'s term
    if (partial(ts))
      alpha = softmax_phase<D, PV, true, BM>(acc, P, cs, rs, g, lim, static_cast<const uint8_t*>(mtile), a.mask_vec4,
                                             cb);
    else
      alpha = softmax_phase<D, PV, false, BM>(acc, P, cs, rs, g, kBlockN - 1, nullptr, false, cb);
    if (__ballot(alpha != 1.f)) scale_acc<D>(o, alpha);
    if (!grp1) {
      stage();
      preload();
      mfma_phase<D, PV>(pre, sK, sV, P, qf, o, acc, lb, g, magic);
    }
    // every wave issues the same loads per step at d = 128: a compile-time wait, so the compiler
    // sees that the k-scale read at the next step's start has landed
    static_assert(G::V_SEGS_ALL % kWaves == 0 && G::K_SEGS_ALL % kWaves == 0, "uniform staging");
    constexpr int kNL = (G::V_SEGS_ALL + G::K_SEGS_ALL) / kWaves;
    wait_vmcnt<kNL + (BM ? 1 : 0)>();  // (one load more with per_block_mean: the row terms)
    c_cur = c_nxt;
    tc = tn;
    tn = tnn;
    tnn = tnnn;
    tnnn = next_tile(tnnn);
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
  if (!PP && n > 0) pv_tile<D, PV>(vring + ((n - 1) % kNS) * G::V_BYTES, P, lb, g, o);

  // epilogue: normalize, store O (bf16, fp16 or fp32) and the LSE.  The arguments it needs are
  // read again from the kernel-argument segment here, so they hold no SGPRs across the loop.
  const AttnArgs& ea = *kernarg_reload<AttnArgs>();
  const float l_tot = rs.l + __shfl_xor(rs.l, 32);
  const float* vsh = PV == 1 ? ea.vscale + bhk * D : nullptr;
  // A row without a visible key (l = 0) stores O = 0 and LSE = -inf, whatever a zero
  // probability times a NaN in V left in o; a NaN l (a NaN score) makes both NaN.
  const bool live = l_tot != 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
  const float* vmh = (ea.vmean && live) ? ea.vmean + bhk * D : nullptr;  // smooth_v
  // channels db*32 + rq*8 + 4g .. +3 of this lane's row, normalized
  auto norm = [&](int db, int rq, float (&f)[4]) {
    const int d0 = db * 32 + rq * 8 + g * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (PV == 1)
        f[e] = o[db][rq * 4 + e] * (vsh[d0 + e] * inv);
      else
        f[e] = o[db][rq * 4 + e] * inv;
      if (vmh) f[e] = f[e] + vmh[d0 + e];
      f[e] = live ? f[e] : 0.f;
    }
  };
  // O leaves through LDS: each wave writes its 32 rows into its own region of the idle ring (rows of
  // RB = 2*D bytes, 16-byte chunks XOR-swizzled by the row) and reads them back so that consecutive
  // lanes store consecutive 16-byte chunks of one row.  16-bit output is one pass; fp32 is two,
  // of D/2 channels each.
  constexpr int RB = 2 * D, CPR = RB / 16;  // region row bytes, chunks per row
  __syncthreads();                          // every wave's last reads of the ring are done
  char* const so = smem + w * (32 * RB);
  const int64_t orow0 = b * ea.o_sb + h * ea.o_sh + (sq.off + r0w) * ea.o_sn;  // elements
  auto store_region = [&](char* outp, int osz, int ch0) {
    __syncthreads();  // the region is written
#pragma unroll
    for (int it = 0; it < CPR / 2; ++it) {
      const int r = it * (64 / CPR) + lane / CPR, c = lane % CPR;
      const v4i val = *reinterpret_cast<const v4i*>(so + r * RB + ((c ^ (r & (CPR - 1))) * 16));
      if (r0w + r < nq)
        *reinterpret_cast<v4i*>(outp + (orow0 + r * ea.o_sn + ch0) * osz + c * 16) = val;
    }
  };
  if (ea.out_kind == 2) {  // fp32, e.g. partial results that are merged later
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (pass) __syncthreads();  // the previous pass's reads of the region are done
#pragma unroll
      for (int db = pass * D / 64; db < (pass + 1) * D / 64; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float f[4];
          norm(db, rq, f);
          const int c = (db - pass * D / 64) * 8 + rq * 2 + g;
          *reinterpret_cast<float4*>(so + lr * RB + ((c ^ (lr & (CPR - 1))) * 16)) = make_float4(f[0], f[1], f[2], f[3]);
        }
      store_region(static_cast<char*>(ea.out), 4, pass * D / 2);
    }
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float f[4];
        norm(db, rq, f);
        uint2 pk;
        if (ea.out_kind == 1) {
          pk.x = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[0], f[1]}), v2h));  // RNE
          pk.y = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[2], f[3]}), v2h));
        } else {
          pk.x = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[0], f[1]}), v2bf));  // RNE
          pk.y = __builtin_bit_cast(unsigned, __builtin_convertvector((v2f{f[2], f[3]}), v2bf));
        }
        const int c = db * 4 + rq;
        *reinterpret_cast<uint2*>(so + lr * RB + ((c ^ (lr & (CPR - 1))) * 16) + g * 8) = pk;
      }
    store_region(static_cast<char*>(ea.out), 2, 0);
  }
  if (row < nq && g == 0 && ea.lse) {
    float v = -INFINITY;
    if (l_tot != 0.f) {
      // l_tot sums 2^(s - pm) over the row (e4m3 P carries its scale 448 * 2^-tau inside pm)
      v = (rs.pm + log2f(l_tot)) * kLn2 + ea.sm_scale * ea.corr[bh * ea.Nq + row];
    }
    ea.lse[b * ea.l_sb + h * ea.l_sh + sq.off + row] = v;
  }
}

// Raw int32 scores of a window of one head, via the same staging (Stager, swizzled LDS rows),
// operand reads (LaneBases, kfrag) and MFMA sequence (qk_mfma) as every tile step of k_attn_fwd.
// grid = (32-row blocks, 64-key tiles) covering the window; block = one wave.
template <int D>
__global__ __launch_bounds__(64) void k_debug_qk(DebugQKArgs a, int64_t Nq_pad) {
  __shared__ __attribute__((aligned(16))) char sK[kBlockN * D];
  const int lane = threadIdx.x, lr = lane & 31, g = lane >> 5;
  const int64_t rb = a.row0 / 32 + blockIdx.x;
  const int kt = (int)(a.col0 / kBlockN) + (int)blockIdx.y;
  Stager<D, 0, 1> st;
  st.init(a.k8h, reinterpret_cast<const uint8_t*>(a.k8h), a.Nk_pad, 0, lane);
  st.load_k(kt, sK);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v4i qf[D / 32];
  const int64_t row = rb * 32 + lr;
  load_q_frags<D>(a.q8h, row, Nq_pad, g, qf);
  LaneBases lb;
  lb.init(lr, g);
  v16i acc[2];
  qk_tile<D>(sK, qf, lb, acc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = (int64_t)kt * kBlockN + key_of(kb, r, g);
      if (row >= a.row0 && row < a.row0 + a.nrows && j >= a.col0 && j < a.col0 + a.ncols)
        a.out[(row - a.row0) * a.ncols + (j - a.col0)] = acc[kb][r];
    }
}

// Every variant instantiated explicitly: the launches below alone do not make hipcc's host pass
// emit the launch stubs of the MF = 0 kernels.
template __global__ void k_attn_fwd<128, 0, 0, 0, 0>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 0, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 0, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 0, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 0, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 1, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 1, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 1, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 1, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 1, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 1, 0>(AttnArgs);
template __global__ void k_attn_fwd<128, 0, 0, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 0, 0>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 1, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 1, 0>(AttnArgs);
template __global__ void k_attn_fwd<128, 1, 0, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<64, 0, 0, 0, 0>(AttnArgs);
template __global__ void k_attn_fwd<64, 0, 0, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<64, 0, 1, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<64, 0, 0, 1, 0>(AttnArgs);
template __global__ void k_attn_fwd<64, 0, 0, 1, 1>(AttnArgs);
template __global__ void k_attn_fwd<64, 1, 0, 0, 0>(AttnArgs);
template __global__ void k_attn_fwd<64, 1, 0, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<64, 1, 1, 0, 1>(AttnArgs);
template __global__ void k_attn_fwd<64, 1, 0, 1, 0>(AttnArgs);
template __global__ void k_attn_fwd<64, 1, 0, 1, 1>(AttnArgs);

// Launches at d = 128 without a float mask run the phase-split schedule (build with -DSAGE_PHASE_SPLIT=0 for the
// interleaved tile_step schedule everywhere, e.g. to compare the two).
#ifndef SAGE_PHASE_SPLIT
#define SAGE_PHASE_SPLIT 1
#endif
constexpr bool kPhaseSplit = SAGE_PHASE_SPLIT;

// a mask always comes with its tile table (the host classifies the tiles first)
template <int D, int PV, int MF, int BM>
static void launch_attn_t(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if constexpr (MF)
    k_attn_fwd<D, PV, MF, BM, 1><<<grid, kAttnThreads, 0, s>>>(a);
  else if (a.mtiles) {
    if constexpr (D == 128 && kPhaseSplit)
      k_attn_fwd<D, PV, MF, BM, 1, 1><<<grid, kAttnThreads, 0, s>>>(a);
    else
      k_attn_fwd<D, PV, MF, BM, 1><<<grid, kAttnThreads, 0, s>>>(a);
  }
  else if constexpr (D == 128 && kPhaseSplit)
    k_attn_fwd<D, PV, MF, BM, 0, 1><<<grid, kAttnThreads, 0, s>>>(a);
  else
    k_attn_fwd<D, PV, MF, BM, 0><<<grid, kAttnThreads, 0, s>>>(a);
}

// the float-mask and per_block_mean variants are not combined (the host rejects both at once)
template <int D, int PV>
static void launch_attn_p(const AttnArgs& a, unsigned grid, hipStream_t s) {
  if (a.mask_f32)
    launch_attn_t<D, PV, 1, 0>(a, grid, s);
  else if (a.blk_corr)
    launch_attn_t<D, PV, 0, 1>(a, grid, s);
  else
    launch_attn_t<D, PV, 0, 0>(a, grid, s);
}

template <int D>
static void launch_attn_d(const AttnArgs& a, int pv_fp8, unsigned grid, hipStream_t s) {
  if (pv_fp8)
    launch_attn_p<D, 1>(a, grid, s);
  else
    launch_attn_p<D, 0>(a, grid, s);
}

hipError_t launch_attn(const AttnArgs& a, int d, int pv_fp8, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nQT * a.B * a.H);
  if (d == 128)
    launch_attn_d<128>(a, pv_fp8, grid, s);
  else
    launch_attn_d<64>(a, pv_fp8, grid, s);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const DebugQKArgs& a, int d, int64_t Nq_pad, hipStream_t s) {
  const int64_t rb0 = a.row0 / 32, rb1 = (a.row0 + a.nrows + 31) / 32;
  const int64_t kt0 = a.col0 / kBlockN, kt1 = (a.col0 + a.ncols + kBlockN - 1) / kBlockN;
  dim3 grid((unsigned)(rb1 - rb0), (unsigned)(kt1 - kt0));
  if (d == 128)
    k_debug_qk<128><<<grid, 64, 0, s>>>(a, Nq_pad);
  else
    k_debug_qk<64><<<grid, 64, 0, s>>>(a, Nq_pad);
  return hipGetLastError();
}

}  // namespace sage
