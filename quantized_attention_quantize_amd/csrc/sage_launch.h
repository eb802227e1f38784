// sage_launch.h -- kernel argument blocks and launcher declarations (internal to libsage_mi355x).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Online-softmax reference maximum (log2 units) by PV type: it moves only when a tile's maximum
// exceeds it by more than this, so O is rarely rescaled.  FP16 P is lazy by 8 (p = exp(s - m)
// stays <= 2^8, well inside fp16); e4m3 P is e4m3(448 * p) against the exact running maximum
// (p <= 1), so the row maximum maps to 448.
constexpr float kSoftmaxTau[2] = {8.f, 0.f};
// Whether the softmax denominator sums P as rounded for the PV product rather than the fp32 p,
// by PV type: both sum the fp32 p.
constexpr int kRowsumRounded[2] = {0, 0};

struct QuantArgs {
  const unsigned short* q;  // bf16 or fp16 (in_fp16), as K
  const unsigned short* k;
  int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn;
  int8_t* q8;
  int8_t* k8;
  float* qs;
  float* ks;
  float* kmean;
  float* corr;
  int64_t B, H, Hkv, Nq, Nk, d, Nq_pad, Nk_pad;  // Q has H heads, K has Hkv (Hkv divides H)
  int nbq, nbk;
  int in_fp16;
  // packed variable-length batch (null: dense): sequence b = rows [cu[b], cu[b+1]) of total rows,
  // at most Nq (Nk) long; the batch stride is then unused
  const int* cu_q;
  const int* cu_k;
  int64_t total_q, total_k;
  // per_block_mean (null: global-mean smoothing): K block means [B][Hkv][nbk][d] and the score
  // terms [B][H][nbk][Nq]; kmean and corr then hold zeros
  float* kbmean;
  float* blk_corr;
};

struct PrepVArgs {
  const unsigned short* v;  // bf16 or fp16 (in_fp16)
  int64_t v_sb, v_sh, v_sn;
  void* vt;             // fp16 or e4m3 [B][H][d][Nk_pad]
  float* vscale;        // fp8 only: [B][H][d]
  float* vmax_partial;  // fp8 only: [B][H][nchunk][d]
  float* vmean;         // fp16 only, smooth_v: [B][H][d] written here and subtracted (null: off)
  double* vsum_partial;  // smooth_v: [B][H][nchunk][d] fp64 partial sums
  int64_t B, H, Nk, d, Nk_pad;
  int nchunk;
  int in_fp16;
  const int* cu_k;  // packed variable-length batch (null: dense), as in QuantArgs
  int64_t total_k;
};

struct MaskTileArgs {
  const void* mask;  // uint8 (nonzero = attend) or, with f32, fp32 additive (-inf = drop)
  int f32;
  int64_t sb, sh, sq;
  int64_t B, Hm, Nq, Nk;
  int nQT, nKT;
  int vec16;  // rows and base are 16-byte aligned: read 16 bytes at a time
  int* state;  // [B*Hm][nQT][nKT]: bits 0-1: 0 all masked, 1 all visible (fp32: all exactly 0), 2 mixed;
               // bits 2+: the row block's next tile that is not all masked (nKT if none), from k_mask_walk
};

struct AttnArgs {
  const int8_t* q8;
  const int8_t* k8;
  const float* qs;
  const float* ks;
  const float* corr;
  const void* vt;  // prepared V
  const float* vscale;
  const float* vmean;  // smooth_v: [B][Hkv][d] added back to O (null: off)
  const float* blk_corr;  // per_block_mean: [B][H][nbk][Nq] score terms (null: global-mean smoothing)
  const void* mask;  // element mask (only read for mixed tiles); strides in elements
  int64_t m_sb, m_sh, m_sq;
  int mask_f32;       // 0: uint8, nonzero = attend; 1: fp32 added to the scaled score, -inf = drop
  const int* mtiles;  // tile states or nullptr
  int64_t Hm;             // 0 = no mask
  void* out;    // out_kind 0: bf16, 1: fp16, 2: fp32
  int out_kind;
  int64_t o_sb, o_sh, o_sn;
  float* lse;  // nullptr = not requested
  int64_t B, H, Hkv, Nq, Nk, Nq_pad, Nk_pad;  // query head h reads key/value head h / (H / Hkv)
  int nbq, nbk, nQT, nKT;
  int causal;
  int mask_vec4;  // mask rows aligned to 4 elements: read 4 mask elements at a time
  float sm_scale;
  // packed variable-length batch (null: dense; Nq / Nk are then the longest sequence): query row
  // i of sequence b is output row cu_q[b] + i, and its LSE sits at b*l_sb + h*l_sh + cu_q[b] + i
  const int* cu_q;
  const int* cu_k;
  int64_t total_q, total_k;
  int64_t l_sb, l_sh;
};

struct MergeArgs {
  const void* parts;      // [S][R][d] partial outputs, part_kind 0: bf16, 1: fp16, 2: fp32
  const float* lse_parts;  // [S][R] natural-log LSEs (-inf: the part saw no key of the row)
  int64_t S, R, d;        // R = B*H*Nq rows, row r = (b*H + h)*Nq + i
  int64_t H, Nq;
  void* out;              // out_kind 0: bf16, 1: fp16, 2: fp32; element strides below
  int64_t o_sb, o_sh, o_sn;
  int out_kind, part_kind;
  float* lse;             // [R] or nullptr
};

struct DebugQKArgs {
  const int8_t* q8h;  // head base
  const int8_t* k8h;
  int64_t Nk_pad;
  int64_t row0, nrows, col0, ncols;
  int32_t* out;
};

// FP4 microscaling method (MX FP4 Q, K, V; e4m3 P).  Layouts (bytes unless noted):
//   q4  [B][H][Nq_pad][d/2], k4 [B][Hkv][Nk_pad][d/2]: e2m1 pairs, low nibble = even channel
//   q_sc [B][H][Nq_pad][d/32], k_sc [B][Hkv][Nk_pad][d/32]: E8M0 bytes in lane order -- block
//        2*cs + g (channels [64 cs + 32 g, +32)) at byte g*(d/64) + cs
//   v4t [B][Hkv][d][Nk_pad/2]: V transposed, e2m1 pairs along tokens, low nibble = even token
//   v_sc [B][Hkv][Nk_pad/32][d]: E8M0 of (32-token block, channel 32 db + l) at byte l*(d/32) + db
//   k_mean fp32 [B][Hkv][d]; q_mean fp32 [B][H][nqm][d]; qk_corr fp32 [B][H][nqm][Nk_pad]
//   (zero past Nk); lse_corr fp32 [B][H][Nq]
struct Fp4QuantArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn;
  uint8_t* q4;
  uint8_t* q_sc;
  uint8_t* k4;
  uint8_t* k_sc;
  uint8_t* v4t;
  uint8_t* v_sc;
  float* k_mean;
  float* q_mean;
  float* qk_corr;
  float* lse_corr;
  int64_t B, H, Hkv, Nq, Nk, d, Nq_pad, Nk_pad;
  int nqm;        // Q smoothing rows: ceil(Nq/128) (per_block) or 1 (global mean)
  int per_block;  // Q smoothed by its 128-token block means (else by its global mean, in q_mean)
  int in_fp16;
};

struct Fp4AttnArgs {
  const uint8_t* q4;
  const uint8_t* q_sc;
  const uint8_t* k4;
  const uint8_t* k_sc;
  const uint8_t* v4t;
  const uint8_t* v_sc;
  const float* qk_corr;
  const float* lse_corr;
  void* out;  // out_kind 0: bf16, 1: fp16, 2: fp32
  int out_kind;
  int64_t o_sb, o_sh, o_sn;
  float* lse;  // nullptr = not requested
  int64_t B, H, Hkv, Nq, Nk, Nq_pad, Nk_pad;
  int nqm, per_block, nQT, causal;
  float sm_scale;
};

struct Fp4DebugArgs {
  Fp4AttnArgs a;
  int64_t b, h, row0, nrows, col0, ncols;
  float* out;  // [nrows][ncols] raw scores S (before sm_scale)
};

hipError_t launch_kmean(const QuantArgs& a, double* partial, int nchunk, hipStream_t s);
hipError_t launch_quant(const QuantArgs& a, hipStream_t s);
hipError_t launch_block_corr(const QuantArgs& a, hipStream_t s);
hipError_t launch_prep_v(const PrepVArgs& a, int pv_fp8, hipStream_t s);
hipError_t launch_mask_tiles(const MaskTileArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int d, int pv_fp8, hipStream_t s);
hipError_t launch_debug_qk(const DebugQKArgs& a, int d, int64_t Nq_pad, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_sclk_probe(unsigned long long* out, int nblocks, int iters, int load, hipStream_t s);
int64_t token_mean_partial_doubles(int64_t B, int64_t H, int64_t N, int64_t d);
hipError_t launch_token_mean(const unsigned short* x, int in_fp16, int d, int64_t B, int64_t H, int64_t N, int64_t sb,
                             int64_t sh, int64_t sn, double* partial, float* mean, hipStream_t s);
// FP4 method: global means (K; Q when not per-block) need `partial` fp64 workspace of
// fp4_mean_partial_doubles() doubles
int64_t fp4_mean_partial_doubles(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d);
hipError_t launch_fp4_quant(const Fp4QuantArgs& a, double* partial, hipStream_t s);
hipError_t launch_fp4_attn(const Fp4AttnArgs& a, hipStream_t s);
hipError_t launch_fp4_debug(const Fp4DebugArgs& a, hipStream_t s);
int fp4_softmax_tau();  // lazy-maximum threshold of k_fp4_attn (log2 units)

}  // namespace sage
