// sage_merge.hip -- merging partial attention results over disjoint key sets (gfx950).
//
// With part s covering keys K_s, O_s = sum_{j in K_s} e^{s_j} v_j / sum_{j in K_s} e^{s_j} and
// LSE_s = log sum_{j in K_s} e^{s_j}, the result over the union is LSE = log sum_s e^{LSE_s} and
// O = sum_s e^{LSE_s - LSE} O_s.  This is what the LSE output is for on the SageAttention docs
// digest ("Utilize SageAttention for Distributed Inference": sequence parallelism, Ring
// Attention); the formula is the softmax's own identity.  The kernel streams the parts once: it is
// HBM-bound (S*d*esize + d*out_esize + 4*(S+1) bytes per row).
#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kMergeThreads = 256;

// eight consecutive elements of a partial output as fp32
template <int PART>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
  if constexpr (PART == 2) {
    const float4 lo = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 hi = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
    x[0] = lo.x;
    x[1] = lo.y;
    x[2] = lo.z;
    x[3] = lo.w;
    x[4] = hi.x;
    x[5] = hi.y;
    x[6] = hi.z;
    x[7] = hi.w;
  } else {
    const u16x8 v = *reinterpret_cast<const u16x8*>(static_cast<const unsigned short*>(base) + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = in_to_f32<PART>(v[j]);
  }
}

// One thread per (row, 8 channels).  grid = ceil(R * d/8 / 256).
template <int PART>
__global__ __launch_bounds__(kMergeThreads) void k_merge_lse(MergeArgs a) {
  const int cgs = (int)(a.d / 8);
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t r = t / cgs;
  if (r >= a.R) return;
  const int cg = (int)(t % cgs);
  // the largest LSE, NaN if any part's is NaN (that NaN then reaches O and the LSE)
  float m = -INFINITY;
  for (int64_t s = 0; s < a.S; ++s) {
    const float x = a.lse_parts[s * a.R + r];
    m = (x != x || x > m) ? x : m;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int64_t s = 0; s < a.S; ++s) {
      const float ls = a.lse_parts[s * a.R + r];
      if (ls == -INFINITY) continue;  // a part without visible keys: its O is not read
      const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);
      tot += w;
      float x[8];
      load8<PART>(a.parts, (s * a.R + r) * a.d + cg * 8, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(w, x[j], acc[j]);
    }
  }
  const float inv = tot != 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] *= inv;
  const int64_t bh = r / a.Nq, i = r % a.Nq, b = bh / a.H, h = bh % a.H;
  const int64_t obase = b * a.o_sb + h * a.o_sh + i * a.o_sn + cg * 8;
  if (a.out_kind == 2) {
    float* o = static_cast<float*>(a.out) + obase;
    *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint4 pk;
    unsigned w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v2f f2 = {acc[2 * q], acc[2 * q + 1]};
      w4[q] = a.out_kind == 1 ? __builtin_bit_cast(unsigned, __builtin_convertvector(f2, v2h))    // RNE
                              : __builtin_bit_cast(unsigned, __builtin_convertvector(f2, v2bf));  // RNE
    }
    pk.x = w4[0];
    pk.y = w4[1];
    pk.z = w4[2];
    pk.w = w4[3];
    *reinterpret_cast<uint4*>(static_cast<unsigned short*>(a.out) + obase) = pk;
  }
  if (cg == 0 && a.lse) a.lse[r] = m == -INFINITY ? -INFINITY : m + log2f(tot) * kLn2;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t threads = a.R * (a.d / 8);
  const unsigned grid = (unsigned)((threads + kMergeThreads - 1) / kMergeThreads);
  if (a.part_kind == 2)
    k_merge_lse<2><<<grid, kMergeThreads, 0, s>>>(a);
  else if (a.part_kind == 1)
    k_merge_lse<1><<<grid, kMergeThreads, 0, s>>>(a);
  else
    k_merge_lse<0><<<grid, kMergeThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sage
