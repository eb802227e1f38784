// sage_device.h -- device-side helpers shared by the gfx950 kernels of libsage_mi355x.
//
// Vector types, bf16 handling, the LDS swizzle and the prepared-V key permutation.  Everything
// here is device code for one target (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kQuantBlock = 64;  // tokens per INT8 quantization block (Q and K)
constexpr int kBlockN = 64;      // keys per attention tile: one K-scale per tile
constexpr int kBlockM = 256;     // query rows per attention workgroup
constexpr int kMaskTileRows = kBlockM;       // mask classification granularity (rows)

// int32 accumulator bias: the bit pattern of 1.5 * 2^23.  For |acc| < 2^22 the int32 sum
// 0x4B400000 + acc is the binary32 pattern of the float 1.5*2^23 + acc, so an MFMA started from
// this value yields the scores already as floats (offset by 1.5*2^23).
constexpr int kMagicBits = 0x4B400000;
constexpr float kLog2e = 1.4426950408889634f;  // log2(e), rounded to fp32
constexpr float kLn2 = 0.6931471805599453f;    // ln(2), rounded to fp32
constexpr float kMagic = 12582912.0f;

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(static_cast<unsigned>(h) << 16);
}

// An input element (Q, K or V) as fp32: bf16 (IN = 0) or IEEE binary16 (IN = 1) bits.  Exact.
template <int IN>
__device__ __forceinline__ float in_to_f32(unsigned short h) {
  if constexpr (IN == 0)
    return bf16_to_f32(h);
  else
    return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<unsigned short>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

// Maximum of two magnitudes (values with a clear sign bit, NaN included) that keeps NaN: the
// unsigned order of such bit patterns is finite < +inf < NaN, so a block holding a NaN gets a NaN
// maximum and hence a NaN scale (fmaxf would drop it).
__device__ __forceinline__ float mag_max(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
}

// Sequence b of a batch: the row of its first token and its length.  Dense batches (cu null)
// have n rows per batch entry, addressed through the batch stride.  A packed variable-length batch
// holds sequence b in rows [cu[b], cu[b+1]) of a buffer of `total` rows; offsets and lengths are
// clamped to that buffer and to n, so any cu contents keep every access inside it.
struct SeqSpan {
  int64_t off, len;
};
__device__ __forceinline__ SeqSpan seq_span(const int* cu, int64_t b, int64_t n, int64_t total) {
  if (cu == nullptr) return {0, n};
  int64_t lo = cu[b], hi = cu[b + 1];
  lo = lo < 0 ? 0 : (lo > total ? total : lo);
  hi = hi < lo ? lo : (hi > total ? total : hi);
  return {lo, hi - lo < n ? hi - lo : n};
}

// LDS swizzle of 16-byte chunks inside a row.  A fragment read (ds_read_b128) fetches one logical
// chunk from each of 32 consecutive rows, and LDS serves it 16 lanes (16 rows) at a time.  With
// 128-byte rows the 16 rows of such a group hit distinct banks iff the even rows land on 8
// distinct chunks and so do the odd rows; with 64-byte rows iff the rows of each residue modulo 4
// land on 4 distinct chunks.  The swizzles below meet that (and keep every 8 consecutive rows on
// distinct chunks) while depending on the row modulo 16 only.
__device__ __forceinline__ int swz128(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
template <int ROW_BYTES>
__device__ __forceinline__ int lds_chunk_offset(int row, int chunk) {
  if constexpr (ROW_BYTES == 128)
    return row * 128 + ((chunk ^ swz128(row)) << 4);
  else
    return row * 64 + ((chunk ^ swz64(row)) << 4);
}

// Direct global -> LDS loads (buffer_load ... lds) take their LDS destination as an address-space-3
// pointer; buffer resources carry this word 3 (gfx9: 32-bit data format).
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kBufferWord3 = 0x00020000;

// s_waitcnt with vmcnt = N (other counters untouched): all but this wave's N most recent vector
// memory operations -- here the direct-to-LDS loads -- have completed
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
}

// Wave-uniform read-only scalars (k-scales, mask-tile states) are read through the constant
// address space so they become scalar loads: a vector load here would be counted by vmcnt, whose
// in-order wait would also drain the in-flight direct-to-LDS prefetches.
typedef __attribute__((address_space(4))) const float cfloat_t;
typedef __attribute__((address_space(4))) const int cint_t;
__device__ __forceinline__ float scalar_ld(const float* p, int i) { return ((cfloat_t*)p)[i]; }
__device__ __forceinline__ int scalar_ld(const int* p, int i) { return ((cint_t*)p)[i]; }

// Attention workgroup -> (query head bh = b*H + h, q-tile qt).  Workgroup ids go round-robin over
// the 8 XCDs (each with its own L2).  When the key/value heads split evenly, XCD x works through
// key/value heads x, x+8, ..., each with all its query heads and q-tiles in a row, so K and V stay
// in one L2 and heads of unequal cost (sequences of a packed batch) spread evenly.  Otherwise
// consecutive logical ids land on the same XCD.  Causal q-tiles run longest first.
__device__ __forceinline__ void map_workgroup(int64_t B, int64_t H, int64_t Hkv, int nQT, int causal, int64_t& bh,
                                              int& qt) {
  const int total = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, jx = bid >> 3;
  const int grp = (int)(H / Hkv);  // query heads per key/value head
  const int64_t units = B * Hkv;
  if (units % 8 == 0 && (int64_t)total == units * grp * nQT) {
    const int per_unit = grp * nQT;
    const int64_t u = xcd + 8 * (int64_t)(jx / per_unit);  // b * Hkv + key/value head
    const int r = jx % per_unit;
    bh = (u / Hkv) * H + (u % Hkv) * grp + r / nQT;
    qt = r % nQT;
  } else {
    const int per = total >> 3, rem = total & 7;
    const int L = xcd < rem ? xcd * (per + 1) + jx : rem * (per + 1) + (xcd - rem) * per + jx;
    bh = L / nQT;
    qt = L % nQT;
  }
  if (causal) qt = nQT - 1 - qt;
}

}  // namespace sage
