// sage_clock.hip -- the shader clock under load, measured on the GPU (gfx950).
//
// k_sclk_probe keeps every SIMD busy with FP16 MFMAs and dependent VALU work (the instruction mix
// of the attention kernels) for a fixed number of loop trips, and its first wave of each workgroup
// reads the shader clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) at
// the start and at the end.  The clock in MHz is 100 * (memtime difference) / (memrealtime
// difference).  k_sclk_idle reads the same counters around a sleep loop instead, to measure the
// clock that other kernels running beside it get.
#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kProbeThreads = 256;  // 4 waves: one per SIMD of the CU the workgroup lands on

// Idle form: one wave per workgroup sleeps (s_sleep, about 8k clocks a trip) between the counter
// reads, adding no load: launched on a second stream beside other kernels it measures the clock
// they run at.
__global__ __launch_bounds__(64) void k_sclk_idle(unsigned long long* __restrict__ out, int iters) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) __builtin_amdgcn_s_sleep(127);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    unsigned long long* o = out + 4 * (int64_t)blockIdx.x;
    o[0] = t0;
    o[1] = r0;
    o[2] = t1;
    o[3] = r1;
  }
}

__global__ __launch_bounds__(kProbeThreads) void k_sclk_probe(unsigned long long* __restrict__ out, int iters,
                                                              float seed) {
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  v16f acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  v8h a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(seed * (float)(i + 1));
    b[i] = (_Float16)(seed * (float)threadIdx.x);
  }
  float x = seed * (float)threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[1], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) x = __builtin_fmaf(x, 0.999f, 1e-3f);
    x = __builtin_amdgcn_exp2f(x * 1e-3f);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    unsigned long long* o = out + 4 * (int64_t)blockIdx.x;
    o[0] = t0;
    o[1] = r0;
    o[2] = t1;
    o[3] = r1;
  }
  // the results are kept alive, so the loop is not removed
  asm volatile("" ::"v"(x));
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(acc[j][i]));
}

hipError_t launch_sclk_probe(unsigned long long* out, int nblocks, int iters, int load, hipStream_t s) {
  if (load)
    k_sclk_probe<<<(unsigned)nblocks, kProbeThreads, 0, s>>>(out, iters, 1e-3f);
  else
    k_sclk_idle<<<(unsigned)nblocks, 64, 0, s>>>(out, iters);
  return hipGetLastError();
}

}  // namespace sage
