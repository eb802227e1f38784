// bench_isa_rates.hip -- instruction throughput of the gfx950 pipes the attention kernels use.
//
// Each probe kernel runs a fixed number of independent instructions of one kind per lane; timed
// with HIP events, the result is the time one SIMD spends per wave-level instruction (ns), at 8
// waves per SIMD (the pipe's throughput) and at 1 wave per SIMD (one wave's issue rate).  The clock
// is measured in the same run: s_memtime (shader clock) against s_memrealtime (100 MHz) across a
// probe kernel.  bench.py turns these rates and the attention kernel's instruction counts into the
// VALU ceiling reported beside the MFMA ceiling.  Each probe's own clock is reported too: under the
// MFMA probes the chip clocks down, so clocks per instruction = ns x that probe's MHz.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o bench_isa_rates bench_isa_rates.hip && ./bench_isa_rates
//
// Prints one JSON object.
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kIter = 2048;  // loop trips; every kind issues 16 instructions per trip

enum Kind { EXP, FMA, ADD, CVT_I2F, CVT_PK_F16, MAX3, MFMA_I8, MFMA_F16, MFMA_F8, NKIND };
const char* kName[NKIND] = {"v_exp_f32", "v_fma_f32", "v_add_f32", "v_cvt_f32_i32", "v_cvt_pk_f16_f32",
                            "v_max3_i32", "v_mfma_i32_32x32x32_i8", "v_mfma_f32_32x32x16_f16",
                            "v_mfma_scale_f32_32x32x64_f8f6f4"};

// One output per thread: out[blockIdx.x * blockDim.x + threadIdx.x] (in bounds by the launch shape).
template <int K>
__global__ void k_rate(float* out, float seed, unsigned long long* clk) {
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float s = 0.f;
  if constexpr (K <= MAX3) {
    float x[16];
    int xi[16];
    const float y = seed * 1e-7f, z = seed * 1e-3f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = seed * (float)(threadIdx.x + i) * 1e-9f - 0.5f;
      xi[i] = (int)threadIdx.x + i;
    }
    for (int it = 0; it < kIter; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (K == EXP) x[i] = __builtin_amdgcn_exp2f(x[i]);
        if constexpr (K == FMA) x[i] = __builtin_fmaf(x[i], y, z);
        if constexpr (K == ADD) x[i] = x[i] + y;
        if constexpr (K == CVT_I2F) x[i] = (float)xi[i];
        if constexpr (K == CVT_PK_F16) x[i] = __builtin_bit_cast(float, __builtin_convertvector((v2f{x[i], y}), v2h));
        if constexpr (K == MAX3) xi[i] = max(max(xi[i], __float_as_int(y)), __float_as_int(z));
        asm volatile("" : "+v"(x[i]), "+v"(xi[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i] + (float)xi[i];
  } else {
    v16i ia[4];
    v16f fa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ia[j][i] = 0;
        fa[j][i] = 0.f;
      }
    const v4i a4 = {1, 2, 3, (int)seed}, b4 = {4, 5, 6, (int)threadIdx.x};
    v8h ha, hb;
    v8i fa8, fb8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ha[i] = (_Float16)(seed * 1e-3f * i);
      hb[i] = (_Float16)(threadIdx.x * 1e-3f);
      fa8[i] = 0x38383838 + i;
      fb8[i] = 0x30303030 + (int)threadIdx.x;
    }
    for (int it = 0; it < kIter / 4; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (K == MFMA_I8) ia[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, ia[j], 0, 0, 0);
          if constexpr (K == MFMA_F16) fa[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, hb, fa[j], 0, 0, 0);
          if constexpr (K == MFMA_F8)
            fa[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa8, fb8, fa[j], 0, 0, 0, 127, 0, 127);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += fa[j][i] + (float)ia[j][i];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    clk[0] = __builtin_amdgcn_s_memtime() - t0;
    clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

typedef void (*kfn)(float*, float, unsigned long long*);
const kfn kFn[NKIND] = {k_rate<EXP>, k_rate<FMA>, k_rate<ADD>, k_rate<CVT_I2F>, k_rate<CVT_PK_F16>,
                        k_rate<MAX3>, k_rate<MFMA_I8>, k_rate<MFMA_F16>, k_rate<MFMA_F8>};

#define CHECK(x)                                                       \
  do {                                                                 \
    hipError_t e_ = (x);                                               \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int ncu = prop.multiProcessorCount, nsimd = 4 * ncu;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  CHECK(hipMalloc(&out, sizeof(float) * (size_t)ncu * 2 * 1024));
  CHECK(hipMalloc(&clk, 2 * sizeof(unsigned long long)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  printf("{\"device\": \"%s\", \"cus\": %d", prop.gcnArchName, ncu);
  double sclk_mhz = 0.0;
  double kind_mhz[2][NKIND] = {};
  for (int wps : {8, 1}) {  // waves per SIMD: two 1024-thread workgroups per CU, or one 256-thread one
    const int threads = wps == 8 ? 1024 : 256, blocks = wps == 8 ? 2 * ncu : ncu;
    printf(", \"ns_per_wave_instr_per_simd_%dwps\": {", wps);
    for (int k = 0; k < NKIND; ++k) {
      for (int w = 0; w < 2; ++w) kFn[k]<<<blocks, threads>>>(out, 1.0f, clk);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e0));
      const int reps = 5;
      for (int r = 0; r < reps; ++r) kFn[k]<<<blocks, threads>>>(out, 1.0f, clk);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double waves_per_simd = (double)blocks * threads / 64 / nsimd;
      const double instr = waves_per_simd * (double)(k >= MFMA_I8 ? kIter / 4 : kIter) * 16;
      printf("%s\"%s\": %.4f", k ? ", " : "", kName[k], ms / reps * 1e6 / instr);
      unsigned long long c[2];  // the shader clock across the last launch of this probe
      CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
      kind_mhz[wps == 8 ? 0 : 1][k] = c[1] ? 100.0 * (double)c[0] / (double)c[1] : 0.0;
      if (wps == 8 && k == FMA) sclk_mhz = kind_mhz[0][k];
    }
    printf("}");
  }
  for (int i = 0; i < 2; ++i) {
    printf(", \"sclk_mhz_per_probe_%dwps\": {", i == 0 ? 8 : 1);
    for (int k = 0; k < NKIND; ++k) printf("%s\"%s\": %.0f", k ? ", " : "", kName[k], kind_mhz[i][k]);
    printf("}");
  }
  printf(", \"sclk_mhz_during_fma_probe\": %.0f}\n", sclk_mhz);
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return 0;
}
