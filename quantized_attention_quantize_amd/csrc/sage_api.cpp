// sage_api.cpp -- host side of the libsage_mi355x C ABI (include/sage_mi355x.h).
//
// Every entry point validates its arguments on the host first, touching no HIP API, so a bad call
// returns a status with nothing enqueued.  Then it checks (once per device) that the current
// device is gfx950, lays out the caller's workspace and enqueues the kernels on the caller's
// stream.  Nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <atomic>

#include "sage_fp4.h"
#include "sage_launch.h"
#include "sage_mi355x.h"

namespace {

using namespace sage;

constexpr int64_t kChunkTokens = 256;   // column-reduction chunk (matches sage_prep.hip)
constexpr int64_t kTileRows = 256;      // attention workgroup rows == mask tile rows
constexpr int64_t kTileKeys = 64;       // attention key tile
constexpr int64_t kMaxTokens = (int64_t)1 << 30;
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxRange = (int64_t)1 << 31;  // bytes a kernel addresses through one buffer range

std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

sage_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SAGE_ERR_HIP;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? SAGE_OK : SAGE_ERR_UNSUPPORTED;
}

// Shape / dtype / stride checks of one Q, K or V descriptor.
sage_status check_desc(const sage_qkv_desc* t) {
  if (!t || !t->data) return SAGE_ERR_INVALID_ARGUMENT;
  if (t->B <= 0 || t->H <= 0 || t->N <= 0 || t->d <= 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (t->N > kMaxTokens || t->B * t->H > 65535) return SAGE_ERR_INVALID_ARGUMENT;
  if (t->dtype != SAGE_BF16 && t->dtype != SAGE_FP16) return SAGE_ERR_INVALID_ARGUMENT;
  if (t->d != 64 && t->d != 128) return SAGE_ERR_UNSUPPORTED;
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_n < t->d) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned16(t->data) || (t->stride_b % 8) || (t->stride_h % 8) || (t->stride_n % 8))
    return SAGE_ERR_INVALID_ARGUMENT;
  return SAGE_OK;
}

sage_status check_qk(const sage_qk_quant* qk) {
  if (!qk || !qk->q8 || !qk->k8 || !qk->q_scale || !qk->k_scale || !qk->k_mean || !qk->lse_corr)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (qk->B <= 0 || qk->H <= 0 || qk->Hkv <= 0 || qk->Nq <= 0 || qk->Nk <= 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (qk->H % qk->Hkv != 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (qk->Nq > kMaxTokens || qk->Nk > kMaxTokens || qk->B * qk->H > 65535) return SAGE_ERR_INVALID_ARGUMENT;
  if (qk->d != 64 && qk->d != 128) return SAGE_ERR_UNSUPPORTED;
  if (qk->Nq_pad != sage_pad_tokens(qk->Nq) || qk->Nk_pad != sage_pad_tokens(qk->Nk))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned16(qk->q8) || !aligned16(qk->k8)) return SAGE_ERR_INVALID_ARGUMENT;
  if ((qk->k_block_mean == nullptr) != (qk->blk_corr == nullptr)) return SAGE_ERR_INVALID_ARGUMENT;
  // One head's K8 rows, and per_block_mean's score terms, are addressed through 32-bit buffer ranges
  if (qk->Nk_pad * qk->d >= kMaxRange) return SAGE_ERR_UNSUPPORTED;
  if (qk->blk_corr && cdiv(qk->Nk, 64) * qk->Nq * 4 >= kMaxRange) return SAGE_ERR_UNSUPPORTED;
  return SAGE_OK;
}

sage_status hip_status(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

size_t vt_bytes(int64_t B, int64_t H, int64_t Nk, int64_t d, sage_pv_dtype pv) {
  return (size_t)(B * H * d * sage_pad_tokens(Nk)) * (pv == SAGE_PV_FP16 ? 2 : 1);
}
// sage_prepare_v scratch: per-chunk partial maxima of |V| (fp8) or fp64 partial sums (smooth_v)
size_t prep_ws_bytes(int64_t B, int64_t H, int64_t Nk, int64_t d, sage_pv_dtype) {
  return align256((size_t)(B * H * cdiv(Nk, kChunkTokens) * d) * sizeof(double));
}
size_t mask_ws_bytes(int64_t B, int64_t Nq, int64_t Nk, int64_t mask_h) {
  return mask_h > 0 ? align256((size_t)(B * mask_h * cdiv(Nq, kTileRows) * cdiv(Nk, kTileKeys)) * sizeof(int)) : 0;
}

// sage_attn_fwd workspace: [prepared V | fp8 V scale | smooth_v V mean | prepare-V scratch | mask tile states]
struct FwdLayout {
  size_t vt, vscale, vmean, prep, mtiles, total;
};

FwdLayout fwd_layout(int64_t B, int64_t Hv, int64_t Nq, int64_t Nk, int64_t d, sage_pv_dtype pv, int64_t mask_h) {
  FwdLayout L;
  size_t off = 0;
  L.vt = off;
  off += align256(vt_bytes(B, Hv, Nk, d, pv));
  L.vscale = off;
  if (pv == SAGE_PV_FP8_E4M3) off += align256((size_t)(B * Hv * d) * 4);
  L.vmean = off;
  off += align256((size_t)(B * Hv * d) * 4);
  L.prep = off;
  off += prep_ws_bytes(B, Hv, Nk, d, pv);
  L.mtiles = off;
  off += mask_ws_bytes(B, Nq, Nk, mask_h);
  L.total = off;
  return L;
}

PrepVArgs prep_v_args(const sage_qkv_desc* v, void* vt, float* vscale, float* vmax_partial) {
  PrepVArgs a;
  a.v = static_cast<const unsigned short*>(v->data);
  a.v_sb = v->stride_b;
  a.v_sh = v->stride_h;
  a.v_sn = v->stride_n;
  a.vt = vt;
  a.vscale = vscale;
  a.vmax_partial = vmax_partial;
  a.B = v->B;
  a.H = v->H;
  a.Nk = v->N;
  a.d = v->d;
  a.Nk_pad = sage_pad_tokens(v->N);
  a.nchunk = (int)cdiv(v->N, kChunkTokens);
  a.in_fp16 = v->dtype == SAGE_FP16;
  a.cu_k = nullptr;
  a.total_k = 0;
  return a;
}

}  // namespace

extern "C" {

int64_t sage_pad_tokens(int64_t n) { return n <= 0 ? 0 : (n + 127) / 128 * 128; }

}  // extern "C"

namespace {

// Byte offsets of the buffers of a sage_qk_quant inside one allocation (each 256-byte aligned).
struct QuantLayout {
  size_t q8, k8, qs, ks, kmean, corr, kbmean, blk, total;
};

bool quant_layout(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int per_block_mean,
                  QuantLayout* L) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || H % Hkv != 0 || (d != 64 && d != 128)) return false;
  if (Nq > kMaxTokens || Nk > kMaxTokens || B * H > 65535) return false;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L->q8 = take((size_t)(B * H * sage_pad_tokens(Nq) * d));
  L->k8 = take((size_t)(B * Hkv * sage_pad_tokens(Nk) * d));
  L->qs = take((size_t)(B * H * cdiv(Nq, 64)) * 4);
  L->ks = take((size_t)(B * Hkv * cdiv(Nk, 64)) * 4);
  L->kmean = take((size_t)(B * Hkv * d) * 4);
  L->corr = take((size_t)(B * H * Nq) * 4);
  L->kbmean = per_block_mean ? take((size_t)(B * Hkv * cdiv(Nk, 64) * d) * 4) : 0;
  L->blk = per_block_mean ? take((size_t)(B * H * cdiv(Nk, 64) * Nq) * 4) : 0;
  L->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t sage_qk_quant_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int per_block_mean) {
  QuantLayout L;
  return quant_layout(B, H, Hkv, Nq, Nk, d, per_block_mean, &L) ? L.total : 0;
}

sage_status sage_qk_quant_init(void* base, size_t bytes, int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                               int64_t d, int per_block_mean, sage_qk_quant* out) {
  QuantLayout L;
  if (!base || !out || ((uintptr_t)base & 255u) != 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (!quant_layout(B, H, Hkv, Nq, Nk, d, per_block_mean, &L) || bytes < L.total) return SAGE_ERR_INVALID_ARGUMENT;
  char* p = static_cast<char*>(base);
  out->q8 = reinterpret_cast<int8_t*>(p + L.q8);
  out->k8 = reinterpret_cast<int8_t*>(p + L.k8);
  out->q_scale = reinterpret_cast<float*>(p + L.qs);
  out->k_scale = reinterpret_cast<float*>(p + L.ks);
  out->k_mean = reinterpret_cast<float*>(p + L.kmean);
  out->lse_corr = reinterpret_cast<float*>(p + L.corr);
  out->k_block_mean = per_block_mean ? reinterpret_cast<float*>(p + L.kbmean) : nullptr;
  out->blk_corr = per_block_mean ? reinterpret_cast<float*>(p + L.blk) : nullptr;
  out->B = B;
  out->H = H;
  out->Hkv = Hkv;
  out->Nq = Nq;
  out->Nk = Nk;
  out->d = d;
  out->Nq_pad = sage_pad_tokens(Nq);
  out->Nk_pad = sage_pad_tokens(Nk);
  return SAGE_OK;
}

int sage_block_n(sage_pv_dtype pv) {
  (void)pv;
  return (int)kTileKeys;
}

double sage_softmax_tau(sage_pv_dtype pv) { return kSoftmaxTau[pv == SAGE_PV_FP8_E4M3 ? 1 : 0]; }

int sage_rowsum_rounded(sage_pv_dtype pv) { return kRowsumRounded[pv == SAGE_PV_FP8_E4M3 ? 1 : 0]; }

size_t sage_quantize_workspace_bytes(int64_t B, int64_t Hkv, int64_t Nk, int64_t d) {
  if (B <= 0 || Hkv <= 0 || Nk <= 0 || d <= 0) return 0;
  return align256((size_t)(B * Hkv * cdiv(Nk, kChunkTokens) * d) * sizeof(double));
}

}  // extern "C"

namespace {

sage_status validate_quantize(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qk_quant* out,
                              const void* workspace, size_t workspace_bytes) {
  sage_status s;
  if ((s = check_desc(q)) != SAGE_OK) return s;
  if ((s = check_desc(k)) != SAGE_OK) return s;
  if (q->B != k->B || q->d != k->d || q->H % k->H != 0 || q->dtype != k->dtype) return SAGE_ERR_INVALID_ARGUMENT;
  if ((s = check_qk(out)) != SAGE_OK) return s;
  if (out->B != q->B || out->H != q->H || out->Hkv != k->H || out->d != q->d || out->Nq != q->N ||
      out->Nk != k->N)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!workspace) return SAGE_ERR_WORKSPACE;
  if (workspace_bytes < sage_quantize_workspace_bytes(k->B, k->H, k->N, k->d)) return SAGE_ERR_WORKSPACE;
  return check_device();
}

QuantArgs quant_args(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qk_quant* out) {
  QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const unsigned short*>(q->data);
  a.k = static_cast<const unsigned short*>(k->data);
  a.q_sb = q->stride_b;
  a.q_sh = q->stride_h;
  a.q_sn = q->stride_n;
  a.k_sb = k->stride_b;
  a.k_sh = k->stride_h;
  a.k_sn = k->stride_n;
  a.q8 = out->q8;
  a.k8 = out->k8;
  a.qs = out->q_scale;
  a.ks = out->k_scale;
  a.kmean = out->k_mean;
  a.corr = out->lse_corr;
  a.B = q->B;
  a.H = q->H;
  a.Hkv = k->H;
  a.Nq = q->N;
  a.Nk = k->N;
  a.d = q->d;
  a.Nq_pad = out->Nq_pad;
  a.Nk_pad = out->Nk_pad;
  a.nbq = (int)cdiv(a.Nq, 64);
  a.nbk = (int)cdiv(a.Nk, 64);
  a.in_fp16 = q->dtype == SAGE_FP16;
  a.kbmean = out->k_block_mean;
  a.blk_corr = out->blk_corr;
  return a;
}

sage_status enqueue_quantize(const QuantArgs& a, void* workspace, hipStream_t st) {
  sage_status s;
  if ((s = hip_status(launch_kmean(a, static_cast<double*>(workspace), (int)cdiv(a.Nk, kChunkTokens), st))) != SAGE_OK)
    return s;
  if ((s = hip_status(launch_quant(a, st))) != SAGE_OK) return s;
  return a.kbmean ? hip_status(launch_block_corr(a, st)) : SAGE_OK;
}

// Packed variable-length batches: the token counts of the descriptors are the longest sequence,
// the cumulative lengths live on the device, and totals bound the packed buffers.
sage_status check_varlen(const int32_t* cu_q, const int32_t* cu_k, int64_t total_q, int64_t total_k) {
  if (!cu_q || !cu_k) return SAGE_ERR_INVALID_ARGUMENT;
  if (total_q < 0 || total_k < 0 || total_q > (int64_t(1) << 31) || total_k > (int64_t(1) << 31))
    return SAGE_ERR_INVALID_ARGUMENT;
  return SAGE_OK;
}

}  // namespace

extern "C" {

sage_status sage_quantize_qk(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qk_quant* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  sage_status s;
  if ((s = validate_quantize(q, k, out, workspace, workspace_bytes)) != SAGE_OK) return s;
  return enqueue_quantize(quant_args(q, k, out), workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Scratch of the allocation-free quantize entry point: the K-mean fp64 partial sums.  One array per
// GPU, in the library's device code, kept until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the device symbol): it takes the
// device address once per device with hipGetSymbolAddress and uses that.
static __device__ __align__(256) double scratch[SAGE_NOALLOC_SCRATCH_BYTES / sizeof(double)];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the device's first call).
sage_status noalloc_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SAGE_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // the same address if two threads race here
  }
  *ptr = p;
  return SAGE_OK;
}

}  // namespace

extern "C" {

sage_status sage_quantize_qk_noalloc(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qk_quant* out,
                                     void* stream) {
  sage_status s;
  // host validation first, with the scratch array standing in as the workspace size
  if ((s = validate_quantize(q, k, out, reinterpret_cast<void*>(uintptr_t(256)), SAGE_NOALLOC_SCRATCH_BYTES)) !=
      SAGE_OK)
    return s;
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != SAGE_OK) return s;
  // every chunk's partial sums are written before they are read, so nothing needs clearing
  return enqueue_quantize(quant_args(q, k, out), ws, static_cast<hipStream_t>(stream));
}

sage_status sage_quantize_qk_varlen(const sage_qkv_desc* q, const sage_qkv_desc* k, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k,
                                    const sage_qk_quant* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  sage_status s;
  if ((s = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k)) != SAGE_OK) return s;
  if ((s = validate_quantize(q, k, out, workspace, workspace_bytes)) != SAGE_OK) return s;
  QuantArgs a = quant_args(q, k, out);
  a.q_sb = a.k_sb = 0;  // rows are addressed from the cumulative lengths
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return enqueue_quantize(a, workspace, static_cast<hipStream_t>(stream));
}

size_t sage_prepare_v_workspace_bytes(int64_t B, int64_t H, int64_t Nk, int64_t d, sage_pv_dtype pv) {
  if (B <= 0 || H <= 0 || Nk <= 0 || d <= 0) return 0;
  if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8_E4M3) return 0;
  return prep_ws_bytes(B, H, Nk, d, pv);
}

size_t sage_mask_workspace_bytes(int64_t B, int64_t Nq, int64_t Nk, int64_t mask_h) {
  if (B <= 0 || Nq <= 0 || Nk <= 0 || mask_h < 0) return 0;
  return mask_ws_bytes(B, Nq, Nk, mask_h);
}

size_t sage_fwd_workspace_bytes(int64_t B, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, sage_pv_dtype pv,
                                int64_t mask_h) {
  if (B <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || mask_h < 0) return 0;
  if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8_E4M3) return 0;
  return fwd_layout(B, Hkv, Nq, Nk, d, pv, mask_h).total;
}

}  // extern "C"

namespace {

sage_status validate_prepare(const sage_qkv_desc* v, sage_pv_dtype pv, const void* v_t, const float* v_scale,
                             const float* v_mean, const void* workspace, size_t workspace_bytes) {
  sage_status s;
  if ((s = check_desc(v)) != SAGE_OK) return s;
  if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8_E4M3) return SAGE_ERR_UNSUPPORTED;
  if (v_mean && pv != SAGE_PV_FP16) return SAGE_ERR_UNSUPPORTED;  // smooth_v belongs to the FP16 PV path
  if (!v_t || !aligned16(v_t)) return SAGE_ERR_INVALID_ARGUMENT;
  if (pv == SAGE_PV_FP8_E4M3 && !v_scale) return SAGE_ERR_INVALID_ARGUMENT;
  if (pv == SAGE_PV_FP8_E4M3 || v_mean) {
    if (!workspace || workspace_bytes < prep_ws_bytes(v->B, v->H, v->N, v->d, pv)) return SAGE_ERR_WORKSPACE;
  }
  return SAGE_OK;
}

sage_status enqueue_prepare(const sage_qkv_desc* v, sage_pv_dtype pv, void* v_t, float* v_scale, float* v_mean,
                            void* workspace, hipStream_t st, const int32_t* cu_k = nullptr, int64_t total_k = 0) {
  const int pv8 = pv == SAGE_PV_FP8_E4M3;
  PrepVArgs pa = prep_v_args(v, v_t, pv8 ? v_scale : nullptr, pv8 ? static_cast<float*>(workspace) : nullptr);
  pa.vmean = pv8 ? nullptr : v_mean;
  pa.vsum_partial = pa.vmean ? static_cast<double*>(workspace) : nullptr;
  if (cu_k) {  // packed variable-length V
    pa.v_sb = 0;
    pa.cu_k = cu_k;
    pa.total_k = total_k;
  }
  return hip_status(launch_prep_v(pa, pv8, st));
}

struct FwdCommon {
  int64_t mh;
};

sage_status validate_fwd_common(const sage_qk_quant* qk, sage_pv_dtype pv, float sm_scale, const void* mask,
                                sage_mask_dtype mask_dtype, int64_t mask_h,
                                int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_q, void* out,
                                sage_dtype out_dtype, int64_t out_stride_b, int64_t out_stride_h,
                                int64_t out_stride_n, FwdCommon* c) {
  sage_status s;
  if ((s = check_qk(qk)) != SAGE_OK) return s;
  if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8_E4M3) return SAGE_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return SAGE_ERR_INVALID_ARGUMENT;  // <= 0 selects 1/sqrt(d)
  // one head's prepared V is addressed through a 32-bit buffer range
  if (qk->Nk_pad * qk->d * (pv == SAGE_PV_FP16 ? 2 : 1) >= kMaxRange) return SAGE_ERR_UNSUPPORTED;
  if (!out) return SAGE_ERR_INVALID_ARGUMENT;
  if (out_dtype != SAGE_BF16 && out_dtype != SAGE_FP16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID_ARGUMENT;
  if (out_stride_b < 0 || out_stride_h < 0 || out_stride_n < qk->d) return SAGE_ERR_INVALID_ARGUMENT;
  const int64_t oel = out_dtype == SAGE_F32 ? 4 : 8;  // elements per 16 bytes
  if (!aligned16(out) || (out_stride_b % oel) || (out_stride_h % oel) || (out_stride_n % oel))
    return SAGE_ERR_INVALID_ARGUMENT;
  c->mh = 0;
  if (mask) {
    if (mask_dtype != SAGE_MASK_BOOL && mask_dtype != SAGE_MASK_F32) return SAGE_ERR_INVALID_ARGUMENT;
    if (mask_dtype == SAGE_MASK_F32 && qk->blk_corr) return SAGE_ERR_UNSUPPORTED;  // not combined
    if (mask_dtype == SAGE_MASK_F32 && (uintptr_t)mask % 4 != 0) return SAGE_ERR_INVALID_ARGUMENT;
    if (mask_h != 1 && mask_h != qk->H) return SAGE_ERR_INVALID_ARGUMENT;
    // mask_stride_q = 0 broadcasts one row of keys over all queries (a key-padding mask)
    if (mask_stride_b < 0 || mask_stride_h < 0 || (mask_stride_q != 0 && mask_stride_q < qk->Nk))
      return SAGE_ERR_INVALID_ARGUMENT;
    c->mh = mask_h;
  }
  return SAGE_OK;
}

// Mask classification (if any) and the attention kernel, on already prepared V.
sage_status enqueue_attention(const sage_qk_quant* qk, const void* v_t, const float* v_scale, const float* v_mean,
                              sage_pv_dtype pv,
                              const void* mask, sage_mask_dtype mask_dtype, int64_t mh, int64_t mask_stride_b, int64_t mask_stride_h,
                              int64_t mask_stride_q, int causal, float sm_scale, void* out, sage_dtype out_dtype,
                              int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse,
                              int* mtiles, hipStream_t st, const int32_t* cu_q = nullptr,
                              const int32_t* cu_k = nullptr, int64_t total_q = 0, int64_t total_k = 0) {
  sage_status s;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  if (cu_q) {  // packed variable-length batch: output rows and the LSE [H][total_q] follow cu_q
    a.cu_q = cu_q;
    a.cu_k = cu_k;
    a.total_q = total_q;
    a.total_k = total_k;
    a.l_sb = 0;
    a.l_sh = total_q;
  } else {  // LSE [B][H][Nq]
    a.l_sb = qk->H * qk->Nq;
    a.l_sh = qk->Nq;
  }
  a.nQT = (int)cdiv(qk->Nq, kTileRows);
  a.nKT = (int)cdiv(qk->Nk, kTileKeys);
  if (mask) {
    const int f32 = mask_dtype == SAGE_MASK_F32;
    const int64_t esz = f32 ? 4 : 1;  // bytes per mask element
    // every row start (and the base) aligned to `bytes`
    auto rows_aligned = [&](int64_t bytes) {
      const int64_t el = bytes / esz;
      return (uintptr_t)mask % bytes == 0 && mask_stride_b % el == 0 && (mh == 1 || mask_stride_h % el == 0) &&
             mask_stride_q % el == 0;
    };
    MaskTileArgs m;
    m.mask = mask;
    m.f32 = f32;
    m.sb = mask_stride_b;
    m.sh = mask_stride_h;
    m.sq = mask_stride_q;
    m.B = qk->B;
    m.Hm = mh;
    m.Nq = qk->Nq;
    m.Nk = qk->Nk;
    m.nQT = a.nQT;
    m.nKT = a.nKT;
    m.vec16 = rows_aligned(16);
    m.state = mtiles;
    if ((s = hip_status(launch_mask_tiles(m, st))) != SAGE_OK) return s;
    a.mask = mask;
    a.m_sb = mask_stride_b;
    a.m_sh = mask_stride_h;
    a.m_sq = mask_stride_q;
    a.mtiles = mtiles;
    a.Hm = mh;
    a.mask_f32 = f32;
    a.mask_vec4 = rows_aligned(4 * esz);  // 4 elements at a time
  }
  a.q8 = qk->q8;
  a.k8 = qk->k8;
  a.blk_corr = qk->blk_corr;
  a.qs = qk->q_scale;
  a.ks = qk->k_scale;
  a.corr = qk->lse_corr;
  a.vt = v_t;
  a.vscale = pv == SAGE_PV_FP8_E4M3 ? v_scale : nullptr;
  a.vmean = pv == SAGE_PV_FP8_E4M3 ? nullptr : v_mean;
  a.out = out;
  a.out_kind = out_dtype == SAGE_F32 ? 2 : (out_dtype == SAGE_FP16 ? 1 : 0);
  a.o_sb = out_stride_b;
  a.o_sh = out_stride_h;
  a.o_sn = out_stride_n;
  a.lse = lse;
  a.B = qk->B;
  a.H = qk->H;
  a.Hkv = qk->Hkv;
  a.Nq = qk->Nq;
  a.Nk = qk->Nk;
  a.Nq_pad = qk->Nq_pad;
  a.Nk_pad = qk->Nk_pad;
  a.nbq = (int)cdiv(qk->Nq, 64);
  a.nbk = (int)cdiv(qk->Nk, 64);
  a.causal = causal ? 1 : 0;
  a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)qk->d));
  return hip_status(launch_attn(a, (int)qk->d, pv == SAGE_PV_FP8_E4M3, st));
}

}  // namespace

extern "C" {

sage_status sage_prepare_v(const sage_qkv_desc* v, sage_pv_dtype pv, void* v_t, float* v_scale, float* v_mean,
                           void* workspace, size_t workspace_bytes, void* stream) {
  sage_status s;
  if ((s = validate_prepare(v, pv, v_t, v_scale, v_mean, workspace, workspace_bytes)) != SAGE_OK) return s;
  if ((s = check_device()) != SAGE_OK) return s;
  return enqueue_prepare(v, pv, v_t, v_scale, v_mean, workspace, static_cast<hipStream_t>(stream));
}

sage_status sage_attn_fwd(const sage_qk_quant* qk, const sage_qkv_desc* v, const void* mask,
                          sage_mask_dtype mask_dtype, int64_t mask_h,
                          int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_q, int causal,
                          float sm_scale, sage_pv_dtype pv, int smooth_v, void* out, sage_dtype out_dtype,
                          int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  sage_status s;
  FwdCommon c;
  if (smooth_v && pv != SAGE_PV_FP16) return SAGE_ERR_UNSUPPORTED;
  if ((s = validate_fwd_common(qk, pv, sm_scale, mask, mask_dtype, mask_h, mask_stride_b, mask_stride_h, mask_stride_q, out,
                               out_dtype, out_stride_b, out_stride_h, out_stride_n, &c)) != SAGE_OK)
    return s;
  if ((s = check_desc(v)) != SAGE_OK) return s;
  if (v->B != qk->B || v->H != qk->Hkv || v->N != qk->Nk || v->d != qk->d) return SAGE_ERR_INVALID_ARGUMENT;
  if (!workspace) return SAGE_ERR_WORKSPACE;
  const FwdLayout L = fwd_layout(qk->B, qk->Hkv, qk->Nq, qk->Nk, qk->d, pv, c.mh);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  if ((s = check_device()) != SAGE_OK) return s;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* vscale = pv == SAGE_PV_FP8_E4M3 ? reinterpret_cast<float*>(ws + L.vscale) : nullptr;
  float* vmean = smooth_v ? reinterpret_cast<float*>(ws + L.vmean) : nullptr;
  if ((s = enqueue_prepare(v, pv, ws + L.vt, vscale, vmean, ws + L.prep, st)) != SAGE_OK) return s;
  return enqueue_attention(qk, ws + L.vt, vscale, vmean, pv, mask, mask_dtype, c.mh, mask_stride_b, mask_stride_h,
                           mask_stride_q, causal, sm_scale, out, out_dtype, out_stride_b, out_stride_h, out_stride_n, lse,
                           reinterpret_cast<int*>(ws + L.mtiles), st);
}

sage_status sage_attn_fwd_prepared(const sage_qk_quant* qk, const void* v_t, const float* v_scale,
                                   const float* v_mean, sage_pv_dtype pv,
                                   const void* mask, sage_mask_dtype mask_dtype, int64_t mask_h, int64_t mask_stride_b, int64_t mask_stride_h,
                                   int64_t mask_stride_q, int causal, float sm_scale, void* out,
                                   sage_dtype out_dtype, int64_t out_stride_b, int64_t out_stride_h,
                                   int64_t out_stride_n, float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  sage_status s;
  FwdCommon c;
  if ((s = validate_fwd_common(qk, pv, sm_scale, mask, mask_dtype, mask_h, mask_stride_b, mask_stride_h, mask_stride_q, out,
                               out_dtype, out_stride_b, out_stride_h, out_stride_n, &c)) != SAGE_OK)
    return s;
  if (!v_t || !aligned16(v_t)) return SAGE_ERR_INVALID_ARGUMENT;
  if (pv == SAGE_PV_FP8_E4M3 && !v_scale) return SAGE_ERR_INVALID_ARGUMENT;
  if (v_mean && pv != SAGE_PV_FP16) return SAGE_ERR_UNSUPPORTED;
  const size_t need = mask_ws_bytes(qk->B, qk->Nq, qk->Nk, c.mh);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SAGE_ERR_WORKSPACE;
  if ((s = check_device()) != SAGE_OK) return s;
  return enqueue_attention(qk, v_t, v_scale, v_mean, pv, mask, mask_dtype, c.mh, mask_stride_b, mask_stride_h, mask_stride_q,
                           causal, sm_scale, out, out_dtype, out_stride_b, out_stride_h, out_stride_n, lse,
                           static_cast<int*>(workspace), static_cast<hipStream_t>(stream));
}

sage_status sage_attn_fwd_varlen(const sage_qk_quant* qk, const sage_qkv_desc* v, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k, int causal,
                                 float sm_scale, sage_pv_dtype pv, int smooth_v, void* out, sage_dtype out_dtype,
                                 int64_t out_stride_h, int64_t out_stride_n, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  sage_status s;
  FwdCommon c;
  if (smooth_v && pv != SAGE_PV_FP16) return SAGE_ERR_UNSUPPORTED;
  if ((s = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k)) != SAGE_OK) return s;
  if ((s = validate_fwd_common(qk, pv, sm_scale, nullptr, SAGE_MASK_BOOL, 0, 0, 0, 0, out, out_dtype, 0, out_stride_h,
                               out_stride_n, &c)) != SAGE_OK)
    return s;
  if ((s = check_desc(v)) != SAGE_OK) return s;
  if (v->B != qk->B || v->H != qk->Hkv || v->N != qk->Nk || v->d != qk->d) return SAGE_ERR_INVALID_ARGUMENT;
  if (!workspace) return SAGE_ERR_WORKSPACE;
  const FwdLayout L = fwd_layout(qk->B, qk->Hkv, qk->Nq, qk->Nk, qk->d, pv, 0);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  if ((s = check_device()) != SAGE_OK) return s;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* vscale = pv == SAGE_PV_FP8_E4M3 ? reinterpret_cast<float*>(ws + L.vscale) : nullptr;
  float* vmean = smooth_v ? reinterpret_cast<float*>(ws + L.vmean) : nullptr;
  if ((s = enqueue_prepare(v, pv, ws + L.vt, vscale, vmean, ws + L.prep, st, cu_seqlens_k, total_k)) != SAGE_OK)
    return s;
  return enqueue_attention(qk, ws + L.vt, vscale, vmean, pv, nullptr, SAGE_MASK_BOOL, 0, 0, 0, 0, causal, sm_scale, out,
                           out_dtype, 0, out_stride_h, out_stride_n, lse, nullptr, st, cu_seqlens_q, cu_seqlens_k,
                           total_q, total_k);
}

sage_status sage_prepare_v_varlen(const sage_qkv_desc* v, const int32_t* cu_seqlens_k, int64_t total_k,
                                  sage_pv_dtype pv, void* v_t, float* v_scale, float* v_mean, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  sage_status s;
  if ((s = check_varlen(cu_seqlens_k, cu_seqlens_k, 0, total_k)) != SAGE_OK) return s;
  if ((s = validate_prepare(v, pv, v_t, v_scale, v_mean, workspace, workspace_bytes)) != SAGE_OK) return s;
  if ((s = check_device()) != SAGE_OK) return s;
  return enqueue_prepare(v, pv, v_t, v_scale, v_mean, workspace, static_cast<hipStream_t>(stream), cu_seqlens_k,
                         total_k);
}

sage_status sage_attn_fwd_prepared_varlen(const sage_qk_quant* qk, const void* v_t, const float* v_scale,
                                          const float* v_mean, sage_pv_dtype pv, const int32_t* cu_seqlens_q,
                                          const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k,
                                          int causal, float sm_scale, void* out, sage_dtype out_dtype,
                                          int64_t out_stride_h, int64_t out_stride_n, float* lse, void* stream) {
  sage_status s;
  FwdCommon c;
  if ((s = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k)) != SAGE_OK) return s;
  if ((s = validate_fwd_common(qk, pv, sm_scale, nullptr, SAGE_MASK_BOOL, 0, 0, 0, 0, out, out_dtype, 0, out_stride_h,
                               out_stride_n, &c)) != SAGE_OK)
    return s;
  if (!v_t || !aligned16(v_t)) return SAGE_ERR_INVALID_ARGUMENT;
  if (pv == SAGE_PV_FP8_E4M3 && !v_scale) return SAGE_ERR_INVALID_ARGUMENT;
  if (v_mean && pv != SAGE_PV_FP16) return SAGE_ERR_UNSUPPORTED;
  if ((s = check_device()) != SAGE_OK) return s;
  return enqueue_attention(qk, v_t, v_scale, v_mean, pv, nullptr, SAGE_MASK_BOOL, 0, 0, 0, 0, causal, sm_scale, out,
                           out_dtype, 0, out_stride_h, out_stride_n, lse, nullptr, static_cast<hipStream_t>(stream),
                           cu_seqlens_q, cu_seqlens_k, total_q, total_k);
}

sage_status sage_merge_lse(int64_t S, int64_t B, int64_t H, int64_t Nq, int64_t d, const void* o_parts,
                           sage_dtype part_dtype, const float* lse_parts, void* out, sage_dtype out_dtype,
                           int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse,
                           void* stream) {
  if (S <= 0 || B <= 0 || H <= 0 || Nq <= 0 || d <= 0 || d % 8 != 0 || d > 1024) return SAGE_ERR_INVALID_ARGUMENT;
  if (B * H > 65535 || Nq > kMaxTokens || S > 4096) return SAGE_ERR_INVALID_ARGUMENT;
  auto dtype_ok = [](sage_dtype t) { return t == SAGE_BF16 || t == SAGE_FP16 || t == SAGE_F32; };
  if (!dtype_ok(part_dtype) || !dtype_ok(out_dtype)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!o_parts || !lse_parts || !out || !aligned16(o_parts) || !aligned16(out)) return SAGE_ERR_INVALID_ARGUMENT;
  if (out_stride_b < 0 || out_stride_h < 0 || out_stride_n < d) return SAGE_ERR_INVALID_ARGUMENT;
  const int64_t oel = out_dtype == SAGE_F32 ? 4 : 8;  // elements per 16 bytes
  if ((out_stride_b % oel) || (out_stride_h % oel) || (out_stride_n % oel)) return SAGE_ERR_INVALID_ARGUMENT;
  sage_status s;
  if ((s = check_device()) != SAGE_OK) return s;
  MergeArgs a;
  a.parts = o_parts;
  a.lse_parts = lse_parts;
  a.S = S;
  a.R = B * H * Nq;
  a.d = d;
  a.H = H;
  a.Nq = Nq;
  a.out = out;
  a.o_sb = out_stride_b;
  a.o_sh = out_stride_h;
  a.o_sn = out_stride_n;
  a.out_kind = out_dtype == SAGE_F32 ? 2 : (out_dtype == SAGE_FP16 ? 1 : 0);
  a.part_kind = part_dtype == SAGE_F32 ? 2 : (part_dtype == SAGE_FP16 ? 1 : 0);
  a.lse = lse;
  return hip_status(launch_merge(a, static_cast<hipStream_t>(stream)));
}

sage_status sage_debug_qk_int32(const sage_qk_quant* qk, int64_t b, int64_t h, int64_t row0, int64_t nrows,
                                int64_t col0, int64_t ncols, int32_t* out, void* stream) {
  sage_status s;
  if ((s = check_qk(qk)) != SAGE_OK) return s;
  if (!out) return SAGE_ERR_INVALID_ARGUMENT;
  if (b < 0 || b >= qk->B || h < 0 || h >= qk->H) return SAGE_ERR_INVALID_ARGUMENT;
  if (row0 < 0 || nrows <= 0 || row0 + nrows > qk->Nq_pad) return SAGE_ERR_INVALID_ARGUMENT;
  if (col0 < 0 || ncols <= 0 || col0 + ncols > qk->Nk_pad) return SAGE_ERR_INVALID_ARGUMENT;
  if ((s = check_device()) != SAGE_OK) return s;
  DebugQKArgs a;
  const int64_t bh = b * qk->H + h, bhk = b * qk->Hkv + h / (qk->H / qk->Hkv);
  a.q8h = qk->q8 + bh * qk->Nq_pad * qk->d;
  a.k8h = qk->k8 + bhk * qk->Nk_pad * qk->d;
  a.Nk_pad = qk->Nk_pad;
  a.row0 = row0;
  a.nrows = nrows;
  a.col0 = col0;
  a.ncols = ncols;
  a.out = out;
  return hip_status(launch_debug_qk(a, (int)qk->d, qk->Nq_pad, static_cast<hipStream_t>(stream)));
}

sage_status sage_sclk_probe(int64_t nblocks, int64_t iters, int load, unsigned long long* out, void* stream) {
  if (nblocks < 1 || nblocks > 65536 || iters < 1 || iters > ((int64_t)1 << 24)) return SAGE_ERR_INVALID_ARGUMENT;
  if ((load != 0 && load != 1) || !out || ((uintptr_t)out & 7u)) return SAGE_ERR_INVALID_ARGUMENT;
  sage_status s;
  if ((s = check_device()) != SAGE_OK) return s;
  return hip_status(launch_sclk_probe(out, (int)nblocks, (int)iters, load, static_cast<hipStream_t>(stream)));
}

const char* sage_status_string(sage_status s) {
  switch (s) {
    case SAGE_OK:
      return "ok";
    case SAGE_ERR_INVALID_ARGUMENT:
      return "invalid argument";
    case SAGE_ERR_UNSUPPORTED:
      return "unsupported (head_dim, dtype, pv dtype or device)";
    case SAGE_ERR_WORKSPACE:
      return "workspace missing or too small";
    case SAGE_ERR_HIP:
      return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// FP4 microscaling method (include/sage_fp4.h)
// ---------------------------------------------------------------------------------------------
namespace {

constexpr int64_t kMaxFp4Tokens = (int64_t)1 << 24;

int64_t fp4_q_blocks(int64_t Nq, int per_block) { return per_block ? cdiv(Nq, 128) : 1; }

sage_status check_fp4_qkv(const sage_fp4_qkv* x) {
  if (!x || !x->q4 || !x->q_scale || !x->k4 || !x->k_scale || !x->v4t || !x->v_scale || !x->k_mean || !x->q_mean ||
      !x->qk_corr || !x->lse_corr)
    return SAGE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x->q4, x->q_scale, x->k4, x->k_scale, x->v4t, x->v_scale, x->k_mean, x->q_mean, x->qk_corr,
                        x->lse_corr};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SAGE_ERR_INVALID_ARGUMENT;
  if (x->B <= 0 || x->H <= 0 || x->Hkv <= 0 || x->Nq <= 0 || x->Nk <= 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (x->H % x->Hkv != 0 || x->B * x->H > 65535) return SAGE_ERR_INVALID_ARGUMENT;
  if (x->per_block_mean != 0 && x->per_block_mean != 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (x->d != 128) return SAGE_ERR_UNSUPPORTED;
  if (x->Nq > kMaxFp4Tokens || x->Nk > kMaxFp4Tokens) return SAGE_ERR_UNSUPPORTED;
  if (x->Nq_pad != sage_pad_tokens(x->Nq) || x->Nk_pad != sage_pad_tokens(x->Nk)) return SAGE_ERR_INVALID_ARGUMENT;
  if (fp4_q_blocks(x->Nq, x->per_block_mean) * x->Nk_pad * 4 >= ((int64_t)1 << 31)) return SAGE_ERR_UNSUPPORTED;
  return SAGE_OK;
}

Fp4AttnArgs fp4_attn_args(const sage_fp4_qkv* x) {
  Fp4AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q4 = x->q4;
  a.q_sc = x->q_scale;
  a.k4 = x->k4;
  a.k_sc = x->k_scale;
  a.v4t = x->v4t;
  a.v_sc = x->v_scale;
  a.qk_corr = x->qk_corr;
  a.lse_corr = x->lse_corr;
  a.B = x->B;
  a.H = x->H;
  a.Hkv = x->Hkv;
  a.Nq = x->Nq;
  a.Nk = x->Nk;
  a.Nq_pad = x->Nq_pad;
  a.Nk_pad = x->Nk_pad;
  a.nqm = (int)fp4_q_blocks(x->Nq, x->per_block_mean);
  a.per_block = x->per_block_mean;
  a.nQT = (int)cdiv(x->Nq, kTileRows);
  a.sm_scale = (float)(1.0 / sqrt((double)x->d));
  return a;
}

}  // namespace

extern "C" {

int64_t sage_fp4_q_blocks(int64_t Nq, int per_block_mean) { return Nq <= 0 ? 0 : fp4_q_blocks(Nq, per_block_mean); }

double sage_fp4_softmax_tau(void) { return (double)fp4_softmax_tau(); }

size_t sage_fp4_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  return align256((size_t)fp4_mean_partial_doubles(B, H, Hkv, Nq, Nk, d) * sizeof(double));
}

sage_status sage_fp4_quantize_qkv(const sage_qkv_desc* q, const sage_qkv_desc* k, const sage_qkv_desc* v,
                                  const sage_fp4_qkv* out, void* workspace, size_t workspace_bytes, void* stream) {
  sage_status s;
  if ((s = check_desc(q)) != SAGE_OK) return s;
  if ((s = check_desc(k)) != SAGE_OK) return s;
  if ((s = check_desc(v)) != SAGE_OK) return s;
  if (q->B != k->B || k->B != v->B || q->d != k->d || k->d != v->d || k->H != v->H || k->N != v->N ||
      q->H % k->H != 0 || q->dtype != k->dtype || k->dtype != v->dtype)
    return SAGE_ERR_INVALID_ARGUMENT;
  if ((s = check_fp4_qkv(out)) != SAGE_OK) return s;
  if (out->B != q->B || out->H != q->H || out->Hkv != k->H || out->d != q->d || out->Nq != q->N || out->Nk != k->N)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < sage_fp4_workspace_bytes(q->B, q->H, k->H, q->N, k->N, q->d))
    return SAGE_ERR_WORKSPACE;
  if ((s = check_device()) != SAGE_OK) return s;
  Fp4QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const unsigned short*>(q->data);
  a.k = static_cast<const unsigned short*>(k->data);
  a.v = static_cast<const unsigned short*>(v->data);
  a.q_sb = q->stride_b;
  a.q_sh = q->stride_h;
  a.q_sn = q->stride_n;
  a.k_sb = k->stride_b;
  a.k_sh = k->stride_h;
  a.k_sn = k->stride_n;
  a.v_sb = v->stride_b;
  a.v_sh = v->stride_h;
  a.v_sn = v->stride_n;
  a.q4 = out->q4;
  a.q_sc = out->q_scale;
  a.k4 = out->k4;
  a.k_sc = out->k_scale;
  a.v4t = out->v4t;
  a.v_sc = out->v_scale;
  a.k_mean = out->k_mean;
  a.q_mean = out->q_mean;
  a.qk_corr = out->qk_corr;
  a.lse_corr = out->lse_corr;
  a.B = q->B;
  a.H = q->H;
  a.Hkv = k->H;
  a.Nq = q->N;
  a.Nk = k->N;
  a.d = q->d;
  a.Nq_pad = out->Nq_pad;
  a.Nk_pad = out->Nk_pad;
  a.nqm = (int)fp4_q_blocks(q->N, out->per_block_mean);
  a.per_block = out->per_block_mean;
  a.in_fp16 = q->dtype == SAGE_FP16;
  return hip_status(launch_fp4_quant(a, static_cast<double*>(workspace), static_cast<hipStream_t>(stream)));
}

sage_status sage_fp4_attn_fwd(const sage_fp4_qkv* qkv, int causal, float sm_scale, void* out, sage_dtype out_dtype,
                              int64_t out_stride_b, int64_t out_stride_h, int64_t out_stride_n, float* lse,
                              void* stream) {
  sage_status s;
  if ((s = check_fp4_qkv(qkv)) != SAGE_OK) return s;
  if (!out) return SAGE_ERR_INVALID_ARGUMENT;
  if (out_dtype != SAGE_BF16 && out_dtype != SAGE_FP16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID_ARGUMENT;
  if (out_stride_b < 0 || out_stride_h < 0 || out_stride_n < qkv->d) return SAGE_ERR_INVALID_ARGUMENT;
  const int64_t oel = out_dtype == SAGE_F32 ? 4 : 8;  // elements per 16 bytes
  if (!aligned16(out) || (out_stride_b % oel) || (out_stride_h % oel) || (out_stride_n % oel))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!isfinite(sm_scale)) return SAGE_ERR_INVALID_ARGUMENT;  // <= 0 selects 1/sqrt(d)
  if ((s = check_device()) != SAGE_OK) return s;
  Fp4AttnArgs a = fp4_attn_args(qkv);
  a.out = out;
  a.out_kind = out_dtype == SAGE_F32 ? 2 : (out_dtype == SAGE_FP16 ? 1 : 0);
  a.o_sb = out_stride_b;
  a.o_sh = out_stride_h;
  a.o_sn = out_stride_n;
  a.lse = lse;
  a.causal = causal ? 1 : 0;
  if (sm_scale > 0.f) a.sm_scale = sm_scale;
  return hip_status(launch_fp4_attn(a, static_cast<hipStream_t>(stream)));
}

sage_status sage_fp4_debug_scores(const sage_fp4_qkv* qkv, int64_t b, int64_t h, int64_t row0, int64_t nrows,
                                  int64_t col0, int64_t ncols, float* out, void* stream) {
  sage_status s;
  if ((s = check_fp4_qkv(qkv)) != SAGE_OK) return s;
  if (!out) return SAGE_ERR_INVALID_ARGUMENT;
  if (b < 0 || b >= qkv->B || h < 0 || h >= qkv->H) return SAGE_ERR_INVALID_ARGUMENT;
  if (row0 < 0 || nrows <= 0 || row0 + nrows > qkv->Nq_pad) return SAGE_ERR_INVALID_ARGUMENT;
  if (col0 < 0 || ncols <= 0 || col0 + ncols > qkv->Nk_pad) return SAGE_ERR_INVALID_ARGUMENT;
  if ((s = check_device()) != SAGE_OK) return s;
  Fp4DebugArgs d;
  d.a = fp4_attn_args(qkv);
  d.b = b;
  d.h = h;
  d.row0 = row0;
  d.nrows = nrows;
  d.col0 = col0;
  d.ncols = ncols;
  d.out = out;
  return hip_status(launch_fp4_debug(d, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
