// C ABI entry points of libsvdq: argument validation, device check, and
// dispatch to the kernels.  Every argument is validated on the host before
// any HIP call; nothing throws across the boundary.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "svdq_internal.h"
#include "svdq_kernels.h"
#include "svdq_prep.h"

using namespace svdq;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

svdq_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int known = g_device_ok[dev].load(std::memory_order_relaxed);
    if (known == 1) return SVDQ_OK;
    if (known == 2) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

svdq_status from_hip(hipError_t e) { return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP; }

// Common validation of the runtime calls.
svdq_status validate_runtime(const svdq_layer_desc* desc, const void* prepared, const void* X, int M) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if ((st = validate_m(M)) != SVDQ_OK) return st;
  if (!prepared || !X) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(prepared) || !aligned16(X)) return SVDQ_ERR_MISALIGNED;
  return SVDQ_OK;
}

struct BlobPtrs {
  const float* inv_lam;
  const uint16_t* l1t;
  const uint16_t* l2t;
  const uint8_t* wcodes;
  const void* wscales;
  const float* bias;
};

BlobPtrs blob_ptrs(const svdq_layer_desc& d, const void* prepared) {
  const svdq_blob_layout L = layout_of(d);
  const uint8_t* b = static_cast<const uint8_t*>(prepared);
  BlobPtrs p;
  p.inv_lam = reinterpret_cast<const float*>(b + L.inv_lambda);
  p.l1t = reinterpret_cast<const uint16_t*>(b + L.l1t);
  p.l2t = reinterpret_cast<const uint16_t*>(b + L.l2t);
  p.wcodes = b + L.wcodes;
  p.wscales = b + L.wscales;
  p.bias = (d.flags & SVDQ_F_HAS_BIAS) ? reinterpret_cast<const float*>(b + L.bias) : nullptr;
  return p;
}

// LayerNorm of the norm-fused pass (gamma == nullptr: none).
struct NormArgs {
  const void* gamma = nullptr;
  const void* beta = nullptr;
  float eps = 0.f;
};

bool norm_ok(const NormArgs& n) { return n.gamma && n.eps > 0.f && n.eps < 3.0e38f; }

// The norm-fused pass's statistics and folded affine into the workspace;
// points the activation arguments at them.
svdq_status setup_norm(const svdq_layer_desc& d, const NormArgs& n, const void* X, int M, uint8_t* w,
                       const ActLayout& A, ActArgs& a, hipStream_t s) {
  float* rowstat = reinterpret_cast<float*>(w + A.rowstat);
  float* fold = reinterpret_cast<float*>(w + A.fold);
  svdq_status st = from_hip(launch_norm_stats(static_cast<const uint16_t*>(X), M, d.K, n.eps,
                                              static_cast<const uint16_t*>(n.gamma),
                                              static_cast<const uint16_t*>(n.beta), a.inv_lam, rowstat, fold, s));
  a.rowstat = rowstat;
  a.inv_lam = fold;
  return st;
}

svdq_status run_layer(const svdq_layer_desc* desc, const void* prepared, const void* X, int M, void* Y,
                      int out_dtype, void* ws, size_t ws_bytes, void* stream, bool unfused,
                      const NormArgs& norm = NormArgs()) {
  svdq_status st = validate_runtime(desc, prepared, X, M);
  if (st != SVDQ_OK) return st;
  if (!Y || !ws) return SVDQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(Y) || !aligned16(ws)) return SVDQ_ERR_MISALIGNED;
  const ActLayout A = act_layout(*desc, M);
  if (ws_bytes < A.required) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;

  const BlobPtrs bp = blob_ptrs(*desc, prepared);
  uint8_t* w = static_cast<uint8_t*>(ws);
  ActArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.M = M;
  a.K = desc->K;
  a.rank = desc->rank;
  a.inv_lam = bp.inv_lam;
  a.l1t = bp.l1t;
  a.codes = w + A.codes;
  a.scales = w + A.scales;
  a.Tb = reinterpret_cast<uint16_t*>(w + A.tb);
  a.tpart = reinterpret_cast<float*>(w + A.tpart);
  const hipStream_t s = as_stream(stream);
  if (norm.gamma && (st = setup_norm(*desc, norm, X, M, w, A, a, s)) != SVDQ_OK) return st;

  GemmArgs g{};
  g.acodes = a.codes;
  g.ascales = a.scales;
  g.wcodes = bp.wcodes;
  g.wscales = bp.wscales;
  g.Tb = a.Tb;
  g.l2t = bp.l2t;
  g.bias = bp.bias;
  g.Y = Y;
  g.M = M;
  g.K = desc->K;
  g.N = desc->N;
  g.rank = desc->rank;
  // the split-K GEMM's partial tiles, where the workspace holds them
  g.ypart = gemm_may_split(*desc, M) && ws_bytes >= A.total ? reinterpret_cast<float*>(w + A.ypart) : nullptr;

  if (!unfused) {
    if ((st = from_hip(launch_act(desc->fmt, true, desc->rank > 0, a, s))) != SVDQ_OK) return st;
    return from_hip(launch_gemm(desc->fmt, desc->rank > 0, out_dtype, g, s));
  }
  if ((st = from_hip(launch_act(desc->fmt, true, false, a, s))) != SVDQ_OK) return st;
  if (desc->rank > 0 && (st = from_hip(launch_act(desc->fmt, false, true, a, s))) != SVDQ_OK) return st;
  if ((st = from_hip(launch_gemm(desc->fmt, false, out_dtype, g, s))) != SVDQ_OK) return st;
  return from_hip(launch_up(out_dtype, a.Tb, bp.l2t, Y, M, desc->N, desc->rank, s));
}

// Scratch of svdq_linear_noalloc: the fused layer's workspace (activation
// codes, scales, Tb, partial down-projections) for callers that cannot
// allocate.  One copy per device (the code object's global), zero at load.
// Host code never passes this name to a kernel: it stands for a host-side
// shadow, not the device address; scratch_ptr() returns the device address.
static __device__ __align__(256) uint8_t scratch[SVDQ_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

svdq_status svdq_act_absmax(const void* d_X, int M, int K, float* d_absmax, int accumulate, void* stream) {
  if (!d_X || !d_absmax) return SVDQ_ERR_INVALID_ARGUMENT;
  if (validate_m(M) != SVDQ_OK || K < 1 || K > kMaxDim) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  svdq_status st = check_device();
  if (st != SVDQ_OK) return st;
  return from_hip(launch_absmax(static_cast<const uint16_t*>(d_X), M, K, d_absmax, accumulate != 0,
                                as_stream(stream)));
}

svdq_status svdq_prepare_weights(const svdq_layer_desc* desc, const void* d_W, const float* d_act_absmax,
                                 const void* d_bias, const void* d_L1, const void* d_L2, void* d_prepared,
                                 size_t prepared_bytes, void* stream) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if (!d_W || !d_prepared) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!(desc->flags & SVDQ_F_NO_SMOOTHING) && !d_act_absmax) return SVDQ_ERR_INVALID_ARGUMENT;
  if ((desc->flags & SVDQ_F_HAS_BIAS) && !d_bias) return SVDQ_ERR_INVALID_ARGUMENT;
  if ((desc->flags & SVDQ_F_FACTORS_GIVEN) && desc->rank > 0 && (!d_L1 || !d_L2)) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_prepared) || !aligned16(d_W)) return SVDQ_ERR_MISALIGNED;
  if (prepared_bytes < layout_of(*desc).total) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  PrepOptions opt;
  if (const char* e = std::getenv("SVDQ_PREP_ITERS")) opt.iterations = std::atoi(e);
  return prepare_impl(*desc, static_cast<const uint16_t*>(d_W), d_act_absmax, static_cast<const uint16_t*>(d_bias),
                      static_cast<const uint16_t*>(d_L1), static_cast<const uint16_t*>(d_L2),
                      static_cast<uint8_t*>(d_prepared), as_stream(stream), opt);
}

svdq_status svdq_prepare_weights_gptq(const svdq_layer_desc* desc, const void* d_W, const float* d_act_absmax,
                                      const void* d_bias, const void* d_L1, const void* d_L2, const void* d_Xcal,
                                      int M_cal, float damp, void* d_prepared, size_t prepared_bytes, void* stream) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if (!d_W || !d_prepared || !d_Xcal) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!(damp >= 0.f && damp < 3.0e38f)) return SVDQ_ERR_INVALID_ARGUMENT;
  if ((st = validate_m(M_cal)) != SVDQ_OK) return st;
  if (!(desc->flags & SVDQ_F_NO_SMOOTHING) && !d_act_absmax) return SVDQ_ERR_INVALID_ARGUMENT;
  if ((desc->flags & SVDQ_F_HAS_BIAS) && !d_bias) return SVDQ_ERR_INVALID_ARGUMENT;
  if ((desc->flags & SVDQ_F_FACTORS_GIVEN) && desc->rank > 0 && (!d_L1 || !d_L2)) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_prepared) || !aligned16(d_W)) return SVDQ_ERR_MISALIGNED;
  if (prepared_bytes < layout_of(*desc).total) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  PrepOptions opt;
  if (const char* e = std::getenv("SVDQ_PREP_ITERS")) opt.iterations = std::atoi(e);
  GptqArgs gq;
  gq.X = static_cast<const uint16_t*>(d_Xcal);
  gq.M = M_cal;
  gq.damp = damp;
  return prepare_impl(*desc, static_cast<const uint16_t*>(d_W), d_act_absmax, static_cast<const uint16_t*>(d_bias),
                      static_cast<const uint16_t*>(d_L1), static_cast<const uint16_t*>(d_L2),
                      static_cast<uint8_t*>(d_prepared), as_stream(stream), opt, &gq);
}

svdq_status svdq_merge_lowrank(const svdq_layer_desc* desc, const void* d_prepared, const void* d_A, const void* d_B,
                               int r_extra, void* d_out, size_t out_bytes, void* stream) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if (r_extra <= 0 || r_extra % 16 != 0 || desc->rank + r_extra > kMaxRank) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!d_prepared || !d_A || !d_B || !d_out) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_prepared) || !aligned16(d_out)) return SVDQ_ERR_MISALIGNED;
  svdq_layer_desc dn = *desc;
  dn.rank += r_extra;
  const svdq_blob_layout L = layout_of(dn);
  if (out_bytes < L.total) return SVDQ_ERR_BUFFER_TOO_SMALL;
  const uint8_t* in = static_cast<const uint8_t*>(d_prepared);
  const uint8_t* out = static_cast<const uint8_t*>(d_out);
  const uint64_t in_bytes = layout_of(*desc).total;
  if (out < in + in_bytes && in < out + L.total) return SVDQ_ERR_INVALID_ARGUMENT;   // overlap
  if ((st = check_device()) != SVDQ_OK) return st;
  return merge_impl(*desc, in, static_cast<const uint16_t*>(d_A), static_cast<const uint16_t*>(d_B), r_extra,
                    static_cast<uint8_t*>(d_out), as_stream(stream));
}

svdq_status svdq_check_blob(const svdq_layer_desc* desc, const void* d_prepared, void* stream) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if (!d_prepared) return SVDQ_ERR_INVALID_ARGUMENT;
  if ((st = check_device()) != SVDQ_OK) return st;
  BlobHeader h;
  if (hipMemcpyAsync(&h, d_prepared, sizeof(h), hipMemcpyDeviceToHost, as_stream(stream)) != hipSuccess ||
      hipStreamSynchronize(as_stream(stream)) != hipSuccess)
    return SVDQ_ERR_HIP;
  if (h.magic != kMagic || h.version != kVersion || h.fmt != desc->fmt || h.K != desc->K || h.N != desc->N ||
      h.rank != desc->rank || h.flags != desc->flags)
    return SVDQ_ERR_BAD_BLOB;
  return SVDQ_OK;
}

svdq_status svdq_quantize_act(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, int M,
                              void* d_codes, void* d_scales, void* d_T, void* d_workspace, size_t ws_bytes,
                              void* stream) {
  svdq_status st = validate_runtime(desc, d_prepared, d_X, M);
  if (st != SVDQ_OK) return st;
  if (!d_codes || !d_scales || (desc->rank > 0 && !d_T)) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_codes) || !aligned16(d_scales) || (d_T && !aligned16(d_T))) return SVDQ_ERR_MISALIGNED;
  if (d_workspace && !aligned16(d_workspace)) return SVDQ_ERR_MISALIGNED;
  if (d_workspace && ws_bytes < act_layout(*desc, M).required) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  const BlobPtrs bp = blob_ptrs(*desc, d_prepared);
  ActArgs a;
  a.X = static_cast<const uint16_t*>(d_X);
  a.M = M;
  a.K = desc->K;
  a.rank = desc->rank;
  a.inv_lam = bp.inv_lam;
  a.l1t = bp.l1t;
  a.codes = static_cast<uint8_t*>(d_codes);
  a.scales = d_scales;
  a.Tb = static_cast<uint16_t*>(d_T);
  // the workspace's partial-T section (if any) lets the pass split K
  a.tpart = d_workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(d_workspace) + act_layout(*desc, M).tpart)
                        : nullptr;
  return from_hip(launch_act(desc->fmt, true, desc->rank > 0, a, as_stream(stream)));
}

svdq_status svdq_gemm(const svdq_layer_desc* desc, const void* d_prepared, const void* d_codes,
                      const void* d_scales, const void* d_T, int M, void* d_Y, int out_dtype, void* d_workspace,
                      size_t ws_bytes, void* stream) {
  svdq_status st = validate_runtime(desc, d_prepared, d_codes, M);
  if (st != SVDQ_OK) return st;
  if (!d_scales || !d_Y || (desc->rank > 0 && !d_T)) return SVDQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_scales) || !aligned16(d_Y) || (d_T && !aligned16(d_T))) return SVDQ_ERR_MISALIGNED;
  const ActLayout A = act_layout(*desc, M);
  if (d_workspace && !aligned16(d_workspace)) return SVDQ_ERR_MISALIGNED;
  if (d_workspace && ws_bytes < A.required) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  const BlobPtrs bp = blob_ptrs(*desc, d_prepared);
  GemmArgs g{};
  g.acodes = static_cast<const uint8_t*>(d_codes);
  g.ascales = d_scales;
  g.wcodes = bp.wcodes;
  g.wscales = bp.wscales;
  g.Tb = static_cast<const uint16_t*>(d_T);
  g.l2t = bp.l2t;
  g.bias = bp.bias;
  g.Y = d_Y;
  g.M = M;
  g.K = desc->K;
  g.N = desc->N;
  g.rank = desc->rank;
  g.ypart = d_workspace && gemm_may_split(*desc, M) && ws_bytes >= A.total
                ? reinterpret_cast<float*>(static_cast<uint8_t*>(d_workspace) + A.ypart)
                : nullptr;
  return from_hip(launch_gemm(desc->fmt, desc->rank > 0, out_dtype, g, as_stream(stream)));
}

svdq_status svdq_quantize_act_ln(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X,
                                 const void* d_gamma, const void* d_beta, float eps, int M, void* d_codes,
                                 void* d_scales, void* d_T, void* d_workspace, size_t ws_bytes, void* stream) {
  svdq_status st = validate_runtime(desc, d_prepared, d_X, M);
  if (st != SVDQ_OK) return st;
  NormArgs n;
  n.gamma = d_gamma;
  n.beta = d_beta;
  n.eps = eps;
  if (!norm_ok(n) || !d_codes || !d_scales || !d_workspace || (desc->rank > 0 && !d_T)) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_codes) || !aligned16(d_scales) || !aligned16(d_workspace) || (d_T && !aligned16(d_T)))
    return SVDQ_ERR_MISALIGNED;
  const ActLayout A = act_layout(*desc, M);
  if (ws_bytes < A.required) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  const BlobPtrs bp = blob_ptrs(*desc, d_prepared);
  uint8_t* w = static_cast<uint8_t*>(d_workspace);
  ActArgs a;
  a.X = static_cast<const uint16_t*>(d_X);
  a.M = M;
  a.K = desc->K;
  a.rank = desc->rank;
  a.inv_lam = bp.inv_lam;
  a.l1t = bp.l1t;
  a.codes = static_cast<uint8_t*>(d_codes);
  a.scales = d_scales;
  a.Tb = static_cast<uint16_t*>(d_T);
  a.tpart = reinterpret_cast<float*>(w + A.tpart);
  const hipStream_t s = as_stream(stream);
  if ((st = setup_norm(*desc, n, d_X, M, w, A, a, s)) != SVDQ_OK) return st;
  return from_hip(launch_act(desc->fmt, true, desc->rank > 0, a, s));
}

svdq_status svdq_linear_ln(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, const void* d_gamma,
                           const void* d_beta, float eps, int M, void* d_Y, int out_dtype, void* d_workspace,
                           size_t ws_bytes, void* stream) {
  NormArgs n;
  n.gamma = d_gamma;
  n.beta = d_beta;
  n.eps = eps;
  svdq_status st = validate_runtime(desc, d_prepared, d_X, M);
  if (st != SVDQ_OK) return st;
  if (!norm_ok(n)) return SVDQ_ERR_INVALID_ARGUMENT;
  return run_layer(desc, d_prepared, d_X, M, d_Y, out_dtype, d_workspace, ws_bytes, stream, false, n);
}

svdq_status svdq_linear_w4a16(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, int M,
                              void* d_Y, int out_dtype, void* d_workspace, size_t ws_bytes, void* stream) {
  svdq_status st = validate_runtime(desc, d_prepared, d_X, M);
  if (st != SVDQ_OK) return st;
  if (desc->rank != 0 || M > kW4A16MaxM) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!d_Y || !d_workspace) return SVDQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != SVDQ_OUT_BF16 && out_dtype != SVDQ_OUT_F32) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_Y) || !aligned16(d_workspace)) return SVDQ_ERR_MISALIGNED;
  const ActLayout A = act_layout(*desc, M);
  if (ws_bytes < A.required) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  const BlobPtrs bp = blob_ptrs(*desc, d_prepared);
  W4A16Args a;
  a.X = static_cast<const uint16_t*>(d_X);
  a.M = M;
  a.K = desc->K;
  a.N = desc->N;
  a.inv_lam = bp.inv_lam;
  a.wcodes = bp.wcodes;
  a.wscales = bp.wscales;
  a.bias = bp.bias;
  a.Y = d_Y;
  a.out_f32 = out_dtype == SVDQ_OUT_F32;
  a.pieces = static_cast<uint8_t*>(d_workspace) + A.w4a16;
  return from_hip(launch_w4a16(desc->fmt, a, as_stream(stream)));
}

svdq_status svdq_linear(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, int M, void* d_Y,
                        int out_dtype, void* d_workspace, size_t ws_bytes, void* stream) {
  return run_layer(desc, d_prepared, d_X, M, d_Y, out_dtype, d_workspace, ws_bytes, stream, false);
}

svdq_status svdq_linear_unfused(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, int M,
                                void* d_Y, int out_dtype, void* d_workspace, size_t ws_bytes, void* stream) {
  return run_layer(desc, d_prepared, d_X, M, d_Y, out_dtype, d_workspace, ws_bytes, stream, true);
}

svdq_status svdq_linear_noalloc(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, int M,
                                void* d_Y, int out_dtype, void* stream) {
  svdq_status st = validate_runtime(desc, d_prepared, d_X, M);
  if (st != SVDQ_OK) return st;
  if (act_layout(*desc, M).required > SVDQ_NOALLOC_SCRATCH_BYTES) return SVDQ_ERR_BUFFER_TOO_SMALL;
  if ((st = check_device()) != SVDQ_OK) return st;
  void* ws = scratch_ptr();
  if (!ws) return SVDQ_ERR_HIP;
  return run_layer(desc, d_prepared, d_X, M, d_Y, out_dtype, ws, SVDQ_NOALLOC_SCRATCH_BYTES, stream, false);
}

}  // extern "C"
