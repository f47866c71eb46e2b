// Descriptor validation, blob layout and size queries.  Host-only, no HIP.
#include <cmath>
#include <cstring>

#include "svdq_internal.h"

namespace svdq {

svdq_status validate_desc(const svdq_layer_desc* d) {
  if (!d) return SVDQ_ERR_INVALID_ARGUMENT;
  if (d->fmt != SVDQ_INT4_G64_FP16 && d->fmt != SVDQ_FP4_E2M1_G32_E8M0) return SVDQ_ERR_INVALID_ARGUMENT;
  if (d->flags & ~kKnownFlags) return SVDQ_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(d->alpha) || d->alpha < 0.f || d->alpha > 1.f) return SVDQ_ERR_INVALID_ARGUMENT;
  if (d->K < 128 || d->K > kMaxDim || d->K % 128 != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (d->N < 64 || d->N > kMaxDim || d->N % 64 != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (d->rank < 0 || d->rank > kMaxRank || d->rank % 16 != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (d->rank > d->K || d->rank > d->N) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  return SVDQ_OK;
}

svdq_status validate_m(int M) {
  if (M < 1 || M > kMaxM) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  return SVDQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

svdq_blob_layout layout_of(const svdq_layer_desc& d) {
  svdq_blob_layout L{};
  const uint64_t K = d.K, N = d.N, r = d.rank;
  const uint64_t g = group_of(d.fmt);
  uint64_t off = 0;
  L.header = off;
  off = align256(off + sizeof(BlobHeader));
  L.lambda = off;
  off = align256(off + 4 * K);
  L.inv_lambda = off;
  off = align256(off + 4 * K);
  L.l1t = off;
  off = align256(off + 2 * r * K);
  L.l2t = off;
  off = align256(off + 2 * N * r);
  L.wcodes = off;
  off = align256(off + N * (K / 2));
  L.wscales = off;
  off = align256(off + (K / g) * N * scale_bytes_of(d.fmt));
  if (d.flags & SVDQ_F_HAS_BIAS) {
    L.bias = off;
    off = align256(off + 4 * N);
  } else {
    L.bias = 0;
  }
  L.total = off;
  return L;
}

ActLayout act_layout(const svdq_layer_desc& d, int M) {
  ActLayout A{};
  const uint64_t m = M, K = d.K;
  const uint64_t mp = ((m + 31) / 32) * 32;         // rows padded to whole 32-row blocks
  A.codes_bytes = mp * (K / 2);
  // scales and T are stored in 32-row blocks too
  A.scales_bytes = mp * (K / group_of(d.fmt)) * scale_bytes_of(d.fmt);
  A.tb_bytes = mp * uint64_t(d.rank) * 2;
  uint64_t off = 0;
  A.codes = off;
  off = align256(off + A.codes_bytes);
  A.scales = off;
  off = align256(off + A.scales_bytes);
  A.tb = off;
  off = align256(off + A.tb_bytes);
  // fp32 partial T of the K parts of the activation pass (at most kMaxKParts)
  A.tpart = off;
  off = align256(off + (m <= kSplitMaxM ? uint64_t(kMaxKParts) * m * uint64_t(d.rank) * 4 : 0));
  // norm-fused pass: per-row mean and 1/std, then gamma' and beta'
  A.rowstat = off;
  off = align256(off + m * 8);
  A.fold = off;
  off = align256(off + K * 8);
  // weight-only layer: the bf16 pieces of x_hat
  A.w4a16 = off;
  if (d.rank == 0 && M <= kW4A16MaxM) off = align256(off + K * 64 * uint64_t(w4a16_planes(M)));
  // split-K INT4 GEMM (few output tiles): the fp32 partial tiles
  A.ypart = off;
  A.required = off;
  if (gemm_may_split(d, M)) off = align256(off + kGemmSplitBytes);
  A.total = off;
  return A;
}

}  // namespace svdq

using namespace svdq;

extern "C" {

const char* svdq_status_string(int s) {
  switch (s) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_ERR_INVALID_ARGUMENT: return "SVDQ_ERR_INVALID_ARGUMENT: a pointer, enum, flag or alpha is invalid";
    case SVDQ_ERR_UNSUPPORTED_SHAPE: return "SVDQ_ERR_UNSUPPORTED_SHAPE: K, N, rank or M is outside the supported set";
    case SVDQ_ERR_UNSUPPORTED_DEVICE: return "SVDQ_ERR_UNSUPPORTED_DEVICE: no gfx950 (MI355X) device is current";
    case SVDQ_ERR_BUFFER_TOO_SMALL: return "SVDQ_ERR_BUFFER_TOO_SMALL: a prepared or workspace buffer is too small";
    case SVDQ_ERR_HIP: return "SVDQ_ERR_HIP: a HIP runtime call or kernel launch failed";
    case SVDQ_ERR_BAD_BLOB: return "SVDQ_ERR_BAD_BLOB: the prepared blob does not match the layer descriptor";
    case SVDQ_ERR_MISALIGNED: return "SVDQ_ERR_MISALIGNED: a buffer is not 16-byte aligned";
    default: return "unknown svdq_status";
  }
}

int svdq_version(void) { return 100; }

size_t svdq_prepared_bytes(const svdq_layer_desc* desc) {
  if (validate_desc(desc) != SVDQ_OK) return 0;
  return static_cast<size_t>(layout_of(*desc).total);
}

size_t svdq_workspace_bytes(const svdq_layer_desc* desc, int M, int unfused) {
  (void)unfused;  // both paths stage the same activation buffers
  if (validate_desc(desc) != SVDQ_OK || validate_m(M) != SVDQ_OK) return 0;
  return static_cast<size_t>(act_layout(*desc, M).total);
}

svdq_status svdq_act_sizes(const svdq_layer_desc* desc, int M, size_t* codes_bytes,
                           size_t* scales_bytes, size_t* t_bytes) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if ((st = validate_m(M)) != SVDQ_OK) return st;
  ActLayout A = act_layout(*desc, M);
  if (codes_bytes) *codes_bytes = A.codes_bytes;
  if (scales_bytes) *scales_bytes = A.scales_bytes;
  if (t_bytes) *t_bytes = A.tb_bytes;
  return SVDQ_OK;
}

svdq_status svdq_blob_layout_of(const svdq_layer_desc* desc, svdq_blob_layout* out) {
  svdq_status st = validate_desc(desc);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_INVALID_ARGUMENT;
  *out = layout_of(*desc);
  return SVDQ_OK;
}

}  // extern "C"
