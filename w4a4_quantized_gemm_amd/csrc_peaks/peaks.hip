// libsvdq_peaks: matrix-core and HBM microbenchmarks (include/svdq_peaks.h).
// Each MFMA probe keeps 8 independent accumulators per wave so the matrix
// core never waits on a result; one wave per SIMD.  The HBM probes stream
// 16-byte vectors with four loads in flight per lane.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "svdq_peaks.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NACC = 8;

// operand bits: a constant, or xorshift bits masked to valid codes of the
// format (no NaN or infinity; bf16 / f16 magnitudes below 2)
__device__ __forceinline__ uint32_t operand_word(uint32_t& seed, bool random, uint32_t mask) {
  if (!random) return 0x3C3C3C3Cu & mask;
  seed ^= seed << 13;
  seed ^= seed >> 17;
  seed ^= seed << 5;
  return seed & mask;
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe(int iters, int random, float* __restrict__ sink) {
  uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
  constexpr uint32_t MASK = KIND == SVDQ_PEAK_FP8 ? 0xF7F7F7F7u
                            : (KIND == SVDQ_PEAK_BF16 || KIND == SVDQ_PEAK_F16) ? 0xBFFFBFFFu
                                                                                : 0xFFFFFFFFu;
  uint32_t wa[8], wb[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    wa[i] = operand_word(seed, random != 0, MASK);
    wb[i] = operand_word(seed, random != 0, MASK);
  }
  float out = 0.f;
  if constexpr (KIND == SVDQ_PEAK_INT8) {
    const i32x4 a = {(int)wa[0], (int)wa[1], (int)wa[2], (int)wa[3]};
    const i32x4 b = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3]};
    i32x16 acc[NACC];
#pragma unroll
    for (int k = 0; k < NACC; k++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[k][v] = 0;
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int k = 0; k < NACC; k++) acc[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[k], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < NACC; k++)
#pragma unroll
      for (int v = 0; v < 16; v++) out += static_cast<float>(acc[k][v]);
  } else {
    f32x16 acc[NACC];
#pragma unroll
    for (int k = 0; k < NACC; k++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[k][v] = 0.f;
    if constexpr (KIND == SVDQ_PEAK_BF16) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{wa[0], wa[1], wa[2], wa[3]});
      const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{wb[0], wb[1], wb[2], wb[3]});
      for (int it = 0; it < iters; it++)
#pragma unroll
        for (int k = 0; k < NACC; k++) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    } else if constexpr (KIND == SVDQ_PEAK_F16) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const f16x4 a = __builtin_bit_cast(f16x4, u32x2{wa[0], wa[1]});
      const f16x4 b = __builtin_bit_cast(f16x4, u32x2{wb[0], wb[1]});
      for (int it = 0; it < iters; it++)
#pragma unroll
        for (int k = 0; k < NACC; k++) acc[k] = __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, acc[k], 0, 0, 0);
    } else {
      // block-scaled 32x32x64: E4M3 uses 8 operand registers, E2M3 6, E2M1 4
      constexpr int FMT = KIND == SVDQ_PEAK_FP4 ? 4 : KIND == SVDQ_PEAK_FP6 ? 2 : 0;
      constexpr int NREG = KIND == SVDQ_PEAK_FP4 ? 4 : KIND == SVDQ_PEAK_FP6 ? 6 : 8;
      i32x8 a, b;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        a[i] = i < NREG ? static_cast<int>(wa[i]) : 0;
        b[i] = i < NREG ? static_cast<int>(wb[i]) : 0;
      }
      for (int it = 0; it < iters; it++)
#pragma unroll
        for (int k = 0; k < NACC; k++)
          acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[k], FMT, FMT, 0, 127, 0, 127);
    }
#pragma unroll
    for (int k = 0; k < NACC; k++)
#pragma unroll
      for (int v = 0; v < 16; v++) out += acc[k][v];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = out;
}

__global__ __launch_bounds__(256) void hbm_read_probe(const u32x4* __restrict__ src, size_t n, u32x4* __restrict__ dst) {
  u32x4 x = {0u, 0u, 0u, 0u};
  const size_t stride = static_cast<size_t>(gridDim.x) * 256 * 4;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 1024 + threadIdx.x; i < n; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = i + u * 256 < n ? __builtin_nontemporal_load(src + i + u * 256) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; u++) x ^= v[u];
  }
  if ((x.x | x.y | x.z | x.w) == 0x9E3779B9u) dst[0] = x;   // practically never: keeps the loads alive
}

__global__ __launch_bounds__(256) void hbm_copy_probe(const u32x4* __restrict__ src, size_t n, u32x4* __restrict__ dst) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256 * 4;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 1024 + threadIdx.x; i < n; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = i + u * 256 < n ? __builtin_nontemporal_load(src + i + u * 256) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; u++)
      if (i + u * 256 < n) __builtin_nontemporal_store(v[u], dst + i + u * 256);
  }
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

// Launch `launch` between two events on the stream; the elapsed ms.
template <typename F>
int timed(hipStream_t st, F launch, double* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return 5;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return 5;
  }
  int rc = 0;
  if (hipEventRecord(e0, st) != hipSuccess) rc = 5;
  if (!rc) {
    launch();
    if (hipGetLastError() != hipSuccess) rc = 5;
  }
  if (!rc && hipEventRecord(e1, st) != hipSuccess) rc = 5;
  if (!rc && hipEventSynchronize(e1) != hipSuccess) rc = 5;
  float t = 0.f;
  if (!rc && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = 5;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *ms = t;
  return rc;
}

}  // namespace

extern "C" {

int svdq_peak_mfma(int kind, int iters, int workgroups, int random_operands, void* d_sink, double* tops, double* ms,
                   void* stream) {
  if (!d_sink || !tops || !ms || iters < 1 || workgroups < 0 || kind < 0 || kind > SVDQ_PEAK_F16) return 1;
  const int wgs = workgroups ? workgroups : cu_count();
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* sink = static_cast<float*>(d_sink);
  const double per_mfma = kind == SVDQ_PEAK_INT8 ? 65536.0 : kind == SVDQ_PEAK_BF16 ? 32768.0
                          : kind == SVDQ_PEAK_F16 ? 16384.0 : 131072.0;
  auto launch = [&]() {
    switch (kind) {
      case SVDQ_PEAK_FP4: hipLaunchKernelGGL(mfma_probe<SVDQ_PEAK_FP4>, dim3(wgs), dim3(256), 0, st, iters, random_operands, sink); break;
      case SVDQ_PEAK_FP6: hipLaunchKernelGGL(mfma_probe<SVDQ_PEAK_FP6>, dim3(wgs), dim3(256), 0, st, iters, random_operands, sink); break;
      case SVDQ_PEAK_FP8: hipLaunchKernelGGL(mfma_probe<SVDQ_PEAK_FP8>, dim3(wgs), dim3(256), 0, st, iters, random_operands, sink); break;
      case SVDQ_PEAK_INT8: hipLaunchKernelGGL(mfma_probe<SVDQ_PEAK_INT8>, dim3(wgs), dim3(256), 0, st, iters, random_operands, sink); break;
      case SVDQ_PEAK_BF16: hipLaunchKernelGGL(mfma_probe<SVDQ_PEAK_BF16>, dim3(wgs), dim3(256), 0, st, iters, random_operands, sink); break;
      default: hipLaunchKernelGGL(mfma_probe<SVDQ_PEAK_F16>, dim3(wgs), dim3(256), 0, st, iters, random_operands, sink); break;
    }
  };
  const int rc = timed(st, launch, ms);
  if (rc) return rc;
  // 4 waves per workgroup, NACC MFMAs per wave and round
  *tops = per_mfma * NACC * 4.0 * wgs * iters / (*ms * 1e-3) / 1e12;
  return 0;
}

int svdq_peak_hbm(int mode, const void* d_src, void* d_dst, size_t bytes, double* gbs, double* ms, void* stream) {
  if (!d_src || !d_dst || !gbs || !ms || bytes == 0 || bytes % 16 || (mode != 0 && mode != 1)) return 1;
  if ((reinterpret_cast<uintptr_t>(d_src) | reinterpret_cast<uintptr_t>(d_dst)) & 15) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n = bytes / 16;
  const int wgs = cu_count() * 8;
  auto launch = [&]() {
    if (mode == 0)
      hipLaunchKernelGGL(hbm_read_probe, dim3(wgs), dim3(256), 0, st, static_cast<const u32x4*>(d_src), n,
                         static_cast<u32x4*>(d_dst));
    else
      hipLaunchKernelGGL(hbm_copy_probe, dim3(wgs), dim3(256), 0, st, static_cast<const u32x4*>(d_src), n,
                         static_cast<u32x4*>(d_dst));
  };
  const int rc = timed(st, launch, ms);
  if (rc) return rc;
  *gbs = static_cast<double>(bytes) * (mode == 0 ? 1.0 : 2.0) / (*ms * 1e-3) / 1e9;
  return 0;
}

}  // extern "C"
