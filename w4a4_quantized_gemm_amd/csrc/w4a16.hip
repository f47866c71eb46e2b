// The weight-only 4-bit layer (16-bit activations) for small M: the
// [diffusers] page's second operator, next to the W4A4 one, for the
// adaptive-norm and modulation projections (a handful of rows).
//
//   x_hat = fp32(x * inv_lambda)            (the layer's smoothing, not quantized)
//   Y     = round(x_hat dequant(Q(R)) + b)  (R = W_hat: a prepared layer of rank 0)
//
// Memory-bound: the 4-bit weights (K N / 2 bytes) are read once, the
// activations are a few KB.  A workgroup owns 32 output columns and one of
// `parts` equal K ranges: it stages the range's x_hat (rows x range fp32) in
// LDS, then each wave walks every fourth 64-wide K block of the range; in a
// block lane l holds column l % 32 and the 32 codes of K half l / 32 (one
// 16-byte load: the weight codes' operand-block order is exactly this),
// dequantizes them exactly in fp32 (INT4: the E4M3 code times s 2^9; FP4:
// the E2M1 value times 2^e) and accumulates rows x 32 products, reading the
// activations from LDS as broadcasts.  The two K halves, the four waves and
// (through the workspace) the K parts are added in a fixed order, so the
// result is deterministic.
#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int W_LDS = 65536;   // bytes of staged activations per workgroup
}  // namespace

template <int FMT, int MB>
__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ X, int M, int K, int N,
                                                    const float* __restrict__ inv_lam,
                                                    const uint8_t* __restrict__ wcodes, const void* __restrict__ wscales,
                                                    const float* __restrict__ bias, void* __restrict__ Y, int out_f32,
                                                    int parts, float* __restrict__ part_out) {
  __shared__ __attribute__((aligned(16))) float xs[W_LDS / 4];
  __shared__ float red[4][MB][32];
  const int nb = blockIdx.x, part = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_uniform(threadIdx.x >> 6);
  const int kblocks = K / 64, kbp = kblocks / parts, kb0 = part * kbp;
  const int range = kbp * 64;                     // K values of this part
  const int k0 = kb0 * 64;

  // stage x_hat of rows < MB (rows past M are zero) for the part's K range
  for (int i = threadIdx.x; i < MB * range / 2; i += 256) {
    const int m = (2 * i) / range, kk = (2 * i) % range;
    float a = 0.f, b = 0.f;
    if (m < M) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(X + static_cast<long>(m) * K + k0 + kk);
      a = bf16_lo(v) * inv_lam[k0 + kk];
      b = bf16_hi(v) * inv_lam[k0 + kk + 1];
    }
    xs[m * range + kk] = a;
    xs[m * range + kk + 1] = b;
  }
  __syncthreads();

  const int col = nb * 32 + (lane & 31), h = lane >> 5;
  const long KB = kblocks;
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; m++) acc[m] = 0.f;
  for (int kb = kb0 + wave; kb < kb0 + kbp; kb += 4) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(wcodes + ((nb * KB + kb) << 10) + lane * 16);
    float w[32];
    if constexpr (FMT == SVDQ_INT4_G64_FP16) {
      // E4M3 code bytes: word & 0x87878787 (codes 0-3), rotr(word, 4) & 0x87878787 (codes 4-7)
      const float s = __half2float(__ushort_as_half(static_cast<const uint16_t*>(wscales)[static_cast<long>(col) * KB + kb])) * 512.0f;
      const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint32_t lo = wd[i] & 0x87878787u, hi = __builtin_amdgcn_alignbit(wd[i], wd[i], 4) & 0x87878787u;
        w[8 * i + 0] = __builtin_amdgcn_cvt_f32_fp8(lo, 0) * s;
        w[8 * i + 1] = __builtin_amdgcn_cvt_f32_fp8(lo, 1) * s;
        w[8 * i + 2] = __builtin_amdgcn_cvt_f32_fp8(lo, 2) * s;
        w[8 * i + 3] = __builtin_amdgcn_cvt_f32_fp8(lo, 3) * s;
        w[8 * i + 4] = __builtin_amdgcn_cvt_f32_fp8(hi, 0) * s;
        w[8 * i + 5] = __builtin_amdgcn_cvt_f32_fp8(hi, 1) * s;
        w[8 * i + 6] = __builtin_amdgcn_cvt_f32_fp8(hi, 2) * s;
        w[8 * i + 7] = __builtin_amdgcn_cvt_f32_fp8(hi, 3) * s;
      }
    } else {
      // E2M1 pairs (even K in the low nibble) at unit scale, then times 2^e
      const int e = static_cast<int>(static_cast<const uint8_t*>(wscales)[fp4_scale_offset(col, kb * 64 + 32 * h, K)]) - 127;
      const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const f32x2 p[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 1.0f, 3)};
#pragma unroll
        for (int b = 0; b < 4; b++) {
          w[8 * i + 2 * b] = __builtin_amdgcn_ldexpf(p[b].x, e);
          w[8 * i + 2 * b + 1] = __builtin_amdgcn_ldexpf(p[b].y, e);
        }
      }
    }
    const float* xr = xs + (kb - kb0) * 64 + 32 * h;
#pragma unroll
    for (int m = 0; m < MB; m++) {
#pragma unroll
      for (int j = 0; j < 32; j += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(xr + m * range + j);
        acc[m] = __builtin_fmaf(x4.x, w[j], acc[m]);
        acc[m] = __builtin_fmaf(x4.y, w[j + 1], acc[m]);
        acc[m] = __builtin_fmaf(x4.z, w[j + 2], acc[m]);
        acc[m] = __builtin_fmaf(x4.w, w[j + 3], acc[m]);
      }
    }
  }
  // K halves (lane l and l + 32), then the waves in order
#pragma unroll
  for (int m = 0; m < MB; m++) {
    const float o = __shfl_xor(acc[m], 32);
    acc[m] = h == 0 ? acc[m] + o : o + acc[m];
  }
  if (h == 0) {
#pragma unroll
    for (int m = 0; m < MB; m++) red[wave][m][lane] = acc[m];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MB * 32; i += 256) {
    const int m = i / 32, cc = i % 32;
    if (m >= M) continue;
    const float v = ((red[0][m][cc] + red[1][m][cc]) + red[2][m][cc]) + red[3][m][cc];
    const long n = static_cast<long>(nb) * 32 + cc;
    if (parts > 1) {
      part_out[(static_cast<long>(part) * M + m) * N + n] = v;
    } else {
      const float y = v + (bias ? bias[n] : 0.f);
      if (out_f32) static_cast<float*>(Y)[static_cast<long>(m) * N + n] = y;
      else static_cast<uint16_t*>(Y)[static_cast<long>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(y));
    }
  }
}

// Y = round(sum over the parts, in part order, + b).
__global__ void w4a16_reduce_kernel(const float* __restrict__ part_out, int parts, int M, int N,
                                    const float* __restrict__ bias, void* __restrict__ Y, int out_f32) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long>(M) * N) return;
  float v = part_out[i];
  for (int p = 1; p < parts; p++) v += part_out[static_cast<long>(p) * M * N + i];
  const float y = v + (bias ? bias[i % N] : 0.f);
  if (out_f32) static_cast<float*>(Y)[i] = y;
  else static_cast<uint16_t*>(Y)[i] = static_cast<uint16_t>(f32_to_bf16_bits(y));
}

hipError_t launch_w4a16(int fmt, const W4A16Args& a, hipStream_t st) {
  const int rows = w4a16_rows(a.M), parts = w4a16_ksplit(a.M, a.K, a.N);
  dim3 grid(a.N / 32, parts), block(256);
#define SVDQ_W(F, MBV)                                                                                              \
  hipLaunchKernelGGL((w4a16_kernel<F, MBV>), grid, block, 0, st, a.X, a.M, a.K, a.N, a.inv_lam, a.wcodes, a.wscales, \
                     a.bias, a.Y, a.out_f32, parts, a.part)
#define SVDQ_WF(F)                       \
  switch (rows) {                        \
    case 1: SVDQ_W(F, 1); break;         \
    case 2: SVDQ_W(F, 2); break;         \
    case 4: SVDQ_W(F, 4); break;         \
    case 8: SVDQ_W(F, 8); break;         \
    case 16: SVDQ_W(F, 16); break;       \
    default: return hipErrorInvalidValue; \
  }
  if (fmt == SVDQ_INT4_G64_FP16) { SVDQ_WF(SVDQ_INT4_G64_FP16) }
  else { SVDQ_WF(SVDQ_FP4_E2M1_G32_E8M0) }
#undef SVDQ_WF
#undef SVDQ_W
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || parts == 1) return e;
  const long n = static_cast<long>(a.M) * a.N;
  hipLaunchKernelGGL(w4a16_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, a.part, parts,
                     a.M, a.N, a.bias, a.Y, a.out_f32);
  return hipGetLastError();
}

}  // namespace svdq
