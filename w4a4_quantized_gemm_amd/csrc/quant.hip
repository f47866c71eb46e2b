// Kernel Q: the fused activation pass of the SVDQuant layer.
//
// One read of X produces (SVDQuant walkthrough, Fig. 6: the down-projection
// and the quantizer consume the same input):
//   x_hat = fp32(x * inv_lambda)                          (eq. (5) smoothing)
//   per token row and K group: absmax scale and 4-bit codes (eq. (1))
//   T = bf16(x_hat) L1b on the bf16 MFMA, fp32 accumulation -> bf16
//
// Work split: a workgroup owns 16 token rows; its 4 waves take interleaved
// 128-wide K chunks (wave w: chunks w, w+4, ...).  In a chunk, lane l holds
// row l % 16 and the 32 consecutive K elements 32 * (l / 16) .. + 31, loaded as
// four 16-byte vectors.  An INT4 group (64) is the lane pair (l, l ^ 16); an
// FP4 group (32) is one lane.  The 32 values are also the A operands of four
// 16x16x32 bf16 MFMAs (8 consecutive K per MFMA), whose B operands come from
// L1 stored transposed (L1t[t][k]), so the k index sets of A and B match.
// The per-wave partial T tiles are summed across the 4 waves in LDS in a
// fixed order, so T is deterministic.
#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

template <int FMT, bool QUANT, bool DOWN, int RB>
__global__ __launch_bounds__(256) void act_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                  const float* __restrict__ inv_lam,
                                                  const uint16_t* __restrict__ l1t,
                                                  uint8_t* __restrict__ codes,
                                                  void* __restrict__ scales,
                                                  uint16_t* __restrict__ Tb) {
  constexpr int R = RB * 16;
  __shared__ float red[(DOWN && RB > 0) ? 4 * 16 * R : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;
  const int kq = lane >> 4;
  const long grow = static_cast<long>(blockIdx.x) * 16 + row;
  const bool valid = grow < M;
  const int iters = K >> 7;

  f32x4 acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int nb = 0; nb < (RB > 0 ? RB : 1); nb++) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = wave; it < iters; it += 4) {
    const int kb = it * 128 + kq * 32;
    float xh[32];
    {
      uint4 raw[4];
      const uint4* src = reinterpret_cast<const uint4*>(X + grow * K + kb);
#pragma unroll
      for (int c = 0; c < 4; c++) raw[c] = valid ? src[c] : make_uint4(0u, 0u, 0u, 0u);
      const float4* il = reinterpret_cast<const float4*>(inv_lam + kb);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const float4 i0 = il[2 * c], i1 = il[2 * c + 1];
        xh[8 * c + 0] = bf16_lo(raw[c].x) * i0.x;
        xh[8 * c + 1] = bf16_hi(raw[c].x) * i0.y;
        xh[8 * c + 2] = bf16_lo(raw[c].y) * i0.z;
        xh[8 * c + 3] = bf16_hi(raw[c].y) * i0.w;
        xh[8 * c + 4] = bf16_lo(raw[c].z) * i1.x;
        xh[8 * c + 5] = bf16_hi(raw[c].z) * i1.y;
        xh[8 * c + 6] = bf16_lo(raw[c].w) * i1.z;
        xh[8 * c + 7] = bf16_hi(raw[c].w) * i1.w;
      }
    }

    if constexpr (QUANT) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; e++) amax = fmaxf(amax, __builtin_fabsf(xh[e]));
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
      if constexpr (FMT == SVDQ_INT4_G64_FP16) {
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        const __half sh = __float2half_rn(amax / 7.0f);
        const float s = __half2float(sh);
        if (s > 0.f) {
          const float r = 1.0f / s;
#pragma unroll
          for (int e = 0; e < 32; e++) {
            float q = rne_quotient(xh[e], s, r);
            q = fminf(fmaxf(q, -7.f), 7.f);
            packed[e >> 3] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xFu) << (4 * (e & 7));
          }
        }
        if (valid && (kq & 1) == 0)
          reinterpret_cast<uint16_t*>(scales)[grow * (K / 64) + kb / 64] = __half_as_ushort(sh);
      } else {
        const int ex = e8m0_exponent(amax);
#pragma unroll
        for (int e = 0; e < 32; e++) {
          const float y = __builtin_amdgcn_ldexpf(xh[e], -ex);
          packed[e >> 3] |= e2m1_code(y) << (4 * (e & 7));
        }
        if (valid) reinterpret_cast<uint8_t*>(scales)[fp4_scale_offset(grow, kb, K)] = static_cast<uint8_t>(ex + 127);
      }
      if (valid)
        *reinterpret_cast<u32x4*>(codes + code_chunk_offset(grow, kb, K)) =
            u32x4{packed[0], packed[1], packed[2], packed[3]};
    }

    if constexpr (DOWN && RB > 0) {
      bf16x8 a[4];
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 8; e++) a[j][e] = static_cast<__bf16>(xh[8 * j + e]);
#pragma unroll
      for (int nb = 0; nb < RB; nb++) {
        const bf16x8* lp = reinterpret_cast<const bf16x8*>(l1t + static_cast<long>(nb * 16 + row) * K + kb);
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], lp[j], acc[nb], 0, 0, 0);
      }
    }
  }

  if constexpr (DOWN && RB > 0) {
    // acc[nb][v] is this wave's partial T[4 * kq + v][nb * 16 + (lane & 15)]
#pragma unroll
    for (int nb = 0; nb < RB; nb++)
#pragma unroll
      for (int v = 0; v < 4; v++) red[(wave * 16 + 4 * kq + v) * R + nb * 16 + row] = acc[nb][v];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * R; idx += 256) {
      const int rr = idx / R, t = idx % R;
      const float s = ((red[(0 * 16 + rr) * R + t] + red[(1 * 16 + rr) * R + t]) + red[(2 * 16 + rr) * R + t]) +
                      red[(3 * 16 + rr) * R + t];
      const long gr = static_cast<long>(blockIdx.x) * 16 + rr;
      if (gr < M) Tb[bf16_block_index(gr, t, R)] = static_cast<uint16_t>(f32_to_bf16_bits(s));
    }
  }
}

template <int FMT, bool QUANT, bool DOWN>
static hipError_t launch_act_rb(int rb, const ActArgs& a, hipStream_t st) {
  dim3 grid((a.M + 15) / 16), block(256);
#define SVDQ_ACT_CASE(RBV)                                                                              \
  case RBV:                                                                                           \
    hipLaunchKernelGGL((act_kernel<FMT, QUANT, DOWN, RBV>), grid, block, 0, st, a.X, a.M, a.K, a.inv_lam, \
                       a.l1t, a.codes, a.scales, a.Tb);                                              \
    break;
  switch (rb) {
    SVDQ_ACT_CASE(0) SVDQ_ACT_CASE(1) SVDQ_ACT_CASE(2) SVDQ_ACT_CASE(3) SVDQ_ACT_CASE(4)
    SVDQ_ACT_CASE(5) SVDQ_ACT_CASE(6) SVDQ_ACT_CASE(7) SVDQ_ACT_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_ACT_CASE
  return hipGetLastError();
}

hipError_t launch_act(int fmt, bool quant, bool down, const ActArgs& a, hipStream_t st) {
  const int rb = down ? a.rank / 16 : 0;
  if (fmt == SVDQ_INT4_G64_FP16) {
    if (quant && down) return launch_act_rb<SVDQ_INT4_G64_FP16, true, true>(rb, a, st);
    if (quant) return launch_act_rb<SVDQ_INT4_G64_FP16, true, false>(0, a, st);
    return launch_act_rb<SVDQ_INT4_G64_FP16, false, true>(rb, a, st);
  }
  if (quant && down) return launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, true, true>(rb, a, st);
  if (quant) return launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, true, false>(0, a, st);
  return launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, false, true>(rb, a, st);
}

// Calibration statistic: absmax[j] = max_i |X[i, j]|.  Non-negative floats
// order like their bit patterns, so an integer atomic max is exact and the
// result does not depend on the order of the atomics.
__global__ void absmax_clear_kernel(float* __restrict__ out, int K) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < K) out[j] = 0.f;
}

__global__ void absmax_kernel(const uint16_t* __restrict__ X, int M, int K, int rows_per_block,
                              float* __restrict__ out) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const long r0 = static_cast<long>(blockIdx.y) * rows_per_block;
  long r1 = r0 + rows_per_block;
  if (r1 > M) r1 = M;
  uint32_t m = 0;
  for (long i = r0; i < r1; i++) {
    const uint32_t b = X[i * K + j] & 0x7FFFu;
    m = b > m ? b : m;
  }
  atomicMax(reinterpret_cast<unsigned int*>(out) + j, m << 16);
}

hipError_t launch_absmax(const uint16_t* X, int M, int K, float* out, bool accumulate, hipStream_t st) {
  if (!accumulate) {
    hipLaunchKernelGGL(absmax_clear_kernel, dim3((K + 255) / 256), dim3(256), 0, st, out, K);
  }
  const int rows = 64;
  dim3 grid((K + 255) / 256, (M + rows - 1) / rows);
  hipLaunchKernelGGL(absmax_kernel, grid, dim3(256), 0, st, X, M, K, rows, out);
  return hipGetLastError();
}

}  // namespace svdq
