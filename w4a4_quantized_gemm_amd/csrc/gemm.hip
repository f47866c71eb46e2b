// Kernel G: the 4-bit GEMM of the SVDQuant layer with the low-rank
// up-projection appended as an extra bf16 K-slab and a fused bias epilogue.
//
//   acc[i, n]  = sum_g s_x[i, g] s_w[g, n] sum_{k in g} q_x[i, k] q_w[k, n]
//                                              (walkthrough eq. (2) per group)
//   acc[i, n] += sum_t Tb[i, t] L2b[t, n]      (eq. (5) low-rank branch, Fig. 6:
//                                               it shares the 4-bit branch's output)
//   Y[i, n]    = round(acc[i, n] + b[n])
//
// INT4 (group 64, fp16 scales): the packed nibbles of a 64-wide K step are
// moved to LDS, and on the way from LDS to the registers each nibble is
// widened to a byte holding 16 * q (shift into the high half of the byte, so
// the sign comes for free); two 32x32x32 i8 MFMAs give 256 * P_g exactly in
// int32 and the group is dequantized into fp32 accumulators with
// s_x * s_w / 256.
// FP4 (group 32, E8M0 scales): the E2M1 nibbles and the power-of-two scales
// are the native operands of the gfx950 block-scaled MFMA (32x32x64), which
// accumulates in fp32 directly; there is no dequantization work.
//
// Tiling: 128 x 128 output tile per workgroup, 4 waves in a 2 x 2 grid, each
// wave 64 x 64 = 2 x 2 MFMA tiles of 32 x 32; K step 64; LDS double buffer
// with one barrier per step.  In every MFMA, lane l owns row (or column)
// l % 32 and the 16-byte half l / 32 of the K step, for A and B alike, so
// both operands enumerate K in the same order.
#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int LDS_STRIDE = 48;  // 32 data bytes per row + 16 pad bytes (bank spread)

__device__ __forceinline__ uint32_t lo_nib_bytes(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi_nib_bytes(uint32_t w) { return w & 0xF0F0F0F0u; }

template <int OUT>
__device__ __forceinline__ void store_out(void* Y, long idx, float v) {
  if constexpr (OUT == SVDQ_OUT_F32) {
    reinterpret_cast<float*>(Y)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(Y)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
}

template <int OUT>
__device__ __forceinline__ float load_out(const void* Y, long idx) {
  if constexpr (OUT == SVDQ_OUT_F32) {
    return reinterpret_cast<const float*>(Y)[idx];
  } else {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(Y)[idx]) << 16);
  }
}

}  // namespace

template <int FMT, bool SLAB, int OUT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) float sSA[2][BM];   // INT4: s_x of the step's group
  __shared__ __attribute__((aligned(16))) float sSB[2][BN];   // INT4: s_w / 256
  __shared__ __attribute__((aligned(16))) uint8_t sEA[2][BM * 2];  // FP4: E8M0 [row][block]
  __shared__ __attribute__((aligned(16))) uint8_t sEB[2][BN * 2];

  const int M = g.M, K = g.K, N = g.N;
  const int tiles_n = (N + BN - 1) / BN;
  const int tile_m = blockIdx.x / tiles_n;
  const int tile_n = blockIdx.x % tiles_n;
  const long m0 = static_cast<long>(tile_m) * BM;
  const long n0 = static_cast<long>(tile_n) * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int ld_r = t >> 1, ld_h = t & 1;
  const long KB = K / 2;             // bytes per code row
  const int steps = K / 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // ---- global -> registers for one K step
  uint4 ra, rb;
  uint32_t rs0 = 0, rs1 = 0;
  auto load_step = [&](int s) {
    const long am = m0 + ld_r, bn = n0 + ld_r;
    ra = am < M ? *reinterpret_cast<const uint4*>(g.acodes + am * KB + s * 32 + ld_h * 16)
                : make_uint4(0u, 0u, 0u, 0u);
    rb = bn < N ? *reinterpret_cast<const uint4*>(g.wcodes + bn * KB + s * 32 + ld_h * 16)
                : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (FMT == SVDQ_INT4_G64_FP16) {
      if (t < BM) {
        const long r = m0 + t;
        rs0 = r < M ? reinterpret_cast<const uint16_t*>(g.ascales)[r * (K / 64) + s] : 0u;
      } else {
        const long c = n0 + (t - BM);
        rs0 = c < N ? reinterpret_cast<const uint16_t*>(g.wscales)[static_cast<long>(s) * N + c] : 0u;
      }
    } else {
      if (t < BM) {
        const long r = m0 + t;
        rs0 = r < M ? reinterpret_cast<const uint16_t*>(g.ascales)[(r * (K / 32) + 2 * s) / 2] : 0x7F7Fu;
      } else {
        const long c = n0 + (t - BM);
        const uint8_t* ws = reinterpret_cast<const uint8_t*>(g.wscales);
        rs0 = c < N ? ws[static_cast<long>(2 * s) * N + c] : 127u;
        rs1 = c < N ? ws[static_cast<long>(2 * s + 1) * N + c] : 127u;
      }
    }
  };
  auto store_step = [&](int buf) {
    *reinterpret_cast<uint4*>(&sA[buf][ld_r * LDS_STRIDE + ld_h * 16]) = ra;
    *reinterpret_cast<uint4*>(&sB[buf][ld_r * LDS_STRIDE + ld_h * 16]) = rb;
    if constexpr (FMT == SVDQ_INT4_G64_FP16) {
      const float f = __half2float(__ushort_as_half(static_cast<unsigned short>(rs0)));
      if (t < BM) sSA[buf][t] = f;
      else sSB[buf][t - BM] = f * (1.0f / 256.0f);
    } else {
      if (t < BM) {
        sEA[buf][2 * t] = static_cast<uint8_t>(rs0 & 0xFFu);
        sEA[buf][2 * t + 1] = static_cast<uint8_t>(rs0 >> 8);
      } else {
        sEB[buf][2 * (t - BM)] = static_cast<uint8_t>(rs0);
        sEB[buf][2 * (t - BM) + 1] = static_cast<uint8_t>(rs1);
      }
    }
  };

  load_step(0);
  store_step(0);
  __syncthreads();

  for (int s = 0; s < steps; s++) {
    const int buf = s & 1;
    if (s + 1 < steps) load_step(s + 1);

    uint4 av[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; i++)
      av[i] = *reinterpret_cast<const uint4*>(&sA[buf][(wm * 64 + i * 32 + l32) * LDS_STRIDE + lh * 16]);
#pragma unroll
    for (int j = 0; j < 2; j++)
      bv[j] = *reinterpret_cast<const uint4*>(&sB[buf][(wn * 64 + j * 32 + l32) * LDS_STRIDE + lh * 16]);

    if constexpr (FMT == SVDQ_INT4_G64_FP16) {
      i32x4 a0[2], a1[2], b0[2], b1[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        a0[i] = i32x4{(int)lo_nib_bytes(av[i].x), (int)hi_nib_bytes(av[i].x), (int)lo_nib_bytes(av[i].y),
                      (int)hi_nib_bytes(av[i].y)};
        a1[i] = i32x4{(int)lo_nib_bytes(av[i].z), (int)hi_nib_bytes(av[i].z), (int)lo_nib_bytes(av[i].w),
                      (int)hi_nib_bytes(av[i].w)};
        b0[i] = i32x4{(int)lo_nib_bytes(bv[i].x), (int)hi_nib_bytes(bv[i].x), (int)lo_nib_bytes(bv[i].y),
                      (int)hi_nib_bytes(bv[i].y)};
        b1[i] = i32x4{(int)lo_nib_bytes(bv[i].z), (int)hi_nib_bytes(bv[i].z), (int)lo_nib_bytes(bv[i].w),
                      (int)hi_nib_bytes(bv[i].w)};
      }
      float4 sx[2][4];
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j4 = 0; j4 < 4; j4++)
          sx[i][j4] = *reinterpret_cast<const float4*>(&sSA[buf][wm * 64 + i * 32 + 8 * j4 + 4 * lh]);
      float sw[2];
#pragma unroll
      for (int j = 0; j < 2; j++) sw[j] = sSB[buf][wn * 64 + j * 32 + l32];
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
          i32x16 p;
#pragma unroll
          for (int v = 0; v < 16; v++) p[v] = 0;
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[i], b0[j], p, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[i], b1[j], p, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 16; v++) {
            const float4 s4 = sx[i][v >> 2];
            const float sxv = (v & 3) == 0 ? s4.x : (v & 3) == 1 ? s4.y : (v & 3) == 2 ? s4.z : s4.w;
            acc[i][j][v] = __builtin_fmaf(static_cast<float>(p[v]), sxv * sw[j], acc[i][j][v]);
          }
        }
    } else {
      i32x8 a[2], b[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        a[i] = i32x8{(int)av[i].x, (int)av[i].y, (int)av[i].z, (int)av[i].w, 0, 0, 0, 0};
        b[i] = i32x8{(int)bv[i].x, (int)bv[i].y, (int)bv[i].z, (int)bv[i].w, 0, 0, 0, 0};
        sa[i] = sEA[buf][(wm * 64 + i * 32 + l32) * 2 + lh];
        sb[i] = sEB[buf][(wn * 64 + i * 32 + l32) * 2 + lh];
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                        sb[j]);
    }

    if (s + 1 < steps) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- low-rank up-projection as one more K slab (K = rank), bf16 MFMA
  if constexpr (SLAB) {
    for (int tb = 0; tb < g.rank / 16; tb++) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const long r = m0 + wm * 64 + i * 32 + l32;
        const long c = n0 + wn * 64 + i * 32 + l32;
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; e++) z[e] = static_cast<__bf16>(0.f);
        a[i] = r < M ? *reinterpret_cast<const bf16x8*>(g.Tb + r * g.rank + tb * 16 + lh * 8) : z;
        b[i] = c < N ? *reinterpret_cast<const bf16x8*>(g.l2t + c * g.rank + tb * 16 + lh * 8) : z;
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: bias, rounding, store
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const long c = n0 + wn * 64 + j * 32 + l32;
    if (c >= N) continue;
    const float bv = g.bias ? g.bias[c] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const long r = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (r < M) store_out<OUT>(g.Y, r * N + c, acc[i][j][v] + bv);
      }
    }
  }
}

// Unfused up-projection: Y = round(Y + Tb L2b), 64 x 64 tile per workgroup.
template <int OUT>
__global__ __launch_bounds__(256) void up_kernel(const uint16_t* __restrict__ Tb, const uint16_t* __restrict__ l2t,
                                                 void* __restrict__ Y, int M, int N, int rank) {
  const int tiles_n = (N + 63) / 64;
  const long m0 = static_cast<long>(blockIdx.x / tiles_n) * 64;
  const long n0 = static_cast<long>(blockIdx.x % tiles_n) * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const long r = m0 + (wave >> 1) * 32 + l32;
  const long c = n0 + (wave & 1) * 32 + l32;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; v++) acc[v] = 0.f;
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; e++) z[e] = static_cast<__bf16>(0.f);
  for (int tb = 0; tb < rank / 16; tb++) {
    const bf16x8 a = r < M ? *reinterpret_cast<const bf16x8*>(Tb + r * rank + tb * 16 + lh * 8) : z;
    const bf16x8 b = c < N ? *reinterpret_cast<const bf16x8*>(l2t + c * rank + tb * 16 + lh * 8) : z;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  if (c >= N) return;
#pragma unroll
  for (int v = 0; v < 16; v++) {
    const long rr = m0 + (wave >> 1) * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
    if (rr < M) {
      const long idx = rr * N + c;
      store_out<OUT>(Y, idx, load_out<OUT>(Y, idx) + acc[v]);
    }
  }
}

hipError_t launch_gemm(int fmt, bool slab, int out_dtype, const GemmArgs& g, hipStream_t st) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles), block(256);
#define SVDQ_G(F, S, O) hipLaunchKernelGGL((gemm_kernel<F, S, O>), grid, block, 0, st, g)
  const bool f32 = out_dtype == SVDQ_OUT_F32;
  if (fmt == SVDQ_INT4_G64_FP16) {
    if (slab) { if (f32) SVDQ_G(SVDQ_INT4_G64_FP16, true, SVDQ_OUT_F32); else SVDQ_G(SVDQ_INT4_G64_FP16, true, SVDQ_OUT_BF16); }
    else      { if (f32) SVDQ_G(SVDQ_INT4_G64_FP16, false, SVDQ_OUT_F32); else SVDQ_G(SVDQ_INT4_G64_FP16, false, SVDQ_OUT_BF16); }
  } else {
    if (slab) { if (f32) SVDQ_G(SVDQ_FP4_E2M1_G32_E8M0, true, SVDQ_OUT_F32); else SVDQ_G(SVDQ_FP4_E2M1_G32_E8M0, true, SVDQ_OUT_BF16); }
    else      { if (f32) SVDQ_G(SVDQ_FP4_E2M1_G32_E8M0, false, SVDQ_OUT_F32); else SVDQ_G(SVDQ_FP4_E2M1_G32_E8M0, false, SVDQ_OUT_BF16); }
  }
#undef SVDQ_G
  return hipGetLastError();
}

hipError_t launch_up(int out_dtype, const uint16_t* Tb, const uint16_t* l2t, void* Y, int M, int N, int rank,
                     hipStream_t st) {
  if (rank == 0) return hipSuccess;
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  if (out_dtype == SVDQ_OUT_F32)
    hipLaunchKernelGGL(up_kernel<SVDQ_OUT_F32>, dim3(tiles), dim3(256), 0, st, Tb, l2t, Y, M, N, rank);
  else
    hipLaunchKernelGGL(up_kernel<SVDQ_OUT_BF16>, dim3(tiles), dim3(256), 0, st, Tb, l2t, Y, M, N, rank);
  return hipGetLastError();
}

}  // namespace svdq
