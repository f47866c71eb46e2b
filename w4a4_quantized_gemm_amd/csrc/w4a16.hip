// The weight-only 4-bit layer (16-bit activations) for small M: the
// [diffusers] page's second operator, next to the W4A4 one, for the
// adaptive-norm and modulation projections (a handful of rows).
//
//   x_hat = fp32(x * inv_lambda)            (the layer's smoothing, not quantized)
//   Y     = round(x_hat dequant(Q(R)) + b)  (R = W_hat: a prepared layer of rank 0)
//
// Memory-bound: the 4-bit weights (K N / 2 bytes) are read once, the
// activations are a few KB.  A workgroup owns 4 x 32 output columns and one
// of `parts` equal K ranges: it stages the range's x_hat (rows x range fp32,
// at most 64 KB, sized at launch) in LDS, then each wave walks every fourth
// 64-wide K block of the range with two to four blocks in flight; in a block lane l
// holds column l % 32 of each of the 4 column blocks and the 32 codes of K
// half l / 32 (one 16-byte load each: the weight codes' operand-block order
// is exactly this), dequantizes them four K at a time exactly in fp32 (INT4:
// the E4M3 code times s 2^9; FP4: the E2M1 value times 2^e) and multiplies
// them with every row's four activations (one LDS broadcast read feeding 16
// fma).  The two K halves, the four waves and
// (through the workspace) the K parts are added in a fixed order, so the
// result is deterministic.
#include <algorithm>

#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {
typedef float f32x2 __attribute__((ext_vector_type(2)));
}  // namespace

constexpr int W_CB = 4;        // 32-column blocks per workgroup (each lane holds one column of each)

template <int FMT, int MB>
__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ X, int M, int K, int N,
                                                    const float* __restrict__ inv_lam,
                                                    const uint8_t* __restrict__ wcodes, const void* __restrict__ wscales,
                                                    const float* __restrict__ bias, void* __restrict__ Y, int out_f32,
                                                    int parts, float* __restrict__ part_out) {
  // MB x range fp32 activations; after the K loop the same memory holds the
  // cross-wave reduction (launch-sized to the larger of the two)
  extern __shared__ __attribute__((aligned(16))) float xs[];
  const int part = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_uniform(threadIdx.x >> 6);
  const int kblocks = K / 64, kbp = kblocks / parts, kb0 = part * kbp;
  const int range = kbp * 64;                     // K values of this part
  const int k0 = kb0 * 64;
  const int ncb = N / 32;                         // 32-column blocks

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

  const int h = lane >> 5;
  const long KB = kblocks;
  // the lane's W_CB columns (blocks past the matrix are clamped to its last
  // one and not stored)
  int cbk[W_CB], col[W_CB];
#pragma unroll
  for (int b = 0; b < W_CB; b++) {
    cbk[b] = min(static_cast<int>(blockIdx.x) * W_CB + b, ncb - 1);
    col[b] = cbk[b] * 32 + (lane & 31);
  }
  float acc[MB][W_CB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int b = 0; b < W_CB; b++) acc[m][b] = 0.f;
  // The wave's blocks kb = kb0 + wave + 4 t, t < nt, per column block one
  // 16-byte code load and one scale load per lane, requested PF blocks ahead
  // through buffer resources (offsets past a part's last block lie past the
  // resource's end and read nothing).
  constexpr int PF = MB <= 2 ? 4 : 2;       // fewer blocks in flight where the accumulators take the registers
  const int nt = (kbp - wave + 3) / 4;
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wcodes), 0, static_cast<int>(ncb * KB * 1024), 0x00020000);
  const uint32_t c_oob = static_cast<uint32_t>(ncb * KB * 1024);
  // scales: INT4 one fp16 per 64-group, FP4 one byte per 32-group: 2 N K / 64 bytes either way
  const int sbytes = N * static_cast<int>(KB) * 2;
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wscales), 0, sbytes, 0x00020000);
  u32x4 cq[PF][W_CB];
  uint32_t sq[PF][W_CB];
  auto fetch = [&](int t, int slot) __attribute__((always_inline)) {
    const int kb = kb0 + wave + 4 * t;
    const bool ok = t < nt;
#pragma unroll
    for (int b = 0; b < W_CB; b++) {
      cq[slot][b] = __builtin_amdgcn_raw_buffer_load_b128(
          cr, ok ? static_cast<uint32_t>((cbk[b] * KB + kb) * 1024 + lane * 16) : c_oob, 0, 0);
      if constexpr (FMT == SVDQ_INT4_G64_FP16)
        sq[slot][b] = __builtin_amdgcn_raw_buffer_load_b16(
            sr, ok ? static_cast<uint32_t>((static_cast<long>(col[b]) * KB + kb) * 2) : static_cast<uint32_t>(sbytes), 0, 0);
      else
        sq[slot][b] = __builtin_amdgcn_raw_buffer_load_b8(
            sr, ok ? static_cast<uint32_t>(fp4_scale_offset(col[b], kb * 64 + 32 * h, K)) : static_cast<uint32_t>(sbytes),
            0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < PF; d++) fetch(d, d);
  for (int t0 = 0; t0 < nt; t0 += PF) {
#pragma unroll
    for (int d = 0; d < PF; d++) {
      const int t = t0 + d;
      u32x4 c[W_CB];
      float sc[W_CB];
#pragma unroll
      for (int b = 0; b < W_CB; b++) {
        c[b] = cq[d][b];
        if constexpr (FMT == SVDQ_INT4_G64_FP16)
          sc[b] = __half2float(__ushort_as_half(static_cast<uint16_t>(sq[d][b]))) * 512.0f;   // s 2^9
        else
          sc[b] = __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(sq[d][b] & 0xFFu) - 127);   // 2^e
      }
      fetch(t + PF, d);
      if (t < nt) {
        const int kb = kb0 + wave + 4 * t;
        const float* xr = xs + (kb - kb0) * 64 + 32 * h;
        // four K values at a time: the exact fp32 weights of the W_CB
        // columns, then every row's four activations (one LDS broadcast
        // read) times them
#pragma unroll 2
        for (int j = 0; j < 8; j++) {
          float w[W_CB][4];
#pragma unroll
          for (int b = 0; b < W_CB; b++) {
            const uint32_t wd = j < 2 ? c[b].x : j < 4 ? c[b].y : j < 6 ? c[b].z : c[b].w;
            if constexpr (FMT == SVDQ_INT4_G64_FP16) {
              // E4M3 code bytes: word & 0x87878787 (codes 0-3), rotr(word, 4) & 0x87878787 (codes 4-7)
              const uint32_t q = ((j & 1) ? __builtin_amdgcn_alignbit(wd, wd, 4) : wd) & 0x87878787u;
              w[b][0] = __builtin_amdgcn_cvt_f32_fp8(q, 0) * sc[b];
              w[b][1] = __builtin_amdgcn_cvt_f32_fp8(q, 1) * sc[b];
              w[b][2] = __builtin_amdgcn_cvt_f32_fp8(q, 2) * sc[b];
              w[b][3] = __builtin_amdgcn_cvt_f32_fp8(q, 3) * sc[b];
            } else {
              // E2M1 pairs, even K in the low nibble: bytes 2 (j % 2) and 2 (j % 2) + 1
              const f32x2 p0 = (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 2)
                                       : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 0);
              const f32x2 p1 = (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 3)
                                       : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 1);
              w[b][0] = p0.x * sc[b];
              w[b][1] = p0.y * sc[b];
              w[b][2] = p1.x * sc[b];
              w[b][3] = p1.y * sc[b];
            }
          }
#pragma unroll
          for (int m = 0; m < MB; m++) {
            const f32x4 x4 = *reinterpret_cast<const f32x4*>(xr + m * range + 4 * j);
#pragma unroll
            for (int b = 0; b < W_CB; b++) {
              acc[m][b] = __builtin_fmaf(x4.x, w[b][0], acc[m][b]);
              acc[m][b] = __builtin_fmaf(x4.y, w[b][1], acc[m][b]);
              acc[m][b] = __builtin_fmaf(x4.z, w[b][2], acc[m][b]);
              acc[m][b] = __builtin_fmaf(x4.w, w[b][3], acc[m][b]);
            }
          }
        }
      }
    }
  }
  // K halves (lane l and l + 32), then the waves in order, through LDS
  __syncthreads();                               // every wave is done with xs
  float* red = xs;                               // [4][MB][W_CB * 32]
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int b = 0; b < W_CB; b++) {
      const float o = __shfl_xor(acc[m][b], 32);
      if (h == 0) red[(wave * MB + m) * (W_CB * 32) + b * 32 + lane] = acc[m][b] + o;
    }
  __syncthreads();
  for (int i = threadIdx.x; i < MB * W_CB * 32; i += 256) {
    const int m = i / (W_CB * 32), cc = i % (W_CB * 32);
    const int cb = static_cast<int>(blockIdx.x) * W_CB + cc / 32;
    if (m >= M || cb >= ncb) continue;
    const int st = MB * W_CB * 32;
    const float v = ((red[m * W_CB * 32 + cc] + red[st + m * W_CB * 32 + cc]) + red[2 * st + m * W_CB * 32 + cc]) +
                    red[3 * st + m * W_CB * 32 + cc];
    const long n = static_cast<long>(cb) * 32 + cc % 32;
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
  dim3 grid((a.N / 32 + W_CB - 1) / W_CB, parts), block(256);
  // the part's activations (at most 64 KB by the choice of parts) or the cross-wave reduction
  const size_t shmem = std::max(static_cast<size_t>(rows) * (a.K / parts) * 4, static_cast<size_t>(4 * rows * W_CB * 32 * 4));
#define SVDQ_W(F, MBV)                                                                                                  \
  hipLaunchKernelGGL((w4a16_kernel<F, MBV>), grid, block, shmem, st, a.X, a.M, a.K, a.N, a.inv_lam, a.wcodes, a.wscales, \
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
