// Kernel Q: the fused activation pass of the SVDQuant layer.
//
// One read of X produces (SVDQuant walkthrough, Fig. 6: the down-projection
// and the quantizer consume the same input):
//   x_hat = fp32(x * inv_lambda)                          (eq. (5) smoothing)
//   per token row and K group: absmax scale and 4-bit codes (eq. (1))
//   T = bf16(x_hat) L1b on the bf16 MFMA, fp32 accumulation -> bf16
//
// Work split: a workgroup owns 16 token rows and one of `kparts` equal
// parts of the 128-wide K chunks (the launch splits K so that there are
// about four workgroups per CU: with one workgroup per 16-row block the M
// of a layer would leave most of the chip idle); its NW (4 or 8) waves take
// interleaved chunks of the part.  In a chunk, lane l holds row l % 16 and
// the 32 consecutive K elements 32 * (l / 16) .. + 31, loaded as four
// 16-byte vectors.  An INT4 group (64) is the lane pair (l, l ^ 16); an FP4
// group (32) is one lane.  The 32 values are also the A operands of four
// 16x16x32 bf16 MFMAs (8 consecutive K per MFMA), whose B operands come from
// L1 stored transposed (L1t[t][k]), so the k index sets of A and B match.
// The per-wave partial T tiles are summed across the NW waves in LDS in a
// fixed order; with several K parts each part writes its fp32 partial and
// t_reduce_kernel adds the parts in order and rounds once, so T is
// deterministic.
#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

// Clears the sign of E2M1 codes that encode zero (the hardware conversion
// keeps the sign of a negative value that rounds to zero; the format here
// encodes every zero as +0): for each nibble, bit 3 survives only if one of
// bits 0-2 is set (nibble + 7 carries into bit 3 exactly then, and never into
// the next nibble).
__device__ __forceinline__ uint32_t e2m1_plus_zero(uint32_t w) {
  const uint32_t nz = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;
  return w & (nz | 0x77777777u);
}

// The same for four E4M3 bytes of INT4 codes: bit 7 survives only if one of
// bits 0-6 is set.
__device__ __forceinline__ uint32_t e4m3_plus_zero(uint32_t w) {
  const uint32_t nz = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
  return w & (nz | 0x7F7F7F7Fu);
}

typedef short fp8x2 __attribute__((ext_vector_type(2)));

// x_hat of the 8 elements 8c .. 8c + 7 of a lane's 32 (row `row`, quarter
// kq) from the staged chunk: x * inv_lambda, or with NORM
// fma((x - mu) * rho, gamma', beta') (the staged factors are gamma' then
// beta').  The exact-rounding path recomputes x_hat with this same code.
template <bool NORM>
__device__ __forceinline__ void x_hat8(const uint8_t* xs, const float* ils, int row, int kq, int c, float mu,
                                       float rho, float* out) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(xs + row * 256 + (((4 * kq + c) ^ row) << 4));
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  const f32x4 i0 = *reinterpret_cast<const f32x4*>(ils + kq * 32 + 8 * c);
  const f32x4 i1 = *reinterpret_cast<const f32x4*>(ils + kq * 32 + 8 * c + 4);
  const float f[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
  if constexpr (NORM) {
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(ils + 128 + kq * 32 + 8 * c);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(ils + 128 + kq * 32 + 8 * c + 4);
    const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; e++) out[e] = __builtin_fmaf((x[e] - mu) * rho, f[e], b[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; e++) out[e] = x[e] * f[e];
  }
}

// NORM: X is the input of a LayerNorm whose affine carries the smoothing
// (the norm-fused pass): x_hat = fma((x - mu) * rho, gamma', beta') with the
// row's mean mu and 1/sqrt(var + eps) rho from `rowstat` (two floats per row)
// and inv_lam pointing at gamma' = gamma * inv_lambda (K floats) followed by
// beta' = beta * inv_lambda (K floats).
// HV: 16-row halves per workgroup (1, or 2 for 32-row blocks whose halves
// share every L1 operand load).
template <int FMT, bool QUANT, bool DOWN, int RB, bool NORM, int NW, int HV = 1>
__global__ __launch_bounds__(NW * 64) void act_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                  const float* __restrict__ inv_lam,
                                                  const float* __restrict__ rowstat,
                                                  const uint16_t* __restrict__ l1op,
                                                  uint8_t* __restrict__ codes,
                                                  void* __restrict__ scales,
                                                  uint16_t* __restrict__ Tb, int kparts,
                                                  float* __restrict__ tpart) {
  constexpr int R = RB * 16;
  constexpr bool LR = DOWN && RB > 0;
  // per wave: the 16 x 128 bf16 X chunk (4 KB, rows of 256 B whose 16-byte
  // pieces are XOR-swizzled by the row index) and the chunk's 128 inverse
  // smoothing factors (512 B; NORM: 128 gamma' then 128 beta'); after the
  // loop the same memory holds the cross-wave T reduction
  constexpr int WSTAGE = 4096 * HV + (NORM ? 1024 : 512);
  constexpr int LDS_BYTES = (LR && NW * 64 * R * HV > NW * WSTAGE) ? NW * 64 * R * HV : NW * WSTAGE;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int row = lane & 15;
  const int kq = lane >> 4;
  const int rblk = static_cast<int>(blockIdx.x) / kparts, part = static_cast<int>(blockIdx.x) - rblk * kparts;
  const long row0 = static_cast<long>(rblk) * 16 * HV;
  const int nrows = static_cast<int>(min(static_cast<long>(M) - row0, 16L * HV));
  const int cpp = (K >> 7) / kparts;              // chunks per part (kparts divides K / 128)
  const int c_end = (part + 1) * cpp;
  uint8_t* xs = lds + wave * WSTAGE;             // this wave's X chunk (per half 4 KB)
  const float* ils = reinterpret_cast<const float*>(xs + 4096 * HV);
  const uint32_t rowb = static_cast<uint32_t>(K) * 2;

  // Buffer resources of the workgroup's rows: X (rows past M read as 0; their
  // results are not stored), codes and scales; L1 and the inverse factors.
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X) + row0 * K, 0, static_cast<int>(static_cast<uint32_t>(nrows) * rowb), 0x00020000);
  const __amdgpu_buffer_rsrc_t ir =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(inv_lam), 0, (NORM ? 2 : 1) * K * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(l1op), 0, static_cast<int>(static_cast<uint32_t>(K) * R * 2), 0x00020000);
  // the workgroup's rows lie in one 32-row block of the code and FP4 scale layouts
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      codes + (row0 >> 5) * (K >> 6) * 1024, 0, (K >> 6) * 1024, 0x00020000);
  // (both scale layouts give each 32-row block and 128-wide stage 128 bytes)
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<uint8_t*>(scales) + (row0 >> 5) * (K >> 7) * 128, 0, (K >> 7) * 128, 0x00020000);
  // the lane's row within its 32-row block, and whether it exists, per half
  int r32[HV];
  bool valid[HV];
#pragma unroll
  for (int h = 0; h < HV; h++) {
    r32[h] = static_cast<int>(row0 & 31) + 16 * h + row;
    valid[h] = row0 + 16 * h + row < M;
  }
  // store offsets past the end of cr / sr: such stores write nothing
  const uint32_t c_oob = static_cast<uint32_t>(K >> 6) * 1024;
  const uint32_t s_oob = static_cast<uint32_t>(K >> 7) * 128;

  f32x4 acc[HV][LR ? RB : 1];
#pragma unroll
  for (int h = 0; h < HV; h++)
#pragma unroll
    for (int nb = 0; nb < (LR ? RB : 1); nb++) acc[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads are row-contiguous: load c of a lane takes the 16-byte piece l % 16
  // of row 4c + l / 16 (four whole 256-byte rows per instruction), and lane
  // l < 32 takes inverse factors 4l .. 4l + 3.  The next chunk of the wave is
  // requested before the current one is processed.
  const int lrow = lane >> 4, piece = lane & 15;
  const uint32_t xoff = static_cast<uint32_t>(lrow) * rowb + piece * 16;
  const uint32_t ioff = static_cast<uint32_t>(lane & 31) * 16 + (NORM && lane >= 32 ? static_cast<uint32_t>(K) * 4 : 0u);
  // NORM: the row's mean and reciprocal standard deviation
  float mu[HV], rho[HV];
#pragma unroll
  for (int h = 0; h < HV; h++) {
    mu[h] = 0.f;
    rho[h] = 0.f;
    if constexpr (NORM) {
      const long sr_row = min(row0 + 16 * h + row, static_cast<long>(M - 1));
      mu[h] = rowstat[2 * sr_row];
      rho[h] = rowstat[2 * sr_row + 1];
    }
  }
  // Two chunks of each wave are in flight while it processes a third (one
  // with two halves): chunk it + PFD NW is requested into the registers
  // chunk it arrived in, right after they are staged.
  const int it0 = part * cpp + wave;
  const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
  u32x4 xa[HV][4], xb[HV][4];
#pragma unroll
  for (int h = 0; h < HV; h++)
#pragma unroll
    for (int c = 0; c < 4; c++) xa[h][c] = xb[h][c] = z4;
  u32x4 ia = z4, ib = z4;
  // Every fetch is issued, also past the part's last chunk: there its offset
  // lies past the buffer's end, so it reads nothing and returns zeros.  The
  // compiler then counts the same number of loads in flight on every path and
  // its waits for the L1 operands never include a prefetch.
  const int x_oob = nrows * static_cast<int>(rowb), i_oob = (NORM ? 2 : 1) * K * 4;
  auto fetch = [&](int c0, u32x4 (&x)[HV][4], u32x4& iv) __attribute__((always_inline)) {
    const bool ok = c0 < c_end;
#pragma unroll
    for (int h = 0; h < HV; h++)
#pragma unroll
      for (int c = 0; c < 4; c++)
        x[h][c] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, xoff, ok ? static_cast<int>((16 * h + 4 * c) * rowb + c0 * 256) : x_oob, 0);
    iv = __builtin_amdgcn_raw_buffer_load_b128(ir, ioff, ok ? c0 * 512 : i_oob, 0);
  };
  // chunks requested ahead: two (one half), or one (two halves: the same
  // bytes in flight, half the prefetch registers)
  constexpr int PFD = HV == 1 ? 2 : 1;
  fetch(it0, xa, ia);
  if constexpr (PFD == 2) fetch(it0 + NW, xb, ib);
  auto body = [&](int it, u32x4 (&x)[HV][4], u32x4& iv) __attribute__((always_inline)) {
    const int kb = it * 128 + kq * 32;
    // stage the chunk: piece p of row r goes to slot p ^ r of the row, so
    // that both these writes and the reads below touch 16 distinct 16-byte
    // bank groups per 16 lanes
#pragma unroll
    for (int h = 0; h < HV; h++)
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const int r = 4 * c + lrow;
        *reinterpret_cast<u32x4*>(xs + h * 4096 + r * 256 + ((piece ^ r) << 4)) = x[h][c];
      }
    if (NORM || lane < 32) *reinterpret_cast<u32x4*>(xs + 4096 * HV + lane * 16) = iv;
    // L1 operands of the chunk: one contiguous 1 KB block per (t block,
    // step), requested before the X prefetch (for up to 4 t blocks; wider
    // ranks load them next to their MFMAs).  The INT4 quantizer needs many
    // registers, so for INT4 the down-projection's MFMAs run before the
    // quantization and the L1 operands are dead by then.
    constexpr bool LT_EARLY = LR && RB <= 4;
    constexpr bool MFMA_FIRST = FMT == SVDQ_INT4_G64_FP16;
    const int lbase = it * RB * 4096;
    auto lt_load = [&](int nb, int j) __attribute__((always_inline)) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(lr, static_cast<uint32_t>(lane) * 16, lbase + (nb * 4 + j) * 1024, 0);
      return __builtin_bit_cast(bf16x8, v);
    };
    bf16x8 lt[LT_EARLY ? RB : 1][4];
    if constexpr (LT_EARLY) {
#pragma unroll
      for (int nb = 0; nb < RB; nb++)
#pragma unroll
        for (int j = 0; j < 4; j++) lt[nb][j] = lt_load(nb, j);
    }
    // The X prefetch is issued after the L1 loads: vector memory counters
    // complete in issue order, so waiting for the L1 operands does not wait
    // for the prefetch.
    fetch(it + PFD * NW, x, iv);
    // each half of the workgroup's rows in turn (the L1 operands above serve both)
#pragma unroll
    for (int h = 0; h < HV; h++) {
      // lane (row, kq): elements kq * 32 .. + 31 of its row = pieces 4 kq .. 4 kq + 3
      float xh[32];
#pragma unroll
      for (int c = 0; c < 4; c++) x_hat8<NORM>(xs + h * 4096, ils, row, kq, c, mu[h], rho[h], xh + 8 * c);

      // bf16 of x_hat, rounded to nearest even (v_cvt_pk_bf16_f32): the A
      // operands of the down-projection, formed before the quantizer reuses xh
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      bf16x8 a[LR ? 4 : 1];
      if constexpr (LR) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const bf16x2 p2 = __builtin_convertvector(f32x2{xh[8 * j + e], xh[8 * j + e + 1]}, bf16x2);
            a[j][e] = p2[0];
            a[j][e + 1] = p2[1];
          }
      }

      auto down = [&]() __attribute__((always_inline)) {
        if constexpr (LR) {
#pragma unroll
          for (int nb = 0; nb < RB; nb++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
              if constexpr (LT_EARLY) acc[h][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], lt[nb][j], acc[h][nb], 0, 0, 0);
              else acc[h][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], lt_load(nb, j), acc[h][nb], 0, 0, 0);
            }
        }
      };
      if constexpr (MFMA_FIRST) down();

      if constexpr (QUANT) {
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 32; e++) amax = fmaxf(amax, __builtin_fabsf(xh[e]));
        uint32_t packed[4] = {0u, 0u, 0u, 0u};
        if constexpr (FMT == SVDQ_INT4_G64_FP16) {
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          // s = fp16(A / 7), saturated at the largest finite fp16 value
          const __half sh = __float2half_rn(fminf(amax / 7.0f, 65504.0f));
          const float s = __half2float(sh);
          const float r = s > 0.f ? 1.0f / s : 0.f;
          // t = x / s with one rounding (the product with the rounded
          // reciprocal) is within 2^-20 of the exact quotient, so rint(t) is
          // RNE(x / s) unless t lies within 2^-18 of a half-integer; a lane
          // with such a value redoes its 32 quotients exactly.  (s = 0 gives
          // r = 0 and all-zero codes.)
          float dmax = 0.f;
#pragma unroll
          for (int e = 0; e < 32; e++) {
            const float t = xh[e] * r;
            const float q = __builtin_rintf(t);
            dmax = fmaxf(dmax, __builtin_fabsf(t - q));
            xh[e] = q;
          }
          if (dmax > 0.5f - 0x1p-18f) {
            // xh holds rint(t) now: recompute x from the staged chunk
#pragma unroll
            for (int c = 0; c < 4; c++) {
              float xv[8];
              x_hat8<NORM>(xs + h * 4096, ils, row, kq, c, mu[h], rho[h], xv);
#pragma unroll
              for (int e = 0; e < 8; e++) xh[8 * c + e] = rne_quotient(xv[e], s, r);
            }
          }
          // codes (sign-magnitude, the E4M3 bits of q * 2^-9; the format's
          // word layout): the hardware conversion of clamp(q, -7, 7) / 2^9
          // (exact: |q| <= 7 are E4M3 subnormals), zeros made +0, then the
          // bytes of codes 4-7 of each word rotated left by 4 bits over those
          // of codes 0-3
#pragma unroll
          for (int w = 0; w < 4; w++) {
            uint32_t d[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
              const float* qv = xh + 8 * w + 4 * h;
              fp8x2 v = {0, 0};
              v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, __builtin_amdgcn_fmed3f(qv[0], -7.0f, 7.0f),
                                                           __builtin_amdgcn_fmed3f(qv[1], -7.0f, 7.0f), 512.0f, false);
              v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, __builtin_amdgcn_fmed3f(qv[2], -7.0f, 7.0f),
                                                           __builtin_amdgcn_fmed3f(qv[3], -7.0f, 7.0f), 512.0f, true);
              d[h] = e4m3_plus_zero(__builtin_bit_cast(uint32_t, v));
            }
            packed[w] = d[0] | __builtin_amdgcn_alignbit(d[1], d[1], 28);
          }
          // INT4 scale block order within the 32-row block (the 4-byte word of
          // row r32[h] holds the stage's two groups); rows past M and the odd lane
          // of each pair store past the buffer's end: no write
          __builtin_amdgcn_raw_buffer_store_b16(
              __half_as_ushort(sh), sr,
              valid[h] && (kq & 1) == 0 ? static_cast<uint32_t>((kb >> 7) * 128 + r32[h] * 4 + ((kb >> 6) & 1) * 2) : s_oob, 0, 0);
        } else {
          // E2M1 of x / 2^ex, rounded to nearest even by the conversion
          // instruction (|x / 2^ex| <= 6 by the choice of ex), two codes per
          // instruction into byte e / 2 % 4 of word e / 8.  Groups whose scale
          // is below 2^-120 (absmax under ~5e-36, all-zero groups included)
          // take the exact bit-level rounding instead, so that no denormal
          // scale or input reaches the conversion.
          const int ex = e8m0_exponent(amax);
          if (ex >= -120) {
            const float sc = __builtin_amdgcn_ldexpf(1.0f, ex);
#pragma unroll
            for (int w = 0; w < 4; w++) {
              uint32_t v = 0u;
              v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[8 * w + 0], xh[8 * w + 1], sc, 0);
              v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[8 * w + 2], xh[8 * w + 3], sc, 1);
              v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[8 * w + 4], xh[8 * w + 5], sc, 2);
              v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, xh[8 * w + 6], xh[8 * w + 7], sc, 3);
              packed[w] = e2m1_plus_zero(v);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 32; e++)
              packed[e >> 3] |= e2m1_code(__builtin_amdgcn_ldexpf(xh[e], -ex)) << (4 * (e & 7));
          }
          // FP4 scale block order within the 32-row block (fp4_scale_offset)
          __builtin_amdgcn_raw_buffer_store_b8(
              static_cast<uint8_t>(ex + 127), sr,
              valid[h] ? static_cast<uint32_t>((kb >> 7) * 128 + (r32[h] + 32 * ((kb >> 5) & 1)) * 2 + ((kb >> 6) & 1)) : s_oob, 0, 0);
        }
        // code block order within the 32-row block (code_chunk_offset)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{packed[0], packed[1], packed[2], packed[3]}, cr,
            valid[h] ? static_cast<uint32_t>((kb >> 6) * 1024 + (r32[h] + 32 * ((kb >> 5) & 1)) * 16) : c_oob, 0, 0);
      }

      if constexpr (!MFMA_FIRST) down();
    }
  };
  int it = it0;
  if constexpr (PFD == 2) {
    for (; it + NW < c_end; it += 2 * NW) {
      body(it, xa, ia);
      body(it + NW, xb, ib);
    }
    if (it < c_end) body(it, xa, ia);
  } else {
    for (; it < c_end; it += NW) body(it, xa, ia);
  }

  if constexpr (LR) {
    // acc[h][nb][v] is this wave's partial T[16 h + 4 kq + v][nb * 16 +
    // (lane & 15)]; the staging memory is reused once every wave has left
    // the loop
    float* red = reinterpret_cast<float*>(lds);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HV; h++)
#pragma unroll
      for (int nb = 0; nb < RB; nb++)
#pragma unroll
        for (int v = 0; v < 4; v++) red[((wave * HV + h) * 16 + 4 * kq + v) * R + nb * 16 + row] = acc[h][nb][v];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * HV * R; idx += NW * 64) {
      const int rr = idx / R, t = idx % R;
      float s = red[rr * R + t];
#pragma unroll
      for (int w = 1; w < NW; w++) s += red[(w * 16 * HV + rr) * R + t];
      const long gr = row0 + rr;
      if (gr < M) {
        if (kparts == 1) Tb[bf16_block_index(gr, t, R)] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else tpart[(static_cast<long>(part) * M + gr) * R + t] = s;
      }
    }
  }
}

// T = sum over the K parts (in part order) of the fp32 partials, rounded once
// to bf16 into the block layout; one thread per 4 consecutive elements of a
// row < M (R % 16 == 0, so the 4 are contiguous in the block layout too).
__global__ __launch_bounds__(256) void t_reduce_kernel(const float* __restrict__ tpart, int kparts, int M, int R,
                                                       uint16_t* __restrict__ Tb) {
  const long idx = (static_cast<long>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const long n = static_cast<long>(M) * R;
  if (idx >= n) return;
  const long row = idx / R;
  const int t = static_cast<int>(idx - row * R);
  // all loads first, unconditionally (parts past kparts lie past the buffer
  // resource's end and read as zeros), then the sum in part order
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(tpart), 0, static_cast<int>(static_cast<uint32_t>(kparts) * static_cast<uint32_t>(n) * 4), 0x00020000);
  f32x4 v[kMaxKParts];
#pragma unroll
  for (int p = 0; p < kMaxKParts; p++)
    v[p] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, static_cast<uint32_t>(idx) * 4, static_cast<int>(p * n * 4), 0));
  f32x4 s = v[0];
#pragma unroll
  for (int p = 1; p < kMaxKParts; p++) s += v[p];
  const uint32_t lo = f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16);
  const uint32_t hi = f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2*>(Tb + bf16_block_index(row, t, R)) = u32x2{lo, hi};
}

// K parts: balances the bytes each CU streams.  With d parts, the
// ceil(row blocks * d / CUs) workgroups of the busiest CU each carry 1/d of a
// row block's K; the waves of a workgroup share its chunks, so a chunk count
// that is not a multiple of 4 leaves some idle; each part adds an fp32
// partial T write and read (about 2% each).  d divides K / 128 and is at most
// kMaxKParts.  Without a partial-T buffer (or for M above kSplitMaxM, where
// the workspace holds none) a pass with a down-projection runs in one part.
// The FP4 pass (light per-element work) over short rows (K <= 4096) with at
// most two row blocks per CU also runs unsplit: there the reduction launch
// costs more than the split gains (measured, 4608 x 3072 FP4: 11.6 us in one
// part against 10.1 us split plus a 4.7 us reduction).
static int choose_kparts(int M, int K, bool down, bool have_tpart, bool fp4) {
  if (down && (!have_tpart || M > kSplitMaxM)) return 1;
  const int nchunks = K >> 7, nrb = (M + 15) / 16;
  const long cus = device_cu_count();
  if (down && fp4 && K <= 4096 && nrb <= 2 * cus) return 1;
  int best = 1;
  double best_cost = 0.0;
  for (int d = 1; d <= kMaxKParts; d++) {
    if (nchunks % d) continue;
    const int cpp = nchunks / d;
    const double per_cu = static_cast<double>((static_cast<long>(nrb) * d + cus - 1) / cus) / d;
    const double waves = static_cast<double>((cpp + 3) / 4) / (cpp / 4.0);
    const double cost = per_cu * waves * (1.0 + (down ? 0.02 * (d - 1) : 0.0));
    if (d == 1 || cost < best_cost) {
      best = d;
      best_cost = cost;
    }
  }
  return best;
}

template <int FMT, bool QUANT, bool DOWN, bool NORM>
static hipError_t launch_act_rb(int rb, const ActArgs& a, hipStream_t st) {
  int kparts = choose_kparts(a.M, a.K, DOWN && rb > 0, a.tpart != nullptr, FMT == SVDQ_FP4_E2M1_G32_E8M0);
  // One or two row blocks per CU over a short K: eight waves per workgroup
  // share a row block's chunks instead of splitting its K over workgroups,
  // so the down-projection needs no second (reduction) launch and each CU
  // still has enough loads in flight.
  const long nrb = (a.M + 15) / 16, cus = device_cu_count();
  const bool wide = DOWN && rb > 0 && nrb >= cus && nrb <= 2 * cus && (a.K >> 7) <= 32;
  if (wide) kparts = 1;
  // More row blocks than CUs: 32-row workgroups instead (one round; each L1
  // operand load serves both halves, so the busiest CU moves a third fewer
  // bytes than with two 16-row blocks).  Up to rank 32, and not for the
  // INT4 norm-fused form: those do not fit the registers twice.
  constexpr bool PAIR_OK = !(NORM && FMT == SVDQ_INT4_G64_FP16);
  const bool pair = PAIR_OK && wide && nrb > cus && rb <= 2;
  dim3 grid(static_cast<unsigned>(pair ? (nrb + 1) / 2 : nrb * kparts)), block(wide ? 512 : 256);
#define SVDQ_ACT_CASE(RBV)                                                                                        \
  case RBV:                                                                                                     \
    if constexpr (PAIR_OK) {                                                                                    \
      if (pair) {                                                                                               \
        hipLaunchKernelGGL((act_kernel<FMT, QUANT, DOWN, (RBV <= 2 ? RBV : 2), NORM, 8, 2>), grid, block, 0, st, \
                           a.X, a.M, a.K, a.inv_lam, a.rowstat, a.l1t, a.codes, a.scales, a.Tb, kparts, a.tpart); \
        break;                                                                                                  \
      }                                                                                                         \
    }                                                                                                           \
    if (wide)                                                                                                   \
      hipLaunchKernelGGL((act_kernel<FMT, QUANT, DOWN, RBV, NORM, 8>), grid, block, 0, st, a.X, a.M, a.K, a.inv_lam, \
                         a.rowstat, a.l1t, a.codes, a.scales, a.Tb, kparts, a.tpart);                           \
    else                                                                                                        \
      hipLaunchKernelGGL((act_kernel<FMT, QUANT, DOWN, RBV, NORM, 4>), grid, block, 0, st, a.X, a.M, a.K, a.inv_lam, \
                         a.rowstat, a.l1t, a.codes, a.scales, a.Tb, kparts, a.tpart);                           \
    break;
  switch (rb) {
    SVDQ_ACT_CASE(0) SVDQ_ACT_CASE(1) SVDQ_ACT_CASE(2) SVDQ_ACT_CASE(3) SVDQ_ACT_CASE(4)
    SVDQ_ACT_CASE(5) SVDQ_ACT_CASE(6) SVDQ_ACT_CASE(7) SVDQ_ACT_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_ACT_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !DOWN || rb == 0 || kparts == 1) return e;
  const long n4 = static_cast<long>(a.M) * rb * 4;   // groups of 4 elements
  hipLaunchKernelGGL(t_reduce_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st, a.tpart, kparts,
                     a.M, rb * 16, a.Tb);
  return hipGetLastError();
}

hipError_t launch_act(int fmt, bool quant, bool down, const ActArgs& a, hipStream_t st) {
  const int rb = down ? a.rank / 16 : 0;
  if (a.rowstat) {
    // the norm-fused pass exists with quantization (and the down-projection
    // where the layer has a rank)
    if (!quant) return hipErrorInvalidValue;
    if (fmt == SVDQ_INT4_G64_FP16)
      return down ? launch_act_rb<SVDQ_INT4_G64_FP16, true, true, true>(rb, a, st)
                  : launch_act_rb<SVDQ_INT4_G64_FP16, true, false, true>(0, a, st);
    return down ? launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, true, true, true>(rb, a, st)
                : launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, true, false, true>(0, a, st);
  }
  if (fmt == SVDQ_INT4_G64_FP16) {
    if (quant && down) return launch_act_rb<SVDQ_INT4_G64_FP16, true, true, false>(rb, a, st);
    if (quant) return launch_act_rb<SVDQ_INT4_G64_FP16, true, false, false>(0, a, st);
    return launch_act_rb<SVDQ_INT4_G64_FP16, false, true, false>(rb, a, st);
  }
  if (quant && down) return launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, true, true, false>(rb, a, st);
  if (quant) return launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, true, false, false>(0, a, st);
  return launch_act_rb<SVDQ_FP4_E2M1_G32_E8M0, false, true, false>(rb, a, st);
}

// Row statistics of the norm-fused pass: blocks below ceil(M / 4) give each
// wave one row: mu = (sum x) / K and rho = 1 / sqrt((sum (x - mu)^2) / K + eps),
// fp32 sums over the 16-byte vectors lane, lane + 64, ... of each lane, in
// that order, then a fixed butterfly across the wave; the remaining blocks
// fold the smoothing into the norm's affine: gamma'[k] = gamma[k] *
// inv_lambda[k], beta'[k] = beta[k] * inv_lambda[k] (beta = 0 when absent),
// each rounded once to fp32.  With NV > 0 (K <= 512 NV) a lane holds its NV
// vectors of the row in registers: every load of the row is issued at once
// and X is read from HBM once; NV = 0 streams the row twice (any K).
__device__ __forceinline__ float vsum8(const u32x4 v) {
  return bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) + bf16_hi(v.z) + bf16_lo(v.w) +
         bf16_hi(v.w);
}

__device__ __forceinline__ float vdev8(const u32x4 v, float mu, float q) {
  const float d[8] = {bf16_lo(v.x) - mu, bf16_hi(v.x) - mu, bf16_lo(v.y) - mu, bf16_hi(v.y) - mu,
                      bf16_lo(v.z) - mu, bf16_hi(v.z) - mu, bf16_lo(v.w) - mu, bf16_hi(v.w) - mu};
#pragma unroll
  for (int e = 0; e < 8; e++) q = __builtin_fmaf(d[e], d[e], q);
  return q;
}

template <int NV>
__global__ __launch_bounds__(256) void norm_stats_kernel(const uint16_t* __restrict__ X, int M, int K, float eps,
                                                         const uint16_t* __restrict__ gamma,
                                                         const uint16_t* __restrict__ beta,
                                                         const float* __restrict__ inv_lam, float* __restrict__ rowstat,
                                                         float* __restrict__ fold) {
  const int row_blocks = (M + 3) / 4;
  if (static_cast<int>(blockIdx.x) >= row_blocks) {
    const int k = (static_cast<int>(blockIdx.x) - row_blocks) * 256 + static_cast<int>(threadIdx.x);
    if (k < K) {
      const float inv = inv_lam[k];
      fold[k] = __uint_as_float(static_cast<uint32_t>(gamma[k]) << 16) * inv;
      fold[K + k] = beta ? __uint_as_float(static_cast<uint32_t>(beta[k]) << 16) * inv : 0.f;
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const long r = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= M) return;
  const u32x4* xr = reinterpret_cast<const u32x4*>(X + r * K);
  const int nv = K / 8;                          // 16-byte vectors per row
  float s = 0.f, q = 0.f;
  if constexpr (NV > 0) {
    u32x4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int i = lane + 64 * j;
      v[j] = i < nv ? xr[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NV; j++)
      if (lane + 64 * j < nv) s += vsum8(v[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    const float mu = s / static_cast<float>(K);
#pragma unroll
    for (int j = 0; j < NV; j++)
      if (lane + 64 * j < nv) q = vdev8(v[j], mu, q);
  } else {
    for (int i = lane; i < nv; i += 64) s += vsum8(xr[i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    const float mu = s / static_cast<float>(K);
    for (int i = lane; i < nv; i += 64) q = vdev8(xr[i], mu, q);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o);
  if (lane == 0) {
    rowstat[2 * r] = s / static_cast<float>(K);
    rowstat[2 * r + 1] = 1.0f / __builtin_sqrtf(q / static_cast<float>(K) + eps);
  }
}

hipError_t launch_norm_stats(const uint16_t* X, int M, int K, float eps, const uint16_t* gamma, const uint16_t* beta,
                             const float* inv_lam, float* rowstat, float* fold, hipStream_t st) {
  const int blocks = (M + 3) / 4 + (K + 255) / 256;
  const int per_lane = (K / 8 + 63) / 64;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, st, X, M, K, eps, gamma, beta, inv_lam, rowstat, fold);
  };
  if (per_lane <= 2) go(norm_stats_kernel<2>);
  else if (per_lane <= 4) go(norm_stats_kernel<4>);
  else if (per_lane <= 6) go(norm_stats_kernel<6>);
  else if (per_lane <= 8) go(norm_stats_kernel<8>);
  else if (per_lane <= 12) go(norm_stats_kernel<12>);
  else if (per_lane <= 16) go(norm_stats_kernel<16>);
  else if (per_lane <= 24) go(norm_stats_kernel<24>);
  else if (per_lane <= 32) go(norm_stats_kernel<32>);
  else go(norm_stats_kernel<0>);
  return hipGetLastError();
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
