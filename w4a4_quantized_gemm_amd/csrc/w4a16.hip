// The weight-only 4-bit layer (16-bit activations) for small M: the
// [diffusers] page's second operator, next to the W4A4 one, for the
// adaptive-norm and modulation projections (a handful of rows).
//
//   x_hat = fp32(x * inv_lambda)            (the layer's smoothing, not quantized)
//   Y     = round(x_hat dequant(Q(R)) + b)  (R = W_hat: a prepared layer of rank 0)
//
// Memory-bound: the 4-bit weights (K N / 2 bytes) are read once, the
// activations are a few KB.  The product runs on the bf16 matrix cores with
// exact products and fp32 accumulation:
//
//  * every x_hat value is cut into three bf16 pieces, x_hat = hi + mid + lo
//    exactly (each piece the leading 8 significant bits of what the previous
//    ones leave: truncation leaves at most 16, then at most 8 bits), and
//    every 4-bit weight is exact in bf16 (INT4: the E4M3 code byte m 2^-9,
//    its fp16 scale applied in fp32 per 64-group; FP4: the E2M1 value times
//    its power-of-two scale), so each MFMA product is exact;
//  * a 32 x 32 x 16 MFMA takes 32 A rows: the pieces of up to 8 token rows
//    fill rows 0-7 (hi), 8-15 (mid), 16-23 (lo) of one operand; up to 16
//    rows take two operands ([hi | mid], [lo | 0]); the output row of a
//    token is the sum of its pieces' rows, added once at the end.
//
// Where the pieces of all of x_hat fit in LDS (3 M K bf16 within 144 KB: up
// to 8 rows at K = 3072) a workgroup computes them itself before its loop:
// one launch.  Otherwise w4a16_split_kernel writes them once into the
// workspace, already in the MFMA A-operand order (1 KB per K step of 16 and
// operand, 64 lanes x 16 bytes), and the workgroups load them from there.
// Either way the K order inside a 64-block is permuted so that lane half h
// of K step s holds K = 32 h + 8 s + 0..7, the order of the weight codes'
// 16-byte lane slots.  A workgroup of 8 waves owns CBW 32-column blocks and
// all of K: wave w takes the 64-blocks kb = w, w + 8, .. and all CBW column
// blocks of each (one A operand serves CBW MFMA chains), with up to six
// blocks of weights in flight; the eight waves' partial sums are added in
// wave order through LDS, so the result is deterministic.  The weight
// scales of the workgroup's column blocks (one contiguous run of CBW K
// bytes in both formats) are copied into LDS once, so the loop's only
// gathers are gone (up to K = 4096 at three blocks).
#include <algorithm>

#include "svdq_device.h"
#include "svdq_internal.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int XW = 8;        // waves per workgroup of the weight-streaming kernel
constexpr int XPF = 2;       // 64-blocks in flight per wave (A operands from the workspace)
constexpr int XDEPTH = 6;    // 64-blocks in flight per wave (A operands in LDS)
constexpr int W_LDS = 147456;  // LDS of the in-LDS form: 3 M K bf16 pieces (M = 8, K = 3072 fit)
constexpr int S_LDS = 12288;   // the workgroup's weight scales (CBW K bytes) staged in LDS up to this size

// bf16 bits of piece p (0 hi, 1 mid, 2 lo) of x: x = hi + mid + lo exactly
// for finite x (fp32 subnormal remainders aside); a non-finite x is carried
// by hi alone (a NaN keeps a set mantissa bit).
__device__ __forceinline__ uint32_t piece_bits(float x, int p) {
  const uint32_t xb = __float_as_uint(x);
  if ((xb & 0x7F800000u) == 0x7F800000u) return p == 0 ? ((xb >> 16) | ((xb & 0x7FFFFFu) ? 0x40u : 0u)) : 0u;
  const uint32_t hi = xb & 0xFFFF0000u;
  if (p == 0) return hi >> 16;
  const float r1 = x - __uint_as_float(hi);                 // exact: x's low 16 significand bits
  const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
  if (p == 1) return mid >> 16;
  return __float_as_uint(r1 - __uint_as_float(mid)) >> 16;  // exact and at most 8 significant bits
}
}  // namespace

// A-operand slot of (64-block kb, K step s, operand o, lane): 16 bytes, the
// bf16 pieces of a token row's x_hat at K = 64 kb + 32 (lane / 32) + 8 s + 0..7.
// Row r = lane % 32 of operand o holds: nop == 1: piece r / 8 of token row
// r % 8 (r >= 24: zero); nop == 2: o == 0: hi (r < 16) or mid (r >= 16) of
// token row r % 16, o == 1: lo of token row r (r < 16), zero above.  Token
// rows >= M are zero.
__global__ __launch_bounds__(256) void w4a16_split_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                          const float* __restrict__ inv_lam, int nop,
                                                          u32x4* __restrict__ A) {
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  const long total = static_cast<long>(K / 64) * 4 * nop * 64;
  if (idx >= total) return;
  const int lane = static_cast<int>(idx & 63);
  const long q = idx >> 6;
  const int o = static_cast<int>(q % nop), s = static_cast<int>((q / nop) & 3);
  const long kb = q / (nop * 4);
  const int r = lane & 31, h = lane >> 5;
  int p, m;
  if (nop == 1) {
    p = r >> 3;
    m = r & 7;
  } else {
    m = r & 15;
    p = o == 0 ? (r >> 4) : (r < 16 ? 2 : 3);
  }
  u32x4 out = u32x4{0u, 0u, 0u, 0u};
  if (p < 3 && m < M) {
    const long k0 = kb * 64 + 32 * h + 8 * s;
    const u32x4 xv = *reinterpret_cast<const u32x4*>(X + static_cast<long>(m) * K + k0);
    const f32x4 l0 = *reinterpret_cast<const f32x4*>(inv_lam + k0);
    const f32x4 l1 = *reinterpret_cast<const f32x4*>(inv_lam + k0 + 4);
    const float lam[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float a = bf16_lo(xw[j]) * lam[2 * j];         // x_hat = fp32(x * inv_lambda)
      const float b = bf16_hi(xw[j]) * lam[2 * j + 1];
      pk[j] = piece_bits(a, p) | (piece_bits(b, p) << 16);
    }
    out = u32x4{pk[0], pk[1], pk[2], pk[3]};
  }
  A[idx] = out;
}

// The weight-streaming kernel.  LDSA: the pieces of all of x_hat sit in
// LDS (3 M K bf16, [piece][row][K]), computed by the workgroup itself from
// X before its loop -- one launch, and the only vector-memory loads in the
// loop are the weights, so DEPTH 64-blocks of them stay in flight per wave
// (vector loads complete in issue order: A operands loaded next to the
// weights would make every wait for them a wait for the whole prefetch).
// Otherwise the A operands come from w4a16_split_kernel's workspace, two
// blocks ahead together with the weights.
// SCL: the scales of the workgroup's CBW column blocks (K bytes per block in
// both formats, contiguous) are copied into LDS once with 16-byte loads and
// read from there; otherwise every lane loads its column's scale per block,
// a gather over 32 cache lines per instruction (most of the loop's cache
// traffic by request count, next to 1 KB of weights per instruction).
template <int FMT, int NOP, int CBW, bool LDSA, bool SCL>
__global__ __launch_bounds__(XW * 64) void w4a16_kernel(const u32x4* __restrict__ A, const uint16_t* __restrict__ X,
                                                        const float* __restrict__ inv_lam, int M, int K, int N,
                                                        const uint8_t* __restrict__ wcodes,
                                                        const void* __restrict__ wscales,
                                                        const float* __restrict__ bias, void* __restrict__ Y,
                                                        int out_f32) {
  constexpr int NV = NOP == 2 ? 8 : 4;       // output values per lane and column block
  constexpr int PF = LDSA ? XDEPTH : XPF;    // 64-blocks in flight per wave
  constexpr int NA = LDSA ? 1 : 4 * NOP;     // A operands held per prefetch slot
  // LDSA: the pieces, then (after the loop) the waves' partial sums
  // [wave][column block][value][lane]; else only the partial sums
  constexpr int LDS_MAIN = LDSA ? W_LDS : XW * CBW * NV * 64 * 4;
  constexpr int LDS_BYTES = LDS_MAIN + (SCL ? S_LDS : 0);
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  uint8_t* const sl = lds + LDS_MAIN;           // SCL: scales of column block c at c K
  float* const red = reinterpret_cast<float*>(lds);
  const int lane = threadIdx.x & 63, wave = wave_uniform(threadIdx.x >> 6);
  const int h = lane >> 5, r = lane & 31;
  const int KB = K / 64, ncb = N / 32;
  const int cb0 = static_cast<int>(blockIdx.x) * CBW;
  // the lane's column of each block (blocks past the matrix are clamped to
  // its last one and not stored)
  int cbk[CBW], col[CBW];
#pragma unroll
  for (int c = 0; c < CBW; c++) {
    cbk[c] = min(cb0 + c, ncb - 1);
    col[c] = cbk[c] * 32 + r;
  }
  // the A row of operand o of this lane: piece pc[o] of token row mr[o], or
  // nothing (act[o] false: zero)
  bool act[NOP];
  int pc[NOP], mr[NOP];
#pragma unroll
  for (int o = 0; o < NOP; o++) {
    if constexpr (NOP == 1) {
      pc[o] = r >> 3;
      mr[o] = r & 7;
      act[o] = pc[o] < 3 && mr[o] < M;
    } else {
      pc[o] = o == 0 ? (r >> 4) : 2;
      mr[o] = r & 15;
      act[o] = mr[o] < M && (o == 0 || r < 16);
    }
  }
  const int nt = wave < KB ? (KB - wave + XW - 1) / XW : 0;
  const uint32_t a_bytes = static_cast<uint32_t>(KB) * 4u * NOP * 1024u;
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(A), 0, static_cast<int>(a_bytes), 0x00020000);
  const uint32_t c_bytes = static_cast<uint32_t>(ncb) * static_cast<uint32_t>(KB) * 1024u;
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wcodes), 0, static_cast<int>(c_bytes), 0x00020000);
  // scales: INT4 one fp16 per 64-group, FP4 one byte per 32-group: 2 N K / 64 bytes either way
  const uint32_t s_bytes = static_cast<uint32_t>(N) * static_cast<uint32_t>(KB) * 2u;
  const __amdgpu_buffer_rsrc_t sr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wscales), 0, static_cast<int>(s_bytes), 0x00020000);

  // SCL: the scale copy's loads go out first (16 bytes per lane, whole
  // blocks; a block past the matrix repeats the last one)
  constexpr int SC_IT = (S_LDS / 16 + XW * 64 - 1) / (XW * 64);
  u32x4 sv[SCL ? SC_IT : 1];
  const int n16 = CBW * K / 16, k16 = K / 16;
  if constexpr (SCL) {
#pragma unroll
    for (int j = 0; j < SC_IT; j++) {
      const int i = static_cast<int>(threadIdx.x) + j * XW * 64;
      const int c = i / k16;
      sv[j] = __builtin_amdgcn_raw_buffer_load_b128(
          sr, i < n16 ? static_cast<uint32_t>(cbk[min(c, CBW - 1)]) * static_cast<uint32_t>(K) + (i - c * k16) * 16u
                      : s_bytes, 0, 0);
    }
  }
  auto store_scales = [&]() __attribute__((always_inline)) {
    if constexpr (SCL) {
#pragma unroll
      for (int j = 0; j < SC_IT; j++) {
        const int i = static_cast<int>(threadIdx.x) + j * XW * 64;
        if (i < n16) *reinterpret_cast<u32x4*>(sl + i * 16) = sv[j];
      }
    }
  };
  // the scale of the lane's column of block c at 64-block kb
  auto scale_lds = [&](int c, int kb) __attribute__((always_inline)) -> uint32_t {
    if constexpr (FMT == SVDQ_INT4_G64_FP16)
      return *reinterpret_cast<const uint16_t*>(sl + c * K + (r * KB + kb) * 2);
    else
      return sl[c * K + static_cast<int>(fp4_scale_offset(r, kb * 64 + 32 * h, K))];
  };

  u32x4 aq[PF][NA], wq[PF][CBW];
  uint32_t sq[PF][SCL ? 1 : CBW];
  auto fetch = [&](int t, int slot) __attribute__((always_inline)) {
    const int kb = wave + XW * t;
    const bool ok = t < nt;
#pragma unroll
    for (int c = 0; c < CBW; c++) {
      wq[slot][c] = __builtin_amdgcn_raw_buffer_load_b128(
          cr, ok ? (static_cast<uint32_t>(cbk[c]) * KB + kb) * 1024u + lane * 16u : c_bytes, 0, 0);
      if constexpr (SCL) {
      } else if constexpr (FMT == SVDQ_INT4_G64_FP16) {
        sq[slot][c] = __builtin_amdgcn_raw_buffer_load_b16(
            sr, ok ? (static_cast<uint32_t>(col[c]) * KB + kb) * 2u : s_bytes, 0, 0);
      } else {
        sq[slot][c] = __builtin_amdgcn_raw_buffer_load_b8(
            sr, ok ? static_cast<uint32_t>(fp4_scale_offset(col[c], kb * 64 + 32 * h, K)) : s_bytes, 0, 0);
      }
    }
    if constexpr (!LDSA) {
#pragma unroll
      for (int so = 0; so < 4 * NOP; so++)
        aq[slot][so] = __builtin_amdgcn_raw_buffer_load_b128(
            ar, ok && act[so % NOP] ? (static_cast<uint32_t>(kb) * 4u * NOP + so) * 1024u + lane * 16u : a_bytes, 0, 0);
    }
  };

  if constexpr (LDSA) {
    // pieces of x_hat into LDS, 8 consecutive K of one row per item: the
    // first item's loads go out before the weight prefetch (the pieces are
    // computed while the weights stream in), later items' after it
    const int kv = K / 8, nvec = M * kv;
    auto load_item = [&](int v, u32x4& xv, f32x4& l0, f32x4& l1) __attribute__((always_inline)) {
      const int m = v / kv, k = (v - m * kv) * 8;
      xv = *reinterpret_cast<const u32x4*>(X + static_cast<long>(m) * K + k);
      l0 = *reinterpret_cast<const f32x4*>(inv_lam + k);
      l1 = *reinterpret_cast<const f32x4*>(inv_lam + k + 4);
    };
    auto store_item = [&](int v, const u32x4& xv, const f32x4& l0, const f32x4& l1) __attribute__((always_inline)) {
      const int m = v / kv, k = (v - m * kv) * 8;
      const float lam[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      float xh[8];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        xh[2 * j] = bf16_lo(xw[j]) * lam[2 * j];           // x_hat = fp32(x * inv_lambda)
        xh[2 * j + 1] = bf16_hi(xw[j]) * lam[2 * j + 1];
      }
#pragma unroll
      for (int p = 0; p < 3; p++) {
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; j++) pk[j] = piece_bits(xh[2 * j], p) | (piece_bits(xh[2 * j + 1], p) << 16);
        *reinterpret_cast<u32x4*>(lds + ((static_cast<long>(p) * M + m) * K + k) * 2) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      }
    };
    const int v0 = threadIdx.x;
    u32x4 xv;
    f32x4 l0, l1;
    if (v0 < nvec) load_item(v0, xv, l0, l1);
#pragma unroll
    for (int d = 0; d < PF; d++) fetch(d, d);
    store_scales();
    if (v0 < nvec) store_item(v0, xv, l0, l1);
    for (int v = v0 + XW * 64; v < nvec; v += XW * 64) {
      load_item(v, xv, l0, l1);
      store_item(v, xv, l0, l1);
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int d = 0; d < PF; d++) fetch(d, d);
    store_scales();
    if constexpr (SCL) __syncthreads();
  }

  f32x16 acc[CBW];
#pragma unroll
  for (int c = 0; c < CBW; c++)
#pragma unroll
    for (int v = 0; v < 16; v++) acc[c][v] = 0.f;

  for (int t0 = 0; t0 < nt; t0 += PF) {
#pragma unroll
    for (int d = 0; d < PF; d++) {
      const int t = t0 + d;
      u32x4 aslot[NA], w[CBW];
      float sc[CBW];
      if constexpr (!LDSA) {
#pragma unroll
        for (int so = 0; so < NA; so++) aslot[so] = aq[d][so];
      }
#pragma unroll
      for (int c = 0; c < CBW; c++) {
        w[c] = wq[d][c];
        const uint32_t sraw = SCL ? scale_lds(c, min(wave + XW * t, KB - 1)) : sq[d][SCL ? 0 : c];
        if constexpr (FMT == SVDQ_INT4_G64_FP16)
          sc[c] = __half2float(__ushort_as_half(static_cast<uint16_t>(sraw))) * 512.0f;   // s 2^9
        else
          sc[c] = __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(sraw & 0xFFu) - 127);   // 2^e
      }
      fetch(t + PF, d);
      if (t < nt) {
        const int kb = wave + XW * t;
        // A operand o of K step s
        auto a_op = [&](int s, int o) __attribute__((always_inline)) {
          if constexpr (LDSA) {
            const long off = ((static_cast<long>(pc[o]) * M + mr[o]) * K + kb * 64 + 32 * h + 8 * s) * 2;
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (act[o] ? off : 0));
            return act[o] ? v : u32x4{0u, 0u, 0u, 0u};
          } else {
            return aslot[s * NOP + o];
          }
        };
        // INT4: the 64-group's exact partial products first, then its scale
        f32x16 P[CBW];
        if constexpr (FMT == SVDQ_INT4_G64_FP16) {
#pragma unroll
          for (int c = 0; c < CBW; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) P[c][v] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < 4; s++) {
          bf16x8 av[NOP];
#pragma unroll
          for (int o = 0; o < NOP; o++) av[o] = __builtin_bit_cast(bf16x8, a_op(s, o));
#pragma unroll
          for (int c = 0; c < CBW; c++) {
            const uint32_t wd = s == 0 ? w[c].x : s == 1 ? w[c].y : s == 2 ? w[c].z : w[c].w;
            bf16x2 e0, e1, e2, e3;
            if constexpr (FMT == SVDQ_INT4_G64_FP16) {
              // E4M3 code bytes: K 8 s + 0..3 in word & 0x87878787, K 8 s + 4..7 in rotr(word, 4) & 0x87878787
              const uint32_t lo = wd & 0x87878787u;
              const uint32_t hi = __builtin_amdgcn_alignbit(wd, wd, 4) & 0x87878787u;
              e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
              e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
              e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
              e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
            } else {
              // E2M1 pairs, even K in the low nibble: byte b holds K 8 s + 2 b, + 1;
              // the power-of-two scale is exact in bf16
              e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[c], 0);
              e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[c], 1);
              e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[c], 2);
              e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[c], 3);
            }
            const bf16x8 b = bf16x8{e0.x, e0.y, e1.x, e1.y, e2.x, e2.y, e3.x, e3.y};
#pragma unroll
            for (int o = 0; o < NOP; o++) {
              if constexpr (FMT == SVDQ_INT4_G64_FP16)
                P[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[o], b, P[c], 0, 0, 0);
              else
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[o], b, acc[c], 0, 0, 0);
            }
          }
        }
        if constexpr (FMT == SVDQ_INT4_G64_FP16) {
#pragma unroll
          for (int c = 0; c < CBW; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[c][v] = __builtin_fmaf(P[c][v], sc[c], acc[c][v]);
        }
      }
    }
  }
  // Lane l, value v of an accumulator is A row 8 (v / 4) + 4 (l / 32) + v % 4
  // of output column l % 32.  Token row of value u: nop == 2: u < 8 is row
  // 8 (u / 4) + 4 h + u % 4, the sum of values u (hi + lo) and u + 8 (mid);
  // nop == 1: row 4 h + u, the sum of values u (hi), u + 4 (mid), u + 8 (lo).
  if constexpr (LDSA) __syncthreads();          // every wave is done with the pieces
#pragma unroll
  for (int c = 0; c < CBW; c++)
#pragma unroll
    for (int u = 0; u < NV; u++) {
      const float y = NOP == 2 ? acc[c][u] + acc[c][u + 8] : (acc[c][u] + acc[c][u + 4]) + acc[c][u + 8];
      red[((wave * CBW + c) * NV + u) * 64 + lane] = y;
    }
  __syncthreads();
  for (int i = threadIdx.x; i < CBW * NV * 64; i += XW * 64) {
    const int c = i / (NV * 64), u = (i / 64) % NV, l = i & 63;
    const int row = NOP == 2 ? 8 * (u >> 2) + 4 * (l >> 5) + (u & 3) : 4 * (l >> 5) + u;
    if (row >= M || cb0 + c >= ncb) continue;
    float v = red[(c * NV + u) * 64 + l];
#pragma unroll
    for (int w = 1; w < XW; w++) v += red[((w * CBW + c) * NV + u) * 64 + l];
    const long n = static_cast<long>(cb0 + c) * 32 + (l & 31);
    const float y = v + (bias ? bias[n] : 0.f);
    if (out_f32) static_cast<float*>(Y)[static_cast<long>(row) * N + n] = y;
    else static_cast<uint16_t*>(Y)[static_cast<long>(row) * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(y));
  }
}

int device_cu_count();

bool w4a16_pieces_in_lds(int M, int K) { return 6L * M * K <= W_LDS; }

hipError_t launch_w4a16(int fmt, const W4A16Args& a, hipStream_t st) {
  const int nop = w4a16_planes(a.M);
  const bool ldsa = w4a16_pieces_in_lds(a.M, a.K);
  if (!ldsa) {
    const long slots = static_cast<long>(a.K / 64) * 4 * nop * 64;
    hipLaunchKernelGGL(w4a16_split_kernel, dim3(static_cast<unsigned>((slots + 255) / 256)), dim3(256), 0, st, a.X,
                       a.M, a.K, a.inv_lam, nop, static_cast<u32x4*>(a.pieces));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // column blocks per workgroup: one workgroup per compute unit where the
  // blocks allow (at most 3 per workgroup: the registers of INT4's per-group
  // partial products)
  const int ncb = a.N / 32, cus = device_cu_count();
  const int cbw = std::min(3, std::max(1, (ncb + cus - 1) / cus));
  const dim3 grid(static_cast<unsigned>((ncb + cbw - 1) / cbw)), block(XW * 64);
  // scales staged in LDS where the workgroup's (cbw K bytes) fit
  const bool scl = static_cast<long>(cbw) * a.K <= S_LDS;
#define SVDQ_W(F, NP, CB, L)                                                                                         \
  do {                                                                                                              \
    if (scl)                                                                                                        \
      hipLaunchKernelGGL((w4a16_kernel<F, NP, CB, L, true>), grid, block, 0, st, static_cast<const u32x4*>(a.pieces), \
                         a.X, a.inv_lam, a.M, a.K, a.N, a.wcodes, a.wscales, a.bias, a.Y, a.out_f32);               \
    else                                                                                                            \
      hipLaunchKernelGGL((w4a16_kernel<F, NP, CB, L, false>), grid, block, 0, st,                                    \
                         static_cast<const u32x4*>(a.pieces), a.X, a.inv_lam, a.M, a.K, a.N, a.wcodes, a.wscales,   \
                         a.bias, a.Y, a.out_f32);                                                                   \
  } while (0)
#define SVDQ_WC(F, NP, L)                  \
  switch (cbw) {                           \
    case 1: SVDQ_W(F, NP, 1, L); break;    \
    case 2: SVDQ_W(F, NP, 2, L); break;    \
    default: SVDQ_W(F, NP, 3, L); break;   \
  }
#define SVDQ_WF(F)                                \
  if (nop == 1) {                                 \
    if (ldsa) { SVDQ_WC(F, 1, true) }             \
    else { SVDQ_WC(F, 1, false) }                 \
  } else {                                        \
    if (ldsa) { SVDQ_WC(F, 2, true) }             \
    else { SVDQ_WC(F, 2, false) }                 \
  }
  if (fmt == SVDQ_INT4_G64_FP16) { SVDQ_WF(SVDQ_INT4_G64_FP16) }
  else { SVDQ_WF(SVDQ_FP4_E2M1_G32_E8M0) }
#undef SVDQ_WF
#undef SVDQ_WC
#undef SVDQ_W
  return hipGetLastError();
}

}  // namespace svdq
