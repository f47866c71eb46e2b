// Kernel G, INT4 variant: the 4-bit GEMM of the SVDQuant layer with the
// low-rank up-projection appended as an extra bf16 K-slab and a fused bias
// epilogue.  (The FP4 variant is in gemm_fp4.hip.)
//
//   acc[i, n]  = sum_t Tb[i, t] L2b[t, n]      (eq. (5) low-rank branch; the
//                                               walkthrough's Fig. 6: it shares
//                                               the 4-bit branch's output)
//   acc[i, n] += sum_g s_x[i, g] s_w[g, n] sum_{k in g} q_x[i, k] q_w[k, n]
//                                              (eq. (2) per group)
//   Y[i, n]    = round(acc[i, n] + b[n])
//
// Group 64, fp16 scales: the packed nibbles of each K stage are moved to
// LDS; on the way from LDS to the registers each nibble is widened to a byte
// holding 16 * q (shifted into the high half of the byte, so the sign comes
// for free); two 32x32x32 i8 MFMAs give 256 * P_g exactly in int32, a
// 32x32x8 f16 MFMA with one nonzero K slot gives the tile's scale products
// s_x[i] s_w[j] (exact in fp32, in the accumulator layout), and the group is
// dequantized with one convert and one fma per accumulator.  The
// accumulators carry 256 x the result (the slab is scaled up to match and
// the epilogue scales down; powers of two, so every rounding is unchanged).
// The dequantization is VALU work (about 3 instructions per accumulator per
// group against 1/16 cycle of i8 MFMA), which bounds this variant well below
// the i8 MFMA peak.  The MFMAs of the next output tile are issued before the
// dequantization of the current one, so the matrix core and the VALU overlap.
//
// Tiling: 4 waves per workgroup in a 2 x 2 grid, 128 x 128 per workgroup,
// 32 x 32 MFMA tiles.  A K stage is 128 wide (two 64-wide MFMA steps); the
// LDS holds two stages, the global loads of a stage are issued three stages
// before its MFMAs (two register sets), and each stage has one barrier.  In
// every MFMA, lane l owns row (column) l % 32 and the 16-byte half l / 32 of
// the 64-wide K step, for A and B alike, so both operands enumerate K in the
// same order.  Workgroups are mapped to tiles so that the workgroups
// resident on one XCD (the hardware deals them round-robin to the 8 XCDs)
// cover a compact block of tiles that shares rows of A and columns of B in
// that XCD's L2.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {

constexpr int BKB = 64;          // code bytes per row per stage (128 K values)
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lo_nib_bytes(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi_nib_bytes(uint32_t w) { return w & 0xF0F0F0F0u; }

template <int OUT, typename I>
__device__ __forceinline__ void store_out(void* Y, I idx, float v) {
  if constexpr (OUT == SVDQ_OUT_F32) {
    reinterpret_cast<float*>(Y)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(Y)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
}

template <int OUT, typename I>
__device__ __forceinline__ float load_out(const void* Y, I idx) {
  if constexpr (OUT == SVDQ_OUT_F32) {
    return reinterpret_cast<const float*>(Y)[idx];
  } else {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(Y)[idx]) << 16);
  }
}

}  // namespace

// Per-format tile shape, all with 4 waves in a 2 x 2 grid:
//  FP4: each wave owns 128 x 128 (4 x 4 MFMA tiles, 256 fp32 accumulators
//       that only the MFMAs touch, so they live in AGPRs); 256 x 256 per
//       workgroup.
//  INT4: the per-group dequantization updates the accumulators with VALU
//       fma, so they must be VGPRs; each wave owns 64 x 64 (2 x 2 tiles);
//       128 x 128 per workgroup.
template <int FMT>
struct Shape {
  static constexpr bool I4 = FMT == SVDQ_INT4_G64_FP16;
  static constexpr int RB = I4 ? 2 : 4;   // 32-row blocks per wave
  static constexpr int CB = I4 ? 2 : 4;   // 32-column blocks per wave
  static constexpr int NTHREADS = 256;
  static constexpr int BM = 2 * RB * 32;
  static constexpr int BN = 2 * CB * 32;
};

// LDS layout of one K stage (128 K values): the code tiles are kept in the
// MFMA operand-block order of global memory, so block (row block rb, step
// j) of the stage sits at ((rb * 2 + j) * 1 KB) and lane l of an MFMA reads
// the 16 bytes at lane * 16 inside it: copies and reads are contiguous.
__device__ __forceinline__ int lds_block(int rowblk, int j) { return (rowblk * 2 + j) << 10; }

template <int FMT, bool SLAB, int OUT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using SH = Shape<FMT>;
  constexpr int BM = SH::BM, BN = SH::BN, RB = SH::RB, CB = SH::CB;
  constexpr int NTHREADS = SH::NTHREADS;
  constexpr int A_CH = BM * 4 / NTHREADS, B_CH = BN * 4 / NTHREADS;   // 16-byte chunks per thread
  constexpr bool I4 = SH::I4;
  // LDS: two stage buffers of A and B codes plus their scales; the
  // epilogue reuses the code buffers to stage the output tile.
  // INT4 scales: [stage][group][row] fp32 (B pre-divided by 256); FP4: the
  // 4 E8M0 bytes of a row (column) per stage as one word, in [.][0][row].
  constexpr int NSG = I4 ? 2 : 1;
  constexpr int LDS_A = 2 * BM * BKB, LDS_B = 2 * BN * BKB;
  constexpr int LDS_SA = 2 * NSG * BM * 4, LDS_SB = 2 * NSG * BN * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_A + LDS_B + LDS_SA + LDS_SB];
  auto sA = reinterpret_cast<uint8_t(*)[BM * BKB]>(smem);
  auto sB = reinterpret_cast<uint8_t(*)[BN * BKB]>(smem + LDS_A);
  auto sSA = reinterpret_cast<uint32_t(*)[NSG][BM]>(smem + LDS_A + LDS_B);
  auto sSB = reinterpret_cast<uint32_t(*)[NSG][BN]>(smem + LDS_A + LDS_B + LDS_SA);

  // kernel arguments in registers (a lambda capturing g would read them
  // from the argument segment with vector loads)
  const int M = g.M, K = g.K, N = g.N, rank = g.rank;
  const uint8_t* __restrict__ acodes = g.acodes;
  const uint8_t* __restrict__ wcodes = g.wcodes;
  const uint32_t* __restrict__ ascales = static_cast<const uint32_t*>(g.ascales);
  const uint32_t* __restrict__ wscales = static_cast<const uint32_t*>(g.wscales);
  const uint16_t* __restrict__ Tb = g.Tb;
  const uint16_t* __restrict__ l2t = g.l2t;
  const float* __restrict__ bias = g.bias;
  void* __restrict__ Yout = g.Y;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const long m0 = static_cast<long>(tm) * BM;
  const long n0 = static_cast<long>(tn) * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int SW = K / 128;                        // scale words (4 bytes) per row
  const int stages = K / 128;
  const int wrow0 = wm * (RB * 32), wcol0 = wn * (CB * 32);

  f32x16 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; i++)
#pragma unroll
    for (int j = 0; j < CB; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // ---- low-rank up-projection first (K = rank, bf16 MFMA).  Rows
  // (columns) past M (N) are clamped to the last valid one: their outputs
  // are computed from real data and never stored, and every load stays
  // unconditional.
  if constexpr (SLAB) {
    for (int tb = 0; tb < rank / 16; tb++) {
      bf16x8 b[CB];
#pragma unroll
      for (int j = 0; j < CB; j++) {
        const long c = min(n0 + wcol0 + j * 32 + l32, static_cast<long>(N - 1));
        b[j] = *reinterpret_cast<const bf16x8*>(l2t + bf16_block_index(c, tb * 16 + lh * 8, rank));
      }
#pragma unroll
      for (int i = 0; i < RB; i++) {
        const long r = min(m0 + wrow0 + i * 32 + l32, static_cast<long>(M - 1));
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Tb + bf16_block_index(r, tb * 16 + lh * 8, rank));
#pragma unroll
        for (int j = 0; j < CB; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
    if constexpr (I4) {
      // the INT4 groups accumulate 256 x their value (codes widened to 16 q);
      // the slab is scaled to match and the epilogue divides by 256 (powers
      // of two: every rounding is the same as without the factor)
#pragma unroll
      for (int i = 0; i < RB; i++)
#pragma unroll
        for (int j = 0; j < CB; j++)
#pragma unroll
          for (int v = 0; v < 16; v++) acc[i][j][v] *= 256.0f;
    }
  }

  // ---- global -> registers -> LDS.  A stage of the A (B) tile is BM / 16
  // (BN / 16) operand blocks of 1 KB; thread t copies 16-byte pieces q =
  // t + 256 i: block q / 64, lane slot q % 64 (64 threads cover one block
  // contiguously).  Row blocks past the matrix are clamped to its last one
  // (their outputs are never stored).  Thread t < BM also loads the scale
  // word of A row t, thread t >= BM that of B column t - BM.
  struct Regs {
    u32x4 a[A_CH], b[B_CH];
    uint32_t sa, sb;
  };
  // INT4 scale word of this thread's row (t < BM: A row t, else B column
  // t - BM) for stage st: sc_base[sc_off + st * sc_step].  Activation scales
  // are in 32-row blocks (word (row, st) at ((row / 32) * SW + st) * 32 +
  // row % 32), weight scales row-major.
  const bool sc_is_a = t < BM;
  const long sc_row = sc_is_a ? min(m0 + t, static_cast<long>(M - 1)) : min(n0 + (t - BM), static_cast<long>(N - 1));
  const uint32_t* __restrict__ sc_base = sc_is_a ? ascales : wscales;
  const long sc_off = sc_is_a ? (sc_row >> 5) * SW * 32 + (sc_row & 31) : sc_row * SW;
  const int sc_step = sc_is_a ? 32 : 1;
  const long KBLK = K / 64;                       // 1 KB blocks per 32-row block
  const long last_ablk = (M + 31) / 32 - 1, last_bblk = N / 32 - 1;
  auto load_stage = [&](Regs& r, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; i++) {
      const int q = t + i * NTHREADS, blk = q >> 6;
      const long rb = min(m0 / 32 + (blk >> 1), last_ablk);
      r.a[i] = *reinterpret_cast<const u32x4*>(acodes + ((rb * KBLK + 2 * st + (blk & 1)) << 10) + (q & 63) * 16);
    }
#pragma unroll
    for (int i = 0; i < B_CH; i++) {
      const int q = t + i * NTHREADS, blk = q >> 6;
      const long rb = min(n0 / 32 + (blk >> 1), last_bblk);
      r.b[i] = *reinterpret_cast<const u32x4*>(wcodes + ((rb * KBLK + 2 * st + (blk & 1)) << 10) + (q & 63) * 16);
    }
    if constexpr (I4) {
      // 128 threads per operand
      r.sa = sc_base[sc_off + st * sc_step];
    } else {
      r.sa = ascales[min(m0 + t, static_cast<long>(M - 1)) * SW + st];
      r.sb = wscales[min(n0 + t, static_cast<long>(N - 1)) * SW + st];
    }
  };
  auto store_stage = [&](const Regs& r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; i++) {
      const int q = t + i * NTHREADS;
      *reinterpret_cast<u32x4*>(&sA[buf][q * 16]) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; i++) {
      const int q = t + i * NTHREADS;
      *reinterpret_cast<u32x4*>(&sB[buf][q * 16]) = r.b[i];
    }
    if constexpr (I4) {
      // fp16 bits of the two groups' scales, as the f16 MFMA operands take them
      uint32_t(*ss)[BM] = t < BM ? sSA[buf] : sSB[buf];
      const int idx = t < BM ? t : t - BM;
      ss[0][idx] = r.sa & 0xFFFFu;
      ss[1][idx] = r.sa >> 16;
    } else {
      sSA[buf][0][t] = r.sa;
      sSB[buf][0][t] = r.sb;
    }
  };

  // Stage k's codes are loaded into register set R[k % 2].  Schedule of
  // stage s: (1) store register set R[(s + 1) % 2] (stage s + 1, loaded two
  // stages earlier) to the other LDS buffer, (2) reuse that set for the
  // global loads of stage s + 3, (3) run the MFMAs of stage s, (4) barrier.
  // Loads past the last stage re-read the last stage (their data is never
  // used), so that every stage issues the same loads and the compiler's
  // wait counts stay exact across the loop.
  Regs R0, R1;
  const int last = stages - 1;
  load_stage(R0, 0);
  load_stage(R1, min(1, last));
  store_stage(R0, 0);
  load_stage(R0, min(2, last));
  __syncthreads();

  auto stage_body = [&](int s, Regs& Rn, auto BUF) __attribute__((always_inline)) {
    constexpr int buf = decltype(BUF)::value;
    store_stage(Rn, buf ^ 1);
    load_stage(Rn, min(s + 3, last));
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < 2; j++) {          // two 64-wide MFMA steps per stage
      const int c = 2 * j + lh;            // this lane's 16-byte chunk of the stage
      u32x4 av[RB], bv[CB];
#pragma unroll
      for (int rb = 0; rb < RB; rb++)
        av[rb] = *reinterpret_cast<const u32x4*>(&sA[buf][lds_block(wrow0 / 32 + rb, j) + lane * 16]);
#pragma unroll
      for (int cb = 0; cb < CB; cb++)
        bv[cb] = *reinterpret_cast<const u32x4*>(&sB[buf][lds_block(wcol0 / 32 + cb, j) + lane * 16]);

      if constexpr (I4) {
        i32x4 a0[RB], a1[RB], b0[CB], b1[CB];
        // scale operands of the f16 MFMA that forms s_x[i] s_w[j] for a
        // 32 x 32 tile: only K slot 0 (lanes 0-31, first element) is nonzero
        // (every lane reads its word; lanes 32-63 mask it to zero, which
        // keeps the reads unconditional)
        f16x4 fa[RB], fb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
          b0[cb] = i32x4{(int)lo_nib_bytes(bv[cb].x), (int)hi_nib_bytes(bv[cb].x), (int)lo_nib_bytes(bv[cb].y),
                         (int)hi_nib_bytes(bv[cb].y)};
          b1[cb] = i32x4{(int)lo_nib_bytes(bv[cb].z), (int)hi_nib_bytes(bv[cb].z), (int)lo_nib_bytes(bv[cb].w),
                         (int)hi_nib_bytes(bv[cb].w)};
          const uint32_t w = sSB[buf][j][wcol0 + cb * 32 + l32] & (lh ? 0u : 0xFFFFu);
          fb[cb] = __builtin_bit_cast(f16x4, u32x2{w, 0u});
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
          a0[rb] = i32x4{(int)lo_nib_bytes(av[rb].x), (int)hi_nib_bytes(av[rb].x), (int)lo_nib_bytes(av[rb].y),
                         (int)hi_nib_bytes(av[rb].y)};
          a1[rb] = i32x4{(int)lo_nib_bytes(av[rb].z), (int)hi_nib_bytes(av[rb].z), (int)lo_nib_bytes(av[rb].w),
                         (int)hi_nib_bytes(av[rb].w)};
          const uint32_t w = sSA[buf][j][wrow0 + rb * 32 + l32] & (lh ? 0u : 0xFFFFu);
          fa[rb] = __builtin_bit_cast(f16x4, u32x2{w, 0u});
        }
        // software pipeline over the wave's output tiles: the MFMAs of tile
        // u + 1 (the group's 256 P_g in int32 and the scale products
        // s_x s_w, exact in fp32) are in flight while tile u is dequantized
        constexpr int NT = RB * CB;
        i32x16 p[2];
        f32x16 sp[2];
        auto mma = [&](int u, i32x16& dst, f32x16& sdst) __attribute__((always_inline)) {
          const int rb = u / CB, cb = u % CB;
          i32x16 z16;
          f32x16 zf;
#pragma unroll
          for (int v = 0; v < 16; v++) {
            z16[v] = 0;
            zf[v] = 0.f;
          }
          dst = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[rb], b0[cb], z16, 0, 0, 0);
          dst = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[rb], b1[cb], dst, 0, 0, 0);
          sdst = __builtin_amdgcn_mfma_f32_32x32x8f16(fa[rb], fb[cb], zf, 0, 0, 0);
        };
        mma(0, p[0], sp[0]);
#pragma unroll
        for (int u = 0; u < NT; u++) {
          const int rb = u / CB, cb = u % CB;
          if (u + 1 < NT) mma(u + 1, p[(u + 1) & 1], sp[(u + 1) & 1]);
          const i32x16& pp = p[u & 1];
          const f32x16& ss = sp[u & 1];
#pragma unroll
          for (int v = 0; v < 16; v++) acc[rb][cb][v] = __builtin_fmaf(static_cast<float>(pp[v]), ss[v], acc[rb][cb][v]);
        }
      } else {
        i32x8 a[RB], b[CB];
        int sa[RB], sb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
          b[cb] = i32x8{(int)bv[cb].x, (int)bv[cb].y, (int)bv[cb].z, (int)bv[cb].w, 0, 0, 0, 0};
          sb[cb] = (sSB[buf][0][wcol0 + cb * 32 + l32] >> (8 * c)) & 0xFF;
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
          a[rb] = i32x8{(int)av[rb].x, (int)av[rb].y, (int)av[rb].z, (int)av[rb].w, 0, 0, 0, 0};
          sa[rb] = (sSA[buf][0][wrow0 + rb * 32 + l32] >> (8 * c)) & 0xFF;
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
          for (int cb = 0; cb < CB; cb++)
            acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[rb], b[cb], acc[rb][cb], 4, 4, 0, sa[rb],
                                                                          0, sb[cb]);
      }
    }
    __syncthreads();
  };
  int s = 0;
  for (; s + 1 < stages; s += 2) {
    stage_body(s, R1, std::integral_constant<int, 0>{});
    stage_body(s + 1, R0, std::integral_constant<int, 1>{});
  }
  if (s < stages) stage_body(s, R1, std::integral_constant<int, 0>{});

  // ---- epilogue: bias, rounding, store.  Each wave stages one 32-row
  // slice of its tile at a time in its own LDS region (row-major, output
  // type), then writes whole rows with 16-byte stores.
  {
    constexpr int OB = OUT == SVDQ_OUT_F32 ? 4 : 2;     // output bytes per element
    constexpr int ROWB = CB * 32 * OB;                  // bytes of one slice row
    constexpr int SLICE = 32 * ROWB;
    static_assert(4 * SLICE <= LDS_A + LDS_B, "epilogue staging must fit the stage buffers");
    uint8_t* stage = smem + wave * SLICE;
    float bv[CB];
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      const long c = min(n0 + wcol0 + cb * 32 + l32, static_cast<long>(N - 1));
      bv[cb] = bias ? bias[c] : 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
#pragma unroll
      for (int cb = 0; cb < CB; cb++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int row = 8 * (v >> 2) + 4 * lh + (v & 3);
          const int off = row * ROWB + (cb * 32 + l32) * OB;
          const float y = (I4 ? acc[rb][cb][v] * (1.0f / 256.0f) : acc[rb][cb][v]) + bv[cb];
          if constexpr (OUT == SVDQ_OUT_F32) *reinterpret_cast<float*>(stage + off) = y;
          else *reinterpret_cast<uint16_t*>(stage + off) = static_cast<uint16_t>(f32_to_bf16_bits(y));
        }
      __builtin_amdgcn_wave_barrier();
      constexpr int CHUNKS = SLICE / 16;                // 16-byte chunks per slice
      constexpr int PER_ROW = ROWB / 16;
#pragma unroll
      for (int i = 0; i < CHUNKS / 64; i++) {
        const int q = lane + 64 * i;
        const int row = q / PER_ROW, cc = q % PER_ROW;
        const long grow = m0 + wrow0 + rb * 32 + row;
        const long gcol = n0 + wcol0 + cc * (16 / OB);
        const u32x4 d = *reinterpret_cast<const u32x4*>(stage + row * ROWB + cc * 16);
        if (grow < M && gcol < N)
          *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(Yout) + (grow * N + gcol) * OB) = d;
      }
      __builtin_amdgcn_wave_barrier();
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
    const bf16x8 a = r < M ? *reinterpret_cast<const bf16x8*>(Tb + bf16_block_index(r, tb * 16 + lh * 8, rank)) : z;
    const bf16x8 b = c < N ? *reinterpret_cast<const bf16x8*>(l2t + bf16_block_index(c, tb * 16 + lh * 8, rank)) : z;
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
  const bool f32 = out_dtype == SVDQ_OUT_F32;
  if (fmt == SVDQ_INT4_G64_FP16) {
    using SH = Shape<SVDQ_INT4_G64_FP16>;
    const int tiles = ((g.M + SH::BM - 1) / SH::BM) * ((g.N + SH::BN - 1) / SH::BN);
    dim3 grid(tiles), block(256);
#define SVDQ_G(S, O) hipLaunchKernelGGL((gemm_kernel<SVDQ_INT4_G64_FP16, S, O>), grid, block, 0, st, g)
    if (slab) { if (f32) SVDQ_G(true, SVDQ_OUT_F32); else SVDQ_G(true, SVDQ_OUT_BF16); }
    else      { if (f32) SVDQ_G(false, SVDQ_OUT_F32); else SVDQ_G(false, SVDQ_OUT_BF16); }
#undef SVDQ_G
    return hipGetLastError();
  }
  return launch_gemm_fp4(slab, out_dtype, g, st);
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
