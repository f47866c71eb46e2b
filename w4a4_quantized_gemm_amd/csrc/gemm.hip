// Kernel G: the 4-bit GEMM of the SVDQuant layer with the low-rank
// up-projection appended as an extra bf16 K-slab and a fused bias epilogue.
//
//   acc[i, n]  = sum_t Tb[i, t] L2b[t, n]      (eq. (5) low-rank branch; the
//                                               walkthrough's Fig. 6: it shares
//                                               the 4-bit branch's output)
//   acc[i, n] += sum_g s_x[i, g] s_w[g, n] sum_{k in g} q_x[i, k] q_w[k, n]
//                                              (eq. (2) per group)
//   Y[i, n]    = round(acc[i, n] + b[n])
//
// INT4 (group 64, fp16 scales): the packed nibbles of each K stage are moved
// to LDS; on the way from LDS to the registers each nibble is widened to a
// byte holding 16 * q (shifted into the high half of the byte, so the sign
// comes for free); two 32x32x32 i8 MFMAs give 256 * P_g exactly in int32 and
// the group is dequantized into the fp32 accumulators with s_x * s_w / 256.
// The MFMAs of the next output tile are issued before the dequantization of
// the current one, so the matrix core and the VALU overlap.
// FP4 (group 32, E8M0 scales): the E2M1 nibbles and the power-of-two scales
// are the native operands of the gfx950 block-scaled MFMA (32x32x64), which
// accumulates in fp32 directly; there is no dequantization work.
//
// Tiling (see Shape): 4 waves per workgroup, FP4 256 x 256, INT4 128 x 128;
// 32 x 32 MFMA tiles.  A K stage is 128 wide (two
// 64-wide MFMA steps); the LDS holds two stages, the global loads of a stage
// are issued three stages before its MFMAs (two register sets), and each
// stage has one barrier.  In every
// MFMA, lane l owns row (column) l % 32 and the 16-byte half l / 32 of the
// 64-wide K step, for A and B alike, so both operands enumerate K in the same
// order.  Workgroups are mapped to tiles so that the workgroups resident on
// one XCD (the hardware deals them round-robin to the 8 XCDs) cover a
// compact block of tiles that shares rows of A and columns of B in that
// XCD's L2.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {

constexpr int BKB = 64;          // code bytes per row per stage (128 K values)
constexpr int NXCD = 8;
constexpr int GROUP_TM = 4;      // tile rows per L2 group

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

// workgroup id -> (tile_m, tile_n): contiguous tile ranges per XCD, grouped
// GROUP_TM tile rows at a time inside each range.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int q = T / NXCD, rem = T % NXCD;
  const int x = b % NXCD, j = b / NXCD;
  const int t = x * q + (x < rem ? x : rem) + j;
  const int per_group = GROUP_TM * tiles_n;
  const int grp = t / per_group;
  const int first = grp * GROUP_TM;
  const int gm = min(GROUP_TM, tiles_m - first);
  const int w = t - grp * per_group;
  tm = first + w % gm;
  tn = w / gm;
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
      const bool is_a = t < BM;
      const long row = is_a ? min(m0 + t, static_cast<long>(M - 1)) : min(n0 + (t - BM), static_cast<long>(N - 1));
      r.sa = (is_a ? ascales : wscales)[row * SW + st];
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
      const float mul = t < BM ? 1.0f : 1.0f / 256.0f;
      uint32_t(*ss)[BM] = t < BM ? sSA[buf] : sSB[buf];
      const int idx = t < BM ? t : t - BM;
      ss[0][idx] = __float_as_uint(__half2float(__ushort_as_half(static_cast<unsigned short>(r.sa & 0xFFFFu))) * mul);
      ss[1][idx] = __float_as_uint(__half2float(__ushort_as_half(static_cast<unsigned short>(r.sa >> 16))) * mul);
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
        float sw[CB];
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
          b0[cb] = i32x4{(int)lo_nib_bytes(bv[cb].x), (int)hi_nib_bytes(bv[cb].x), (int)lo_nib_bytes(bv[cb].y),
                         (int)hi_nib_bytes(bv[cb].y)};
          b1[cb] = i32x4{(int)lo_nib_bytes(bv[cb].z), (int)hi_nib_bytes(bv[cb].z), (int)lo_nib_bytes(bv[cb].w),
                         (int)hi_nib_bytes(bv[cb].w)};
          sw[cb] = __uint_as_float(sSB[buf][j][wcol0 + cb * 32 + l32]);
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++) {
          a0[rb] = i32x4{(int)lo_nib_bytes(av[rb].x), (int)hi_nib_bytes(av[rb].x), (int)lo_nib_bytes(av[rb].y),
                         (int)hi_nib_bytes(av[rb].y)};
          a1[rb] = i32x4{(int)lo_nib_bytes(av[rb].z), (int)hi_nib_bytes(av[rb].z), (int)lo_nib_bytes(av[rb].w),
                         (int)hi_nib_bytes(av[rb].w)};
        }
        // software pipeline over the wave's output tiles: the MFMAs of tile
        // u + 1 are in flight while tile u is dequantized
        constexpr int NT = RB * CB;
        i32x16 p[2];
        auto mma = [&](int u, i32x16& dst) __attribute__((always_inline)) {
          const int rb = u / CB, cb = u % CB;
          i32x16 z16;
#pragma unroll
          for (int v = 0; v < 16; v++) z16[v] = 0;
          dst = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[rb], b0[cb], z16, 0, 0, 0);
          dst = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[rb], b1[cb], dst, 0, 0, 0);
        };
        mma(0, p[0]);
        f32x4 sx[4];
#pragma unroll
        for (int u = 0; u < NT; u++) {
          const int rb = u / CB, cb = u % CB;
          if (u + 1 < NT) mma(u + 1, p[(u + 1) & 1]);
          if (cb == 0) {
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
              sx[q4] = *reinterpret_cast<const f32x4*>(&sSA[buf][j][wrow0 + rb * 32 + 8 * q4 + 4 * lh]);
          }
          const i32x16& pp = p[u & 1];
#pragma unroll
          for (int v = 0; v < 16; v++)
            acc[rb][cb][v] = __builtin_fmaf(static_cast<float>(pp[v]), sx[v >> 2][v & 3] * sw[cb], acc[rb][cb][v]);
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
          const float y = acc[rb][cb][v] + bv[cb];
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

// ---------------------------------------------------------------------------
// FP4 GEMM: gfx950 block-scaled MFMA, persistent workgroups of 8 waves, a
// deep ring of direct global->LDS copies.
//
// Operand roles: the MFMA's A operand is the weight tile (its rows are output
// columns n) and its B operand the activation tile (output rows m).  A 32x32
// accumulator then gives lane l output row m = l % 32 and, for element v,
// column 8 (v / 4) + 4 (l / 32) + v % 4.
//
// Waves: 8 per workgroup, two per SIMD (so one wave's waits hide behind the
// other's MFMAs, and twice as many waves keep copies in flight: the copy
// throughput of a wave is limited, not the bytes in flight).  The 256 x 256
// output tile is split 2 (m) x 4 (n): each wave owns 128 rows x 64 columns,
// 4 x 2 MFMA tiles, 128 fp32 accumulators.
//
// Stages: the reduction of one output tile is a sequence of stages, first
// rank / 16 low-rank stages (16 ranks of Tb and L2b, bf16 32x32x16 MFMA),
// then K / 64 FP4 stages (32x32x64 block-scaled MFMA).  Both kinds move 8 KB
// of activation-side and 8 KB of weight-side operand blocks (1 KB = 32 rows
// in MFMA lane order, contiguous in global memory) plus 1 KB of E8M0 scale
// bytes straight from global memory into a ring of LDS stage
// buffers; copies run P_AHEAD stages ahead of the MFMAs.  A wave completes
// copy instructions at a limited rate whatever their size, so every copy
// moves 16 bytes per lane: each wave copies one activation and one weight
// block per stage, the scale kilobyte of a stage is copied by one wave in
// turn, and a tile's bias (1 KB) once per tile.  Each workgroup walks its
// tiles in sequence and the stage stream continues across tile boundaries.
// One barrier per stage publishes the next stage (wait for this wave's
// copies of it, then s_barrier) and frees the buffer the new copies go to.
//
// Epilogue: bias, rounding, and 16-row slices staged in the X/W part of the
// just-consumed stage buffer (free until the next stage's barrier), read
// back as whole rows and stored 16 bytes per lane, contiguous.
namespace {
constexpr int P_TILE = 256;                        // output tile P_TILE x P_TILE
constexpr int P_X = 0, P_W = 8192, P_S = 16384;    // parts of a stage buffer
constexpr int P_STAGE = 17408;                     // + 1 KB of scales: 8 x 64 activation, 8 x 64 weight

// wait until at most n vector-memory operations of this wave are
// outstanding, then barrier; a compiler memory barrier as well
#define SVDQ_WAIT_VM_BARRIER(n) asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_barrier" ::: "memory")
}  // namespace

// BIG: every tile has more than P_AHEAD stages, so the copies run at most
// one tile ahead and their source follows from the consumed stage without a
// separate cursor.  RS_ODD: rank / 16 is odd (decides how many stages of a
// tile are peeled off its even-length loops).
template <bool SLAB, int OUT, bool RS_ODD, bool BIG>
__global__ __launch_bounds__(512) void gemm_fp4_kernel(GemmArgs g) {
  // Ring of P_NBUF stage buffers (P_AHEAD = P_NBUF - 1 stages in flight),
  // then P_NBIAS tile bias buffers of 1 KB (by turn % P_NBIAS).  The copies
  // run at most P_AHEAD stages ahead, so with 8 bias buffers a tile's bias
  // is not overwritten before its epilogue for any tile of 2 stages or more.
  // (A ninth stage buffer measured slower.)
  constexpr int P_NBUF = 8;
  constexpr int P_AHEAD = P_NBUF - 1;
  constexpr int P_NBIAS = 8;
  constexpr int P_BIAS = P_NBUF * P_STAGE;
  constexpr int P_LDS = P_BIAS + P_NBIAS * 1024;   // 147456 bytes
  __shared__ __attribute__((aligned(1024))) uint8_t smem[P_LDS];

  const int M = g.M, K = g.K, N = g.N;
  const int RS = SLAB ? g.rank / 16 : 0;        // low-rank stages per tile
  const int KS = K / 64;                         // FP4 stages per tile
  const int S = RS + KS;
  const uint8_t* __restrict__ acodes = g.acodes;
  const uint8_t* __restrict__ wcodes = g.wcodes;
  const uint8_t* __restrict__ ascales = static_cast<const uint8_t*>(g.ascales);
  const uint8_t* __restrict__ wscales = static_cast<const uint8_t*>(g.wscales);
  const uint8_t* __restrict__ tbb = reinterpret_cast<const uint8_t*>(g.Tb);
  const uint8_t* __restrict__ l2b = reinterpret_cast<const uint8_t*>(g.l2t);
  const bool has_bias = g.bias != nullptr;
  const float* __restrict__ bias = g.bias;
  void* __restrict__ Yout = g.Y;

  const int tiles_m = (M + P_TILE - 1) / P_TILE, tiles_n = (N + P_TILE - 1) / P_TILE;
  const int ntiles = tiles_m * tiles_n;
  const int grid = static_cast<int>(gridDim.x), wg = static_cast<int>(blockIdx.x);
  const int my_tiles = (ntiles - wg + grid - 1) / grid;   // >= 1: the grid never exceeds the tile count
  const int last_ablk = (M + 31) / 32 - 1, last_bblk = N / 32 - 1;

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;       // 128-row half, 64-column quarter
  const int l32 = lane & 31, lh = lane >> 5;

  // 32-row block indices of the tile a workgroup handles in its seq-th turn
  auto tile_blocks = [&](int seq, int& mb0, int& nb0) __attribute__((always_inline)) {
    int tm, tn;
    tile_of(wg + seq * grid, tiles_m, tiles_n, tm, tn);
    mb0 = tm * (P_TILE / 32);
    nb0 = tn * (P_TILE / 32);
  };

  // ---- copy side.  For stage C, wave w copies activation block w and
  // weight block w (1 KB each); wave C % 8 also copies the stage's scale
  // kilobyte (lanes 0-31: 64 bytes per activation block, 4 lanes each;
  // lanes 32-63 the weight blocks); on the last stage of a tile with a bias,
  // wave 0 also copies the tile's 256 bias values into bias buffer
  // turn % P_NBIAS (a tile's bias buffer is not reused before its epilogue:
  // the copies run at most P_AHEAD stages ahead).  Blocks past the matrix are clamped to its last
  // block; copies past the last stage repeat the last stage.  Sources are
  // byte offsets turned into pointers at the copy (plain locals are the form
  // the host compilation pass of this kernel also accepts).
  struct Src {
    long x, w, sc, b;      // operand blocks, this lane's scale bytes, this lane's bias values
    bool lr;               // low-rank stage (Tb / L2b bases)
    bool scales, bias;     // this wave copies the scales / the bias of the stage
    uint32_t dst, bdst;    // LDS byte offsets of the stage buffer and the bias buffer
  };
  auto stage_src = [&](int seq, int st, long C, int mb0, int nb0) __attribute__((always_inline)) {
    Src q;
    q.lr = SLAB && st < RS;
    const int ks = q.lr ? st : st - RS;           // stage index inside its matrix
    const long stride = q.lr ? RS : KS;           // 1 KB blocks per 32-row block
    q.x = (min(mb0 + wave, last_ablk) * stride + ks) << 10;
    q.w = (min(nb0 + wave, last_bblk) * stride + ks) << 10;
    const int kst = q.lr ? 0 : ks;                // low-rank stages copy (unused) scales of stage 0
    const int sblk = (lane >> 2) & 7;
    const long srow = lh ? min(nb0 + sblk, last_bblk) : min(mb0 + sblk, last_ablk);
    q.sc = (srow * KS + kst) * 64 + (lane & 3) * 16;
    q.b = min(nb0 * 32 + lane * 4, N - 4);
    q.scales = wave == static_cast<int>(C & 7);     // the 8 waves take turns
    q.bias = wave == 0 && has_bias && st == S - 1;
    q.dst = static_cast<uint32_t>(C % P_NBUF) * P_STAGE;
    q.bdst = P_BIAS + (seq & (P_NBIAS - 1)) * 1024;
    return q;
  };
  auto copy = [&](const Src& q, int i) __attribute__((always_inline)) {
    if (i < 2) {
      const uint8_t* src = (i == 0 ? (q.lr ? tbb : acodes) + q.x : (q.lr ? l2b : wcodes) + q.w) + lane * 16;
      uint8_t* dst = smem + q.dst + (i == 0 ? P_X : P_W) + wave * 1024;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    } else if (i == 2) {
      if (q.scales) {
        const uint8_t* src = (lh ? wscales : ascales) + q.sc;
        uint8_t* dst = smem + q.dst + P_S;
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      }
    } else {
      if (q.bias) {
        const float* src = bias + q.b;
        uint8_t* dst = smem + q.bdst;
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      }
    }
  };
  constexpr int NCOPY = 4;                        // copy slots per stage (the last two conditional)

  // tile being consumed, and the next one (BIG: the copies' only other tile)
  int seq = 0, mb0, nb0, nmb0, nnb0;
  tile_blocks(0, mb0, nb0);
  nmb0 = mb0;
  nnb0 = nb0;
  // general cursor (small tiles): the next stage to copy
  int iseq = 0, ist = 0, imb0 = mb0, inb0 = nb0;
  // sources of the copies issued while stage st of the current tile is consumed
  auto ahead_src = [&](int st, long G) __attribute__((always_inline)) {
    if constexpr (BIG) {
      const int t = st + P_AHEAD;
      const bool wrap = t >= S, has_next = seq + 1 < my_tiles;
      const bool nxt = wrap && has_next;
      // past the last tile: repeat its last stage
      const int cst = wrap ? (has_next ? t - S : S - 1) : t;
      return stage_src(nxt ? seq + 1 : seq, cst, G + P_AHEAD, nxt ? nmb0 : mb0, nxt ? nnb0 : nb0);
    } else {
      const bool past = iseq >= my_tiles;
      const Src q = stage_src(past ? my_tiles - 1 : iseq, past ? S - 1 : ist, G + P_AHEAD, imb0, inb0);
      if (!past && ++ist == S) {
        ist = 0;
        if (++iseq < my_tiles) tile_blocks(iseq, imb0, inb0);
      }
      return q;
    }
  };

  // ---- compute side: operand piece p of a stage (p = 0: weight block 0,
  // 1..4: activation blocks 0..3, 5: weight block 1, the order the 8 MFMAs
  // first need them), with its scale byte.  A stage's reads use four
  // per-lane base addresses (the ring offset is uniform, the lane part
  // loop-invariant) and constant offsets.
  struct Ops {
    u32x4 w[2], x[4];
    uint32_t sw[2], sx[4];
  };
  struct Addr {
    uint32_t x, w, sx, sw;
  };
  const uint32_t lane16 = lane * 16, lanes = l32 * 2 + lh;
  auto addr_of = [&](long G) __attribute__((always_inline)) {
    const uint32_t b = static_cast<uint32_t>(G % P_NBUF) * P_STAGE;
    Addr a;
    a.x = b + P_X + wm * 4096 + lane16;           // activation blocks 4 wm + j
    a.w = b + P_W + wn * 2048 + lane16;           // weight blocks 2 wn + i
    a.sx = b + P_S + wm * 256 + lanes;            // scales of activation block 4 wm + j: + j * 64
    a.sw = b + P_S + 512 + wn * 128 + lanes;      // scales of weight block 2 wn + i: + i * 64
    return a;
  };
  auto read_piece = [&](Ops& o, const Addr& a, int p) __attribute__((always_inline)) {
    if (p == 0 || p == 5) {
      const int i = p == 0 ? 0 : 1;
      o.w[i] = *reinterpret_cast<const u32x4*>(smem + a.w + i * 1024);
      o.sw[i] = smem[a.sw + i * 64];
    } else {
      const int j = p - 1;
      o.x[j] = *reinterpret_cast<const u32x4*>(smem + a.x + j * 1024);
      o.sx[j] = smem[a.sx + j * 64];
    }
  };

  f32x16 acc[2][4];
  // MFMA k of a stage: weight block i = k / 4, activation block j = k % 4.
  // The first stage of a tile adds to a constant zero instead of the
  // accumulators (which therefore never need clearing).
  auto mfma = [&](const Ops& o, int k, auto LR, auto FIRST) __attribute__((always_inline)) {
    const int i = k >> 2, j = k & 3;
    f32x16 c = acc[i][j];
    if constexpr (decltype(FIRST)::value) {
#pragma unroll
      for (int v = 0; v < 16; v++) c[v] = 0.f;
    }
    if constexpr (decltype(LR)::value) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, o.w[i]),
                                                         __builtin_bit_cast(bf16x8, o.x[j]), c, 0, 0, 0);
    } else {
      const i32x8 av = i32x8{(int)o.w[i].x, (int)o.w[i].y, (int)o.w[i].z, (int)o.w[i].w, 0, 0, 0, 0};
      const i32x8 bv = i32x8{(int)o.x[j].x, (int)o.x[j].y, (int)o.x[j].z, (int)o.x[j].w, 0, 0, 0, 0};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)o.sw[i], 0, (int)o.sx[j]);
    }
  };

  // One stage (index st of the tile, G overall): 8 MFMAs on `cur`; between
  // them the reads of stage G + 1 into `nxt` and the copies of stage
  // G + P_AHEAD.  The wait at the top publishes stage G + 1: at least the
  // block copies of the P_AHEAD - 2 stages issued after it may stay in flight (the
  // occasional scale or bias copy among them only makes the wait slightly
  // longer), and in the first P_AHEAD - 1 stages of a tile also the
  // previous tile's epilogue stores, which were issued after them.  It also
  // frees the buffer of stage G - 1.  The order is fixed with scheduling
  // fences.
  constexpr int NSTORE = OUT == SVDQ_OUT_F32 ? 32 : 16;   // epilogue stores per wave
  auto stage = [&](const Ops& cur, Ops& nxt, long G, int st, auto LR, auto FIRST) __attribute__((always_inline)) {
    const Src q = ahead_src(st, G);
    const Addr an = addr_of(G + 1);
    mfma(cur, 0, LR, FIRST);
    // 5 stages of 2 block copies after stage G + 1 (+ the epilogue stores)
    if (BIG && seq > 0 && st <= P_AHEAD - 2) {
      if constexpr (NSTORE == 32) SVDQ_WAIT_VM_BARRIER(42);
      else SVDQ_WAIT_VM_BARRIER(26);
    } else {
      SVDQ_WAIT_VM_BARRIER(10);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 1; k < 8; k++) {
      mfma(cur, k, LR, FIRST);
      if (k <= 6) read_piece(nxt, an, k - 1);
      if (k >= 3 && k - 3 < NCOPY) copy(q, k - 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue of the tile at (mb0, nb0), after its last stage G: bias,
  // rounding, then per 16-row (bf16) or 8-row (fp32) slice: the lanes holding
  // those rows write them into this wave's 2 KB of the X/W part of stage
  // buffer G (16-byte chunks XOR-swizzled by row against bank conflicts),
  // and the wave reads whole rows back and stores them 16 bytes per lane.
  // The bias of the tile was copied into the tail of the same buffer.  The
  // stores are bounds-checked buffer stores over the tile's rows: rows past
  // M and columns past N get an offset past the buffer and are dropped, so
  // every store instruction issues (the waits count them).
  auto epilogue = [&](long G) __attribute__((always_inline)) {
    // lane indices recomputed here through an opaque move, so that the
    // compiler does not hoist the epilogue's per-lane addresses out of the
    // tile loop (they would stay live through the main loops and spill)
    int lane_e;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_e) : "v"(lane));
    const int l32 = lane_e & 31, lh = lane_e >> 5, lane = lane_e;
    constexpr int OB = OUT == SVDQ_OUT_F32 ? 4 : 2;
    constexpr int CPR = 64 * OB / 16;             // 16-byte chunks per staged row
    constexpr int RPS = 2048 / (64 * OB);         // rows per slice
    const uint32_t buf = static_cast<uint32_t>(G % P_NBUF) * P_STAGE;
    uint8_t* stg = smem + buf + wave * 2048;
    const float* bl = reinterpret_cast<const float*>(smem + P_BIAS + (seq & (P_NBIAS - 1)) * 1024);
    const long col0 = static_cast<long>(nb0) * 32 + wn * 64;
    const bool cols_ok = col0 < N;                // N % 64 == 0: all 64 columns or none
    const long m0 = static_cast<long>(mb0) * 32;
    const uint32_t rowb = static_cast<uint32_t>(N * OB);                     // output row bytes
    const uint32_t nrec = static_cast<uint32_t>(min(static_cast<long>(M) - m0, static_cast<long>(P_TILE))) * rowb;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(Yout) + m0 * rowb, 0, static_cast<int>(nrec), 0x00020000);
    // read-back position of this lane's two chunks: slice row rr[q2], chunk kk[q2]
    const int rr0 = lane / CPR, rr1 = (lane + 64) / CPR, kk0 = lane % CPR, kk1 = (lane + 64) % CPR;
    const uint32_t coff = static_cast<uint32_t>(col0 * OB);
    const uint32_t loff0 = rr0 * rowb + coff + kk0 * 16, loff1 = rr1 * rowb + coff + kk1 * 16;
    const int valid_rows = static_cast<int>(min(static_cast<long>(M) - m0, static_cast<long>(P_TILE)));
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int h = 0; h < 32 / RPS; h++) {
        // rows 32 j + RPS h .. of the wave's 128: held by lanes with l32 / RPS == h
        if (l32 / RPS == h) {
          const int r = l32 % RPS;
#pragma unroll
          for (int i = 0; i < 2; i++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
              // bias of tile columns 64 wn + 32 i + 8 gq + 4 lh .. + 3
              f32x4 b4 = f32x4{0.f, 0.f, 0.f, 0.f};
              if (has_bias) b4 = *reinterpret_cast<const f32x4*>(bl + wn * 64 + i * 32 + 8 * gq + 4 * lh);
              const float y0 = acc[i][j][4 * gq] + b4.x, y1 = acc[i][j][4 * gq + 1] + b4.y;
              const float y2 = acc[i][j][4 * gq + 2] + b4.z, y3 = acc[i][j][4 * gq + 3] + b4.w;
              if constexpr (OUT == SVDQ_OUT_F32) {
                const int ch = i * 8 + gq * 2 + lh;  // 16-byte chunk of the 256-byte row
                *reinterpret_cast<f32x4*>(stg + r * 256 + ((ch ^ (r % CPR)) << 4)) = f32x4{y0, y1, y2, y3};
              } else {
                const int ch = i * 4 + gq;           // 16-byte chunk of the 128-byte row; lh picks its half
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<u32x2*>(stg + r * 128 + ((ch ^ (r % CPR)) << 4) + lh * 8) =
                    u32x2{f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16),
                          f32_to_bf16_bits(y2) | (f32_to_bf16_bits(y3) << 16)};
              }
            }
        }
        __builtin_amdgcn_wave_barrier();
        // 2 KB slice: 128 chunks of 16 bytes, two per lane
        const int srow = (wm * 4 + j) * 32 + h * RPS;                       // first slice row in the tile
        const uint32_t soff = static_cast<uint32_t>(srow) * rowb;
#pragma unroll
        for (int q2 = 0; q2 < 2; q2++) {
          const int r = q2 ? rr1 : rr0, k = q2 ? kk1 : kk0;
          const u32x4 d = *reinterpret_cast<const u32x4*>(stg + r * (CPR * 16) + ((k ^ (r % CPR)) << 4));
          const uint32_t off = cols_ok && srow + r < valid_rows ? soff + (q2 ? loff1 : loff0) : nrec;
          __builtin_amdgcn_raw_buffer_store_b128(d, yr, static_cast<int>(off), 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  };

  // ---- prologue: P_AHEAD stages in flight, stage 0 published and read
  Ops oa, ob;
  if constexpr (BIG) {
#pragma unroll 1
    for (int st = 0; st < P_AHEAD; st++) {
      const Src q = stage_src(0, st, st, mb0, nb0);
#pragma unroll
      for (int i = 0; i < NCOPY; i++) copy(q, i);
    }
  } else {
#pragma unroll 1
    for (int st = 0; st < P_AHEAD; st++) {
      const Src q = ahead_src(0, st - P_AHEAD);
#pragma unroll
      for (int i = 0; i < NCOPY; i++) copy(q, i);
    }
  }
  // stage 0 complete: at least the block copies of the P_AHEAD - 1 stages
  // after it may stay in flight
  SVDQ_WAIT_VM_BARRIER(12);
#pragma unroll
  for (int p = 0; p < 6; p++) read_piece(oa, addr_of(0), p);

  // ---- per tile: S stages (the first starts the accumulators), then the
  // epilogue.  The copies run P_AHEAD stages ahead, across tile boundaries.
  long G = 0;
#pragma unroll 1
  for (; seq < my_tiles; seq++) {
    if (seq > 0) {
      mb0 = nmb0;
      nb0 = nnb0;
    }
    if (seq + 1 < my_tiles) tile_blocks(seq + 1, nmb0, nnb0);
    // Stages [from, to) of one kind, two per trip (the operand register sets
    // alternate: `c` holds the current stage's operands on entry and again
    // on exit); every run has an even length, so there is no odd tail whose
    // join would force the accumulators through VGPRs.
    auto run = [&](Ops& c, Ops& d, int from, int to, auto LR) __attribute__((always_inline)) {
#pragma unroll 1
      for (int st = from; st < to; st += 2) {
        stage(c, d, G, st, LR, std::false_type{});
        stage(d, c, G + 1, st + 1, LR, std::false_type{});
        G += 2;
      }
    };
    // One stage is peeled when rank / 16 is odd, two otherwise, which leaves
    // even-length runs (K / 64 is even).
    stage(oa, ob, G, 0, std::bool_constant<SLAB>{}, std::true_type{});
    G++;
    if constexpr (SLAB && RS_ODD) {
      run(ob, oa, 1, RS, std::true_type{});
      run(ob, oa, RS, S, std::false_type{});
    } else {
      stage(ob, oa, G, 1, std::bool_constant<SLAB>{}, std::false_type{});
      G++;
      if constexpr (SLAB) run(oa, ob, 2, RS, std::true_type{});
      run(oa, ob, SLAB ? RS : 2, S, std::false_type{});
    }
    epilogue(G - 1);
    // with one peeled stage the next tile's operands were read into ob
    if constexpr (SLAB && RS_ODD) oa = ob;
  }
  // no copy may still be writing this workgroup's LDS when it exits
  SVDQ_WAIT_VM_BARRIER(0);
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

// Compute units of the current device (cached per device): the persistent
// FP4 kernel launches at most one workgroup per CU.
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
  const int tiles = ((g.M + P_TILE - 1) / P_TILE) * ((g.N + P_TILE - 1) / P_TILE);
  dim3 grid(std::min(tiles, cu_count())), block(512);
  const bool odd = slab && ((g.rank / 16) & 1);
  const bool big = (slab ? g.rank / 16 : 0) + g.K / 64 > 7;     // more stages than the ring has in flight
#define SVDQ_F(S, O, R, B) hipLaunchKernelGGL((gemm_fp4_kernel<S, O, R, B>), grid, block, 0, st, g)
#define SVDQ_F2(S, O, R) do { if (big) SVDQ_F(S, O, R, true); else SVDQ_F(S, O, R, false); } while (0)
  if (slab) {
    if (odd) { if (f32) SVDQ_F2(true, SVDQ_OUT_F32, true); else SVDQ_F2(true, SVDQ_OUT_BF16, true); }
    else     { if (f32) SVDQ_F2(true, SVDQ_OUT_F32, false); else SVDQ_F2(true, SVDQ_OUT_BF16, false); }
  } else {
    if (f32) SVDQ_F2(false, SVDQ_OUT_F32, false); else SVDQ_F2(false, SVDQ_OUT_BF16, false);
  }
#undef SVDQ_F2
#undef SVDQ_F
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
