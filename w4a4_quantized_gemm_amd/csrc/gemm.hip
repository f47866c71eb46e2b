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
// Group 64, fp16 scales: the packed codes of each K stage are moved to LDS
// as they are stored.  An INT4 code is kept as the E4M3 bits of q * 2^-9
// (sign-magnitude: |q| <= 7 is a subnormal), two per byte, so that on the
// way from LDS to the registers one AND (codes 0-3 of a word) or one rotate
// and AND (codes 4-7) per 4 codes yields the 8-bit float operands.  One
// block-scaled 32x32x64 MFMA with E4M3 operands and both block scales 2^9
// then gives the group's P_g = sum_k q_x q_w exactly in fp32, a 32x32x8 f16
// MFMA with one nonzero K slot gives the tile's scale products s_x[i]
// s_w[j] (exact in fp32, in the accumulator layout), and the group is
// dequantized with one fma per accumulator.  That fma (16 per 32 x 32 tile
// and group) is VALU work, which bounds this variant below the 8-bit MFMA
// peak.  The MFMAs of the next output tile are issued before the
// dequantization of the current one, so the matrix core and the VALU
// overlap.
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

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E4M3 operand bytes of 16 bytes of INT4 codes: codes 0-3 of each word are
// bits 7 and 0-2 of its bytes, codes 4-7 the same positions rotated left by
// 4 bits.
__device__ __forceinline__ u32x4 e4m3_lo(const u32x4& c) {
  constexpr uint32_t MSK = 0x87878787u;
  return u32x4{c.x & MSK, c.y & MSK, c.z & MSK, c.w & MSK};
}
__device__ __forceinline__ u32x4 e4m3_hi(const u32x4& c) {
  constexpr uint32_t MSK = 0x87878787u;
  return u32x4{__builtin_amdgcn_alignbit(c.x, c.x, 4) & MSK, __builtin_amdgcn_alignbit(c.y, c.y, 4) & MSK,
               __builtin_amdgcn_alignbit(c.z, c.z, 4) & MSK, __builtin_amdgcn_alignbit(c.w, c.w, 4) & MSK};
}

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

// Tile: 4 waves in a 2 x 2 grid, each owning 64 x 64 (2 x 2 MFMA tiles).
// The per-group dequantization updates the accumulators with VALU fma, so
// they are VGPRs; 128 x 128 per workgroup.  About 300 registers per lane:
// one wave per SIMD, one workgroup per CU (a bound to two waves per SIMD
// fits in 256 without spilling but measured no faster).
constexpr int RB = 2, CB = 2;                      // 32-row (-column) blocks per wave
constexpr int BM = 2 * RB * 32, BN = 2 * CB * 32;
constexpr int NTHREADS = 256;
constexpr int A_CH = BM * 4 / NTHREADS, B_CH = BN * 4 / NTHREADS;   // 16-byte code pieces per thread and stage

// LDS layout of one K stage (128 K values) of one operand: the codes are
// widened to E4M3 operand bytes once, as they are stored.  The 2 KB block of
// (32-row block rb, 64-wide step j) sits at (rb * 2 + j) * 2 KB; lane l of an
// MFMA finds the bytes of codes 0-3 of its four words at l * 16 and those of
// codes 4-7 at 1 KB + l * 16, so stores and reads are contiguous.  Both
// operands use the same byte order, which is all the MFMA's K sum needs.
__device__ __forceinline__ int lds_block(int rowblk, int j) { return (rowblk * 2 + j) << 11; }

template <bool SLAB, int OUT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int STAGE_A = (BM / 32) * 2 * 2048, STAGE_B = (BN / 32) * 2 * 2048;
  // LDS: two stage buffers of A and B operands plus the scales as f16 MFMA
  // operand words ([stage][group][row]: fp16 bits in the low half); the
  // epilogue reuses the operand buffers to stage the output tile.
  constexpr int LDS_A = 2 * STAGE_A, LDS_B = 2 * STAGE_B;
  constexpr int LDS_SA = 2 * 2 * BM * 4, LDS_SB = 2 * 2 * BN * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_A + LDS_B + LDS_SA + LDS_SB];
  auto sA = reinterpret_cast<uint8_t(*)[STAGE_A]>(smem);
  auto sB = reinterpret_cast<uint8_t(*)[STAGE_B]>(smem + LDS_A);
  auto sSA = reinterpret_cast<uint32_t(*)[2][BM]>(smem + LDS_A + LDS_B);
  auto sSB = reinterpret_cast<uint32_t(*)[2][BN]>(smem + LDS_A + LDS_B + LDS_SA);

  // kernel arguments in registers (a lambda capturing g would read them
  // from the argument segment with vector loads)
  const int M = g.M, K = g.K, N = g.N, rank = g.rank;
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
  const int lane = t & 63, wave = wave_uniform(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
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

  // ---- global -> registers -> LDS, through buffer resources over the
  // workgroup's own row blocks (32-bit offsets; the stage is the scalar
  // offset).  A stage of the A (B) tile is BM / 16 (BN / 16) operand blocks
  // of 1 KB; thread t copies 16-byte pieces q = t + 256 i: block q / 64, lane
  // slot q % 64 (64 threads cover one block contiguously).  Row blocks past
  // the matrix are clamped to its last one (their outputs are never
  // stored).  Waves 0-1 load the scale words of the 128 A rows, waves 2-3
  // those of the 128 B columns.
  struct Regs {
    u32x4 a[A_CH], b[B_CH];
    uint32_t sc;
  };
  const long KBLK = K / 64;                       // 1 KB blocks per 32-row block
  const int a_blks = static_cast<int>(min(static_cast<long>(BM / 32), (M + 31) / 32 - m0 / 32));
  const int b_blks = static_cast<int>(min(static_cast<long>(BN / 32), N / 32 - n0 / 32));
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.acodes + (m0 / 32) * KBLK * 1024), 0, static_cast<int>(a_blks * KBLK * 1024), 0x00020000);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.wcodes + (n0 / 32) * KBLK * 1024), 0, static_cast<int>(b_blks * KBLK * 1024), 0x00020000);
  uint32_t aoff[A_CH], boff[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; i++) {
    const int q = t + i * NTHREADS, blk = q >> 6;
    aoff[i] = static_cast<uint32_t>(((min(blk >> 1, a_blks - 1) * KBLK + (blk & 1)) << 10) + (q & 63) * 16);
  }
#pragma unroll
  for (int i = 0; i < B_CH; i++) {
    const int q = t + i * NTHREADS, blk = q >> 6;
    boff[i] = static_cast<uint32_t>(((min(blk >> 1, b_blks - 1) * KBLK + (blk & 1)) << 10) + (q & 63) * 16);
  }
  // scale words: activation scales in 32-row blocks (word (row, st) at
  // ((row / 32) * SW + st) * 32 + row % 32), weight scales row-major
  const bool sc_is_a = wave < 2;
  __amdgpu_buffer_rsrc_t sr;
  uint32_t soff;
  int sstep;
  if (sc_is_a) {
    const long rows = min(static_cast<long>(BM), static_cast<long>(M) - m0);
    const long r = min(static_cast<long>(t), rows - 1);
    sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const uint32_t*>(g.ascales) + (m0 >> 5) * SW * 32)), 0,
        static_cast<int>(((rows + 31) >> 5) * SW * 128), 0x00020000);
    soff = static_cast<uint32_t>(((r >> 5) * SW * 32 + (r & 31)) * 4);
    sstep = 128;
  } else {
    const long cols = min(static_cast<long>(BN), static_cast<long>(N) - n0);
    const long c = min(static_cast<long>(t - BM), cols - 1);
    sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const uint32_t*>(g.wscales) + n0 * SW)), 0,
        static_cast<int>(cols * SW * 4), 0x00020000);
    soff = static_cast<uint32_t>(c * SW * 4);
    sstep = 4;
  }
  auto load_stage = [&](Regs& r, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; i++) r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], st * 2048, 0);
#pragma unroll
    for (int i = 0; i < B_CH; i++) r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(br, boff[i], st * 2048, 0);
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(sr, soff, st * sstep, 0);
  };
  auto store_stage = [&](const Regs& r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CH; i++) {
      const int q = t + i * NTHREADS, off = ((q >> 6) << 11) + (q & 63) * 16;
      *reinterpret_cast<u32x4*>(&sA[buf][off]) = e4m3_lo(r.a[i]);
      *reinterpret_cast<u32x4*>(&sA[buf][off + 1024]) = e4m3_hi(r.a[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; i++) {
      const int q = t + i * NTHREADS, off = ((q >> 6) << 11) + (q & 63) * 16;
      *reinterpret_cast<u32x4*>(&sB[buf][off]) = e4m3_lo(r.b[i]);
      *reinterpret_cast<u32x4*>(&sB[buf][off + 1024]) = e4m3_hi(r.b[i]);
    }
    // fp16 bits of the two groups' scales, as the f16 MFMA operands take them
    uint32_t(*ss)[BM] = sc_is_a ? sSA[buf] : sSB[buf];
    const int idx = sc_is_a ? t : t - BM;
    ss[0][idx] = r.sc & 0xFFFFu;
    ss[1][idx] = r.sc >> 16;
  };

  // Stage k's codes are loaded into register set R[k % 2].  Schedule of
  // stage s: (1) store register set R[(s + 1) % 2] (stage s + 1, loaded two
  // stages earlier) to the other LDS buffer, (2) reuse that set for the
  // global loads of stage s + 3, (3) run the MFMAs of stage s, (4) barrier.
  // Loads past the last stage re-read the last stage (their data is never
  // used), so that every stage issues the same loads and the compiler's
  // wait counts stay exact across the loop.
  // The prologue issues its loads stage by stage (no interleaving), in the
  // same order as the loop, so that the compiler's load counters agree at
  // the loop head and each wait covers exactly the stage it needs.
  Regs R0, R1;
  const int last = stages - 1;
  load_stage(R0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(R1, min(1, last));
  __builtin_amdgcn_sched_barrier(0);
  store_stage(R0, 0);
  load_stage(R0, min(2, last));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  auto stage_body = [&](int s, Regs& Rn, auto BUF) __attribute__((always_inline)) {
    constexpr int buf = decltype(BUF)::value;
    store_stage(Rn, buf ^ 1);
    load_stage(Rn, min(s + 3, last));
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < 2; j++) {          // two 64-wide MFMA steps per stage
      // E4M3 operands (codes 0-3 of the lane's words, then codes 4-7) and
      // the scale operands of the f16 MFMA that forms the tile's scale
      // products: every lane holds its row's (column's) fp16 scale in its
      // first element, so K slots 0 and 4 both carry s_x[i] s_w[j] and the
      // MFMA gives 2 s_x[i] s_w[j] (exact); the E4M3 MFMA's block scales
      // (2^9, 2^8) give P_g / 2 to match.
      i32x8 a8[RB], b8[CB];
      f16x4 fa[RB], fb[CB];
#pragma unroll
      for (int rb = 0; rb < RB; rb++) {
        const int o = lds_block(wrow0 / 32 + rb, j) + lane * 16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&sA[buf][o]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&sA[buf][o + 1024]);
        a8[rb] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        fa[rb] = __builtin_bit_cast(f16x4, u32x2{sSA[buf][j][wrow0 + rb * 32 + l32], 0u});
      }
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const int o = lds_block(wcol0 / 32 + cb, j) + lane * 16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&sB[buf][o]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&sB[buf][o + 1024]);
        b8[cb] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        fb[cb] = __builtin_bit_cast(f16x4, u32x2{sSB[buf][j][wcol0 + cb * 32 + l32], 0u});
      }
      // software pipeline over the wave's output tiles: the MFMAs of tile
      // u + 1 (P_g / 2 = sum q_x q_w / 2, exact in fp32: codes are q 2^-9;
      // and 2 s_x s_w) are in flight while tile u is dequantized with one fma
      // per accumulator (the product of the two is P_g s_x s_w exactly)
      constexpr int NT = RB * CB;
      f32x16 p[2], sp[2];
      auto mma = [&](int u, f32x16& dst, f32x16& sdst) __attribute__((always_inline)) {
        const int rb = u / CB, cb = u % CB;
        f32x16 zf;
#pragma unroll
        for (int v = 0; v < 16; v++) zf[v] = 0.f;
        dst = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[rb], b8[cb], zf, 0, 0, 0, 127 + 9, 0, 127 + 8);
        sdst = __builtin_amdgcn_mfma_f32_32x32x8f16(fa[rb], fb[cb], zf, 0, 0, 0);
      };
      mma(0, p[0], sp[0]);
#pragma unroll
      for (int u = 0; u < NT; u++) {
        const int rb = u / CB, cb = u % CB;
        if (u + 1 < NT) mma(u + 1, p[(u + 1) & 1], sp[(u + 1) & 1]);
        const f32x16& pp = p[u & 1];
        const f32x16& ss = sp[u & 1];
#pragma unroll
        for (int v = 0; v < 16; v++) acc[rb][cb][v] = __builtin_fmaf(pp[v], ss[v], acc[rb][cb][v]);
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
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    dim3 grid(tiles), block(256);
#define SVDQ_G(S, O) hipLaunchKernelGGL((gemm_kernel<S, O>), grid, block, 0, st, g)
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
