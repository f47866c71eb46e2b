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
// Group 64, fp16 scales.  An INT4 code is kept as the E4M3 bits of q * 2^-9
// (sign-magnitude: |q| <= 7 is a subnormal), two per byte, so that on the
// way from LDS to the registers one AND (codes 0-3 of a word) or one rotate
// and AND (codes 4-7) per 4 codes yields the 8-bit float operands.  One
// block-scaled 32x32x64 MFMA with E4M3 operands and both block scales 2^9
// then gives the group's P_g = sum_k q_x q_w exactly in fp32, a 32x32x8 f16
// MFMA with one nonzero K slot gives the tile's scale products s_x[i]
// s_w[j] (exact in fp32, in the accumulator layout), and the group is
// dequantized with one fma per accumulator.  That fma (16 per 32 x 32 tile
// and group) is VALU work, which bounds this variant below the 8-bit MFMA
// peak.  The E4M3 MFMA of the next output tile is issued before the
// dequantization of the current one and its f16 MFMA after it, so each
// MFMA executes under VALU work (a wave issues in order, and a second MFMA
// would wait for the matrix core with the VALU work behind it); operand
// parts are read from LDS one MFMA slot before they are widened, so no
// read's latency stalls the wave right after the read.
//
// Tiling: 4 waves per workgroup in a 2 x 2 grid, 128 x 128 per workgroup,
// 32 x 32 MFMA tiles.  A K stage is 128 wide (two 64-wide MFMA steps): its
// raw codes (the 1 KB operand blocks as they lie in HBM) and scales are
// copied global -> LDS directly (global_load_lds, 16 bytes per lane) into a
// ring of 4 stage buffers, 3 stages ahead of the MFMAs, and widened as each
// wave reads its operands; each stage has one barrier.  In every MFMA, lane
// l owns row (column) l % 32 and the 16-byte half l / 32 of the 64-wide K
// step, for A and B alike, so both operands enumerate K in the same order.
// Workgroups are mapped to tiles so that the workgroups resident on one XCD
// (the hardware deals them round-robin to the 8 XCDs) share rows of A or
// columns of B in that XCD's L2.
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

}  // namespace

// Tile: 4 waves in a 2 x 2 grid, each owning 64 x 64 (2 x 2 MFMA tiles).
// The per-group dequantization updates the accumulators with VALU fma, so
// they are VGPRs; 128 x 128 per workgroup.  About 300 registers per lane:
// one wave per SIMD, one workgroup per CU (a bound to two waves per SIMD
// fits in 256 without spilling but measured no faster).
constexpr int RB = 2, CB = 2;                      // 32-row (-column) blocks per wave
constexpr int BM = 2 * RB * 32, BN = 2 * CB * 32;

// LDS layout of one K stage (128 K values) of one operand: the codes are
// widened to E4M3 operand bytes once, as they are stored.  The 2 KB block of
// (32-row block rb, 64-wide step j) sits at (rb * 2 + j) * 2 KB; lane l of an
// MFMA finds the bytes of codes 0-3 of its four words at l * 16 and those of
// codes 4-7 at 1 KB + l * 16, so stores and reads are contiguous.  Both
// operands use the same byte order, which is all the MFMA's K sum needs.
__device__ __forceinline__ int lds_block(int rowblk, int j) { return (rowblk * 2 + j) << 11; }

template <bool SLAB, int OUT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  // LDS: a ring of NBUF stages, each the raw codes of the tile's rows and
  // columns for 128 K (A then B: per 32-row block the two 1 KB operand
  // blocks of the stage, as they lie in HBM) and their scales (A: the 128-byte
  // scale blocks of the four 32-row blocks; B: one 4-byte word per column);
  // the epilogue reuses the ring to stage the output tile.
  constexpr int RING_A = 0, RING_B = (BM / 32) * 2048, RING_SA = RING_B + (BN / 32) * 2048;
  constexpr int RING_SB = RING_SA + (BM / 32) * 128, RING_STAGE = RING_SB + BN * 4;
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * RING_STAGE];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)smem));

  // kernel arguments in registers (a lambda capturing g would read them
  // from the argument segment with vector loads)
  const int M = g.M, K = g.K, N = g.N, rank = g.rank;
  const uint16_t* __restrict__ Tb = g.Tb;
  const uint16_t* __restrict__ l2t = g.l2t;
  const float* __restrict__ bias = g.bias;
  void* __restrict__ Yout = g.Y;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, g.xcd_map, tm, tn);
  const long m0 = static_cast<long>(tm) * BM;
  const long n0 = static_cast<long>(tn) * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = wave_uniform(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31;
  const int lh = lane >> 5;
  const int SW = K / 128;                        // scale words (4 bytes) per row
  // K part of this workgroup (grid.y parts; one unless the launch splits K):
  // stages [s_begin, s_begin + stages) of the K / 128
  const int part = static_cast<int>(blockIdx.y), kparts = g.kparts;
  const int s_begin = part * SW / kparts;
  const int stages = (part + 1) * SW / kparts - s_begin;
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
    // (the first K part only)
    for (int tb = 0; tb < (part == 0 ? rank / 16 : 0); tb++) {
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

  // ---- global -> LDS copies (global_load_lds, 16 or 4 bytes per lane) of
  // the raw codes and scales, NBUF - 1 stages ahead of the MFMAs.  Per stage
  // wave w copies: the two 1 KB blocks of A row block w, those of B column
  // block w, and a quarter of the scales (waves 0-1: A scale blocks 2w,
  // 2w + 1; waves 2-3: B scale words of 64 columns each).  Row (column)
  // blocks past the matrix repeat its last one (never stored); stages past
  // the last repeat the last one (never consumed), so every stage issues the
  // same 5 copies per wave and the explicit waits count exactly.
  const long KBLK = K / 64;                       // 1 KB blocks per 32-row block
  const int last_ablk = (M + 31) / 32 - 1, last_bblk = N / 32 - 1;
  const int last = stages - 1;
  // (the bases start at the part's first stage: 2 KB of codes per stage)
  const uint8_t* cpa = g.acodes + ((static_cast<long>(min(static_cast<int>(m0 / 32) + wave, last_ablk)) * KBLK) << 10) +
                       static_cast<long>(s_begin) * 2048;
  const uint8_t* cpb = g.wcodes + ((static_cast<long>(min(static_cast<int>(n0 / 32) + wave, last_bblk)) * KBLK) << 10) +
                       static_cast<long>(s_begin) * 2048;
  const uint8_t* cps;
  uint32_t svoff, sstride;
  if (wave < 2) {
    // A scale blocks: per 32-row block and stage 128 bytes at ((row block) *
    // SW + st) * 128; lanes 0-31 block 2w, lanes 32-63 block 2w + 1
    const int rb = min(static_cast<int>(m0 / 32) + 2 * wave + (lane >> 5), last_ablk);
    cps = static_cast<const uint8_t*>(g.ascales);
    svoff = static_cast<uint32_t>(rb * SW * 128 + (lane & 31) * 4);
    sstride = 128;
  } else {
    // B scale words: column n's two fp16 scales of stage st at (n * SW + st) * 4
    const long c = min(n0 + (wave - 2) * 64 + lane, static_cast<long>(N - 1));
    cps = static_cast<const uint8_t*>(g.wscales);
    svoff = static_cast<uint32_t>(c * SW * 4);
    sstride = 4;
  }
  svoff += static_cast<uint32_t>(s_begin) * sstride;
  const uint32_t lane16 = lane * 16u;
  const uint32_t sdst = wave < 2 ? RING_SA + wave * 256 : RING_SB + (wave - 2) * 256;
  // copy item i (0..4) of stage st into ring slot st % NBUF
  auto copy_item = [&](int st, int i) __attribute__((always_inline)) {
    const int cs = min(st, last);
    const uint32_t slot = lds0 + static_cast<uint32_t>(st % NBUF) * RING_STAGE;
    switch (i) {
      case 0: set_m0_nop(slot + RING_A + wave * 2048); dma16<0>(cpa + cs * 2048, lane16); break;
      case 1: dma16<1024>(cpa + cs * 2048, lane16); break;
      case 2: set_m0_nop(slot + RING_B + wave * 2048); dma16<0>(cpb + cs * 2048, lane16); break;
      case 3: dma16<1024>(cpb + cs * 2048, lane16); break;
      default: set_m0_nop(slot + sdst); dma4<0>(cps, svoff + static_cast<uint32_t>(cs) * sstride); break;
    }
  };

  // Operands of one 64-wide MFMA step, read from the ring and widened: the
  // E4M3 operand words of the wave's row blocks (A) and column blocks (B) --
  // codes 0-3 of the lane's words, then codes 4-7 -- and the operands of the
  // f16 MFMA that forms the tile's scale products: every lane holds its row's
  // (column's) fp16 scale in its first element, so K slots 0 and 4 both
  // carry s_x[i] s_w[j] and the MFMA gives 2 s_x[i] s_w[j] (exact); the E4M3
  // MFMA's block scales (2^9, 2^8) give P_g / 2 to match.
  struct Ops {
    i32x8 a[RB], b[CB];
    f16x4 fa[RB], fb[CB];
  };
  // part p of the operands of step j of stage st: p < RB row block p, else
  // column block p - RB
  // Per-lane LDS addresses of a ring slot, made opaque so that the
  // compiler keeps them in two registers per slot and puts every block's
  // constant offset into the read instruction (it would otherwise add each
  // one to the slot offset separately).
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  struct Bases {
    uint32_t a, b, sa, sb;    // this wave's first A / B code block and scales in the slot
  };
  auto bases_of = [&](int st) __attribute__((always_inline)) {
    Bases r;
    const uint32_t slot = lds0 + static_cast<uint32_t>(st % NBUF) * RING_STAGE;
    r.a = slot + RING_A + static_cast<uint32_t>(wrow0 / 32) * 2048u + lane16;
    r.b = slot + RING_B + static_cast<uint32_t>(wcol0 / 32) * 2048u + lane16;
    r.sa = slot + RING_SA + static_cast<uint32_t>(wrow0 / 32) * 128u + static_cast<uint32_t>(l32) * 4u;
    r.sb = slot + RING_SB + static_cast<uint32_t>(wcol0 / 32) * 128u + static_cast<uint32_t>(l32) * 4u;
    asm volatile("" : "+v"(r.a), "+v"(r.b), "+v"(r.sa), "+v"(r.sb));
    return r;
  };
  auto lds_at = [](uint32_t addr) __attribute__((always_inline)) {
    return reinterpret_cast<lds_u8*>(static_cast<uintptr_t>(addr));
  };
  // An operand part is read raw (codes and scale) in one MFMA slot and
  // widened in the next, so the read's latency passes under that slot's
  // MFMAs and fmas instead of stalling the wave right after the read.
  struct Raw {
    u32x4 c;
    uint32_t sc;
  };
  auto read_raw = [&](Raw& r, const Bases& bs, int j, int p) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) const uint16_t lds_u16;
    if (p < RB) {
      r.c = *reinterpret_cast<lds_u32x4*>(lds_at(bs.a) + (p * 2 + j) * 1024);
      r.sc = *reinterpret_cast<lds_u16*>(lds_at(bs.sa) + p * 128 + j * 2);
    } else {
      r.c = *reinterpret_cast<lds_u32x4*>(lds_at(bs.b) + ((p - RB) * 2 + j) * 1024);
      r.sc = *reinterpret_cast<lds_u16*>(lds_at(bs.sb) + (p - RB) * 128 + j * 2);
    }
  };
  auto widen = [&](Ops& o, const Raw& r, int p) __attribute__((always_inline)) {
    const u32x4 lo = e4m3_lo(r.c), hi = e4m3_hi(r.c);
    const i32x8 v = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const f16x4 f = __builtin_bit_cast(f16x4, u32x2{r.sc, 0u});
    if (p < RB) {
      o.a[p] = v;
      o.fa[p] = f;
    } else {
      o.b[p - RB] = v;
      o.fb[p - RB] = f;
    }
  };

  // The MFMAs of output tile u of a step (P_g / 2 = sum q_x q_w / 2, exact
  // in fp32: codes are q 2^-9; and 2 s_x s_w) go to result slot u % 2; the
  // tile is retired (dequantized into its accumulators, one fma per value:
  // the product of the two is P_g s_x s_w exactly) after the next tile's
  // MFMAs are issued, across step and stage boundaries, so the matrix core
  // and the VALU overlap continuously.  Slot 1 starts at zero: the first
  // retirement (of a "previous" tile 3) adds 0 * 0 to its accumulators.
  constexpr int NT = RB * CB;
  static_assert(NT == 4, "the schedule below retires tile NT - 1 of the previous step first");
  static_assert(RB + CB == NT, "one operand part is read per MFMA slot");
  f32x16 P[2], Sc[2];
#pragma unroll
  for (int v = 0; v < 16; v++) P[1][v] = Sc[1][v] = 0.f;
  auto issue_p = [&](const Ops& o, int u, int slot) __attribute__((always_inline)) {
    const int rb = u / CB, cb = u % CB;
    f32x16 zf;
#pragma unroll
    for (int v = 0; v < 16; v++) zf[v] = 0.f;
    P[slot] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[rb], o.b[cb], zf, 0, 0, 0, 127 + 9, 0, 127 + 8);
  };
  auto issue_s = [&](const Ops& o, int u, int slot) __attribute__((always_inline)) {
    const int rb = u / CB, cb = u % CB;
    f32x16 zf;
#pragma unroll
    for (int v = 0; v < 16; v++) zf[v] = 0.f;
    Sc[slot] = __builtin_amdgcn_mfma_f32_32x32x8f16(o.fa[rb], o.fb[cb], zf, 0, 0, 0);
  };
  auto retire = [&](int u, int slot) __attribute__((always_inline)) {
    const int rb = u / CB, cb = u % CB;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[rb][cb][v] = __builtin_fmaf(P[slot][v], Sc[slot][v], acc[rb][cb][v]);
  };

  // Schedule of stage s (its codes in ring slot s % NBUF; its step-0
  // operands already in registers):
  //   step 0: per output tile its MFMAs, the fmas of the previous tile, the
  //           reads of a quarter of step 1's operands, one copy item of stage
  //           s + 3 (into the slot stage s - 1 released);
  //   wait + barrier: this wave's copies of stage s + 1 are complete once at
  //           most those of stages s + 2 and s + 3 (10) are outstanding, the
  //           barrier publishes stage s + 1 and every wave is done reading
  //           stage s - 1 ... s;
  //   step 1: the same with step 0's operands of stage s + 1.
  constexpr int NCOPY = 5;
  static_assert(NCOPY == NT + 1, "one copy per tile slot of step 0, the fifth with the last");
#pragma unroll 1
  for (int p = 0; p < NBUF - 1; p++)
#pragma unroll
    for (int i = 0; i < NCOPY; i++) copy_item(p, i);
  SVDQ_VM_BARRIER(10);
  Ops OA, OB;
  // bases of ring slot 0 (opaque); slot k is slot 0 + k * RING_STAGE, a
  // constant offset where k is known at compile time
  const Bases base0 = bases_of(0);
  auto slot_bases = [&](int k) __attribute__((always_inline)) {
    const uint32_t o = static_cast<uint32_t>(k) * RING_STAGE;
    return Bases{base0.a + o, base0.b + o, base0.sa + o, base0.sb + o};
  };
  Raw raw[2];
#pragma unroll
  for (int p = 0; p < RB + CB - 1; p++) {
    read_raw(raw[0], base0, 0, p);
    widen(OA, raw[0], p);
  }
  read_raw(raw[1], base0, 0, RB + CB - 1);     // widened in the first slot of the loop
  // stage s with the bases of its slot (bs) and of the next stage's (bn)
  auto stage_body = [&](int s, const Bases& bs, const Bases& bn) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NT; u++) {
        // the fences keep the order: the E4M3 MFMA, the fmas of the previous
        // tile (they run while it executes), the f16 MFMA, then the reads,
        // widening and copies (they run while that one executes).  A wave
        // issues in order and a second MFMA waits for the matrix core, so two
        // MFMAs back to back would hold the VALU work behind them.
        issue_p(OA, u, u & 1);
        __builtin_amdgcn_sched_barrier(0);
        retire(u == 0 ? NT - 1 : u - 1, (u + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        issue_s(OA, u, u & 1);
        __builtin_amdgcn_sched_barrier(0);
        // part u of OB is read; the part read in the previous slot is
        // widened (in slot 0: OA's last part, read in the previous step)
        read_raw(raw[u & 1], bs, 1, u);
        if (u == 0) widen(OA, raw[1], NT - 1);
        else widen(OB, raw[(u - 1) & 1], u - 1);
        copy_item(s + NBUF - 1, u);
        if (u == NT - 1) copy_item(s + NBUF - 1, NT);
        __builtin_amdgcn_sched_barrier(0);
      }
      SVDQ_VM_BARRIER(10);
#pragma unroll
      for (int u = 0; u < NT; u++) {
        issue_p(OB, u, u & 1);
        __builtin_amdgcn_sched_barrier(0);
        retire(u == 0 ? NT - 1 : u - 1, (u + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        issue_s(OB, u, u & 1);
        __builtin_amdgcn_sched_barrier(0);
        read_raw(raw[u & 1], bn, 0, u);
        if (u == 0) widen(OB, raw[1], NT - 1);
        else widen(OA, raw[(u - 1) & 1], u - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // unrolled by the ring depth so that every slot offset is a constant of
  // the read instructions; the remaining stages with computed bases
  int s = 0;
#pragma unroll 1
  for (; s + NBUF <= stages; s += NBUF) {
    static_assert(NBUF == 4, "the unrolled loop walks four ring slots");
    stage_body(s, slot_bases(0), slot_bases(1));
    stage_body(s + 1, slot_bases(1), slot_bases(2));
    stage_body(s + 2, slot_bases(2), slot_bases(3));
    stage_body(s + 3, slot_bases(3), slot_bases(0));
  }
#pragma unroll 1
  for (; s < stages; s++) stage_body(s, bases_of(s), bases_of(s + 1));
  retire(NT - 1, 1);
  // no copy may still be writing the ring, and every wave is done reading
  // it, before the epilogue stages its output there
  SVDQ_VM_BARRIER(0);

  // ---- K split: the part's fp32 partial tile (no bias) goes to the
  // workspace, row-major 128 x 128 per (part, tile); gemm_ysum_kernel adds
  // the parts
  if (kparts > 1) {
    float* yp = g.ypart + (static_cast<long>(part) * tiles_m * tiles_n + static_cast<long>(tm) * tiles_n + tn) *
                              (BM * BN);
#pragma unroll
    for (int rb = 0; rb < RB; rb++)
#pragma unroll
      for (int cb = 0; cb < CB; cb++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int row = wrow0 + rb * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          yp[row * BN + wcol0 + cb * 32 + l32] = acc[rb][cb][v];
        }
    return;
  }

  // ---- epilogue: bias, rounding, store.  Each wave stages one 32-row
  // slice of its tile at a time in its own LDS region (row-major, output
  // type), then writes whole rows with 16-byte stores.
  {
    constexpr int OB = OUT == SVDQ_OUT_F32 ? 4 : 2;     // output bytes per element
    constexpr int ROWB = CB * 32 * OB;                  // bytes of one slice row
    constexpr int SLICE = 32 * ROWB;
    static_assert(4 * SLICE <= NBUF * RING_STAGE, "epilogue staging must fit the ring");
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

// K-split epilogue: Y = round(sum over the parts, in part order, of the
// fp32 partial tiles + b); one thread per 4 consecutive columns of a row
// (N % 32 == 0, so the 4 lie in one tile).
template <int OUT>
__global__ __launch_bounds__(256) void gemm_ysum_kernel(const float* __restrict__ ypart, int kparts, int M, int N,
                                                        const float* __restrict__ bias, void* __restrict__ Y) {
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (idx >= static_cast<long>(M) * n4) return;
  const long row = idx / n4;
  const int col = static_cast<int>(idx - row * n4) * 4;
  const int tiles_n = (N + BN - 1) / BN;
  const long tiles = (static_cast<long>(M) + BM - 1) / BM * tiles_n;
  const long tile = row / BM * tiles_n + col / BN;
  const float* p = ypart + tile * (BM * BN) + (row % BM) * BN + col % BN;
  f32x4 s = *reinterpret_cast<const f32x4*>(p);
  for (int q = 1; q < kparts; q++) s += *reinterpret_cast<const f32x4*>(p + q * tiles * (BM * BN));
  if (bias) s += *reinterpret_cast<const f32x4*>(bias + col);
  if constexpr (OUT == SVDQ_OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(Y) + row * N + col) = s;
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Y) + row * N + col) =
        u32x2{f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16), f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16)};
  }
}

// Unfused up-projection: Y = round(Y + Tb L2b) in place, the separate second
// pass of the naive pipeline (re-reads and re-writes the 16-bit output).  It
// is HBM-bound (Y is read and written once; Tb and L2b are small), so a
// workgroup owns 64 rows x 128 columns: the Y loads (16 bytes per lane, whole
// rows) are issued first, the low-rank tile is computed meanwhile on the
// bf16 MFMA (wave w: column block w, both 32-row blocks) and staged in LDS
// as fp32, then every lane adds it to its Y pieces, rounds and stores them
// (16 bytes per lane).  Rows past M and columns past N are neither read nor
// written (buffer offsets past the resource).
template <int OUT>
__global__ __launch_bounds__(256) void up_kernel(const uint16_t* __restrict__ Tb, const uint16_t* __restrict__ l2t,
                                                 void* __restrict__ Y, int M, int N, int rank) {
  constexpr int OB = OUT == SVDQ_OUT_F32 ? 4 : 2;       // output bytes per element
  constexpr int ROWB = 128 * OB;                        // bytes of one tile row
  constexpr int PIECES = 64 * ROWB / 16 / 256;          // 16-byte pieces per thread
  __shared__ __attribute__((aligned(16))) float low[64][128 + 4];
  const int tiles_n = (N + 127) / 128;
  const long m0 = static_cast<long>(blockIdx.x / tiles_n) * 64;
  const long n0 = static_cast<long>(blockIdx.x % tiles_n) * 128;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int rows = static_cast<int>(min(static_cast<long>(M) - m0, 64L));
  const int cols = static_cast<int>(min(static_cast<long>(N) - n0, 128L));
  const uint32_t gro = static_cast<uint32_t>(N) * OB;   // global row bytes
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<uint8_t*>(Y) + (m0 * N + n0) * OB, 0, static_cast<int>(static_cast<uint32_t>(rows - 1) * gro + cols * OB),
      0x00020000);
  // piece q = t + 256 i: tile row q / (ROWB / 16), 16-byte column piece q % (ROWB / 16)
  uint32_t off[PIECES];
  u32x4 y[PIECES];
#pragma unroll
  for (int i = 0; i < PIECES; i++) {
    const int q = t + 256 * i, r = q / (ROWB / 16), c = q % (ROWB / 16);
    const bool ok = r < rows && c * 16 < cols * OB;
    off[i] = ok ? static_cast<uint32_t>(r) * gro + c * 16 : 0x80000000u;
    y[i] = __builtin_amdgcn_raw_buffer_load_b128(yr, off[i], 0, 0);
  }
  // low-rank tile: column block `wave`, row blocks 0 and 1 (rows and
  // columns past the matrix clamp to its last one; never stored)
  f32x16 acc[2];
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int v = 0; v < 16; v++) acc[rb][v] = 0.f;
  const long c = min(n0 + wave * 32 + l32, static_cast<long>(N - 1));
  for (int tb = 0; tb < rank / 16; tb++) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(l2t + bf16_block_index(c, tb * 16 + lh * 8, rank));
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      const long r = min(m0 + rb * 32 + l32, static_cast<long>(M - 1));
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Tb + bf16_block_index(r, tb * 16 + lh * 8, rank));
      acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[rb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int v = 0; v < 16; v++) low[rb * 32 + 8 * (v >> 2) + 4 * lh + (v & 3)][wave * 32 + l32] = acc[rb][v];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PIECES; i++) {
    const int q = t + 256 * i, r = q / (ROWB / 16), c0 = (q % (ROWB / 16)) * (16 / OB);
    u32x4 o;
    if constexpr (OUT == SVDQ_OUT_F32) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&low[r][c0]);
      o = u32x4{__float_as_uint(__uint_as_float(y[i].x) + l4.x), __float_as_uint(__uint_as_float(y[i].y) + l4.y),
                __float_as_uint(__uint_as_float(y[i].z) + l4.z), __float_as_uint(__uint_as_float(y[i].w) + l4.w)};
    } else {
      const f32x4 la = *reinterpret_cast<const f32x4*>(&low[r][c0]);
      const f32x4 lb = *reinterpret_cast<const f32x4*>(&low[r][c0 + 4]);
      const uint32_t w[4] = {y[i].x, y[i].y, y[i].z, y[i].w};
      const float l8[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
      uint32_t out[4];
#pragma unroll
      for (int e = 0; e < 4; e++)
        out[e] = f32_to_bf16_bits(bf16_lo(w[e]) + l8[2 * e]) | (f32_to_bf16_bits(bf16_hi(w[e]) + l8[2 * e + 1]) << 16);
      o = u32x4{out[0], out[1], out[2], out[3]};
    }
    __builtin_amdgcn_raw_buffer_store_b128(o, yr, off[i], 0, 0);
  }
}

int gemm_xcd_map(int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr double L2_SLICE = 3.0 * (1 << 20);   // of the 4 MB L2 of an XCD
  const double a = static_cast<double>(M) * K / 2 / 8, b = static_cast<double>(N) * K / 2 / 8;
  const bool cols = tiles_n % 8 == 0 && b <= L2_SLICE;
  const bool rows = tiles_m % 8 == 0 && a <= L2_SLICE;
  if (cols && (!rows || b <= a)) return 1;
  if (rows) return 2;
  return 0;
}

hipError_t launch_gemm(int fmt, bool slab, int out_dtype, const GemmArgs& ga, hipStream_t st) {
  const bool f32 = out_dtype == SVDQ_OUT_F32;
  if (fmt == SVDQ_INT4_G64_FP16) {
    const int tiles_m = (ga.M + BM - 1) / BM, tiles_n = (ga.N + BN - 1) / BN;
    GemmArgs g = ga;
    g.xcd_map = gemm_xcd_map(g.M, g.N, g.K, tiles_m, tiles_n);
    // K split where the tiles leave at least half of the CUs idle: parts up
    // to the CU count, at least 4 stages each (the copy ring runs 3 ahead)
    const int tiles = tiles_m * tiles_n, stages = g.K / 128;
    g.kparts = 1;
    if (g.ypart && tiles <= kGemmSplitMaxTiles && 2 * tiles <= device_cu_count())
      g.kparts = std::max(1, std::min({kGemmMaxParts, device_cu_count() / tiles, kGemmSplitItems / tiles, stages / 4}));
    dim3 grid(tiles, g.kparts), block(256);
#define SVDQ_G(S, O) hipLaunchKernelGGL((gemm_kernel<S, O>), grid, block, 0, st, g)
    if (slab) { if (f32) SVDQ_G(true, SVDQ_OUT_F32); else SVDQ_G(true, SVDQ_OUT_BF16); }
    else      { if (f32) SVDQ_G(false, SVDQ_OUT_F32); else SVDQ_G(false, SVDQ_OUT_BF16); }
#undef SVDQ_G
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.kparts == 1) return e;
    const long n4 = static_cast<long>(g.M) * (g.N / 4);
    const dim3 rgrid(static_cast<unsigned>((n4 + 255) / 256));
    if (f32) hipLaunchKernelGGL(gemm_ysum_kernel<SVDQ_OUT_F32>, rgrid, dim3(256), 0, st, g.ypart, g.kparts, g.M, g.N, g.bias, g.Y);
    else hipLaunchKernelGGL(gemm_ysum_kernel<SVDQ_OUT_BF16>, rgrid, dim3(256), 0, st, g.ypart, g.kparts, g.M, g.N, g.bias, g.Y);
    return hipGetLastError();
  }
  return launch_gemm_fp4(slab, out_dtype, ga, st);
}

hipError_t launch_up(int out_dtype, const uint16_t* Tb, const uint16_t* l2t, void* Y, int M, int N, int rank,
                     hipStream_t st) {
  if (rank == 0) return hipSuccess;
  const int tiles = ((M + 63) / 64) * ((N + 127) / 128);
  if (out_dtype == SVDQ_OUT_F32)
    hipLaunchKernelGGL(up_kernel<SVDQ_OUT_F32>, dim3(tiles), dim3(256), 0, st, Tb, l2t, Y, M, N, rank);
  else
    hipLaunchKernelGGL(up_kernel<SVDQ_OUT_BF16>, dim3(tiles), dim3(256), 0, st, Tb, l2t, Y, M, N, rank);
  return hipGetLastError();
}

}  // namespace svdq
