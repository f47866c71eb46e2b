// Kernel G, FP4 variant: the 4-bit GEMM of the SVDQuant layer on the gfx950
// block-scaled MFMA, with the low-rank up-projection as extra bf16 stages of
// the same reduction and a fused bias epilogue.
//
//   acc[m, n]  = sum_t Tb[m, t] L2b[t, n]            (eq. (5) low-rank branch,
//                                                     sharing the 4-bit branch's
//                                                     output as in Fig. 6 of the
//                                                     walkthrough)
//   acc[m, n] += sum_k 2^ex[m, k/32] 2^ew[n, k/32] qx[m, k] qw[n, k]
//                                                    (eq. (2); E2M1 codes with
//                                                     E8M0 group scales)
//   Y[m, n]    = round(acc[m, n] + b[n])
//
// The E2M1 nibbles and their power-of-two scales are the native operands of
// the 32x32x64 block-scaled MFMA, which applies the scales per 32-wide group
// and accumulates in fp32: no dequantization work remains.
//
// Shape and data movement (chosen by measurement on MI355X):
//  - persistent: one workgroup of 4 waves per CU (the LDS ring takes the CU)
//    walks its 256 x 256 output tiles in sequence, XCD-aware tile order;
//  - one wave per SIMD, 2 x 2 waves, each owning 128 x 128 outputs (4 x 4
//    MFMA tiles, 256 fp32 accumulators): every operand kilobyte a wave reads
//    from LDS feeds 4 MFMAs, which keeps the LDS read traffic at 2 KB per
//    MFMA-kilocycle -- the LDS, shared by the DMA writes and the operand
//    reads, is the tightest resource after the matrix core;
//  - the reduction of a tile is a stream of stages: rank/32 low-rank stages
//    (32 ranks of Tb and L2b, two 32x32x16 bf16 MFMA steps) then K/128 FP4
//    stages (two 32x32x64 steps).  A stage is 16 KB of activation blocks +
//    16 KB of weight blocks (1 KB = 32 rows in MFMA lane order, contiguous in
//    HBM) + 2 KB of scales, copied global -> LDS directly (global_load_lds,
//    16 bytes per lane) into a ring of 4 stage buffers; the copies of stage
//    G + 4 are issued while stage G is consumed, into the buffer stage G has
//    just released, and the stream continues across tile boundaries;
//  - one wait + barrier per stage, between its two MFMA steps: it publishes
//    stage G + 1 and releases stage G's buffer.  Operand reads run one MFMA
//    step ahead of the MFMAs, interleaved with them by scheduling fences;
//  - bias: copied into LDS with the tile's stages; the accumulators start
//    at it.  Epilogue: rounding, rows staged through a per-wave LDS area and
//    stored as contiguous 16-byte lanes with bounds-checked buffer stores.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "svdq_device.h"
#include "svdq_kernels.h"

namespace svdq {

namespace {

constexpr int F_TILE = 256;                       // output tile F_TILE x F_TILE
constexpr int F_NBUF = 4;                         // stage ring depth (copies run F_NBUF stages ahead)
constexpr int F_XB = 0, F_WB = 16384;             // activation / weight halves of a stage buffer
constexpr int F_STAGE = 32768;
constexpr int F_SC = F_NBUF * F_STAGE;            // scale ring: per stage 1 KB activation + 1 KB weight
constexpr int F_EPI = F_SC + F_NBUF * 2048;       // epilogue staging: 4 KB per wave
constexpr int F_NBIAS = 2;                        // tile bias buffers (1 KB each, by turn parity)
constexpr int F_BIAS = F_EPI + 4 * 4096;
constexpr int F_LDS = F_BIAS + F_NBIAS * 1024;    // 157696 bytes
constexpr int F_NCOPY = 11;                       // copies per wave per stage

// The global -> LDS copies are written as inline asm, so the compiler's own
// wait insertion neither sees them nor adds conservative waits before LDS
// reads; every wait on them is explicit below (s_waitcnt vmcnt counts them in
// issue order, together with the epilogue's stores).  m0 holds the LDS
// destination of lane 0; lane l writes 16 (or 4) bytes at m0 + 16 l (4 l).
// An LDS copy reading m0 right after a scalar write of it needs one wait
// state (the s_nop).
// m0 is set by every copy itself; nothing else in these kernels uses it (the
// compiler warns that a reserved register in a clobber list may not be
// preserved, which these copies do not rely on).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Four accumulator values (held in AGPRs) read out where the epilogue uses
// them: the volatile asm keeps the reads in program order, so the compiler
// cannot move all 256 reads to the start of the epilogue (whose register
// pressure would spill).
__device__ __forceinline__ f32x4 acc_read4(float a, float b, float c, float d) {
  f32x4 r;
  asm volatile(
      "v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\t"
      "v_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
      : "=v"(r.x), "=v"(r.y), "=v"(r.z), "=v"(r.w)
      : "a"(a), "a"(b), "a"(c), "a"(d));
  return r;
}

// s_waitcnt vmcnt(n) lgkmcnt(0), then s_barrier; also a compiler memory barrier
#define SVDQ_VM_BARRIER(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

}  // namespace

template <bool SLAB, int OUT>
__global__ __launch_bounds__(256) void gemm_fp4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F_LDS];
  // LDS byte address of smem (the m0 operand of the copies)
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)smem));

  const int M = g.M, K = g.K, N = g.N;
  const int RK = SLAB ? g.rank / 16 : 0;          // 16-rank blocks of Tb / L2b
  const int RS = (RK + 1) >> 1;                   // low-rank stages, 32 ranks each
  const int KS = K >> 7;                          // FP4 stages, 128 K each
  const int S = RS + KS;                          // stages per tile (>= 1)
  const long KB64 = K >> 6;                       // 1 KB code blocks per 32-row block
  const uint8_t* __restrict__ acodes = g.acodes;
  const uint8_t* __restrict__ wcodes = g.wcodes;
  const uint8_t* __restrict__ ascales = static_cast<const uint8_t*>(g.ascales);
  const uint8_t* __restrict__ wscales = static_cast<const uint8_t*>(g.wscales);
  const uint8_t* __restrict__ tbb = reinterpret_cast<const uint8_t*>(g.Tb);
  const uint8_t* __restrict__ l2b = reinterpret_cast<const uint8_t*>(g.l2t);
  const bool has_bias = g.bias != nullptr;
  // the bias copy reads a valid address even without a bias (never used then)
  const uint8_t* __restrict__ biasb = has_bias ? reinterpret_cast<const uint8_t*>(g.bias) : acodes;
  void* __restrict__ Yout = g.Y;

  const int tiles_m = (M + F_TILE - 1) / F_TILE, tiles_n = (N + F_TILE - 1) / F_TILE;
  const int ntiles = tiles_m * tiles_n;
  const int grid = static_cast<int>(gridDim.x), wg = static_cast<int>(blockIdx.x);
  const int my_tiles = (ntiles - wg + grid - 1) / grid;   // >= 1: the grid never exceeds the tile count
  const int last_ablk = (M + 31) / 32 - 1, last_bblk = N / 32 - 1;

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;        // 128-row half, 128-column half of the tile
  const uint32_t lane16 = lane * 16;

  auto tile_blocks = [&](int seq, int& mb0, int& nb0) __attribute__((always_inline)) {
    int tm, tn;
    tile_of(wg + seq * grid, tiles_m, tiles_n, tm, tn);
    // uniform by construction; made scalar so that addresses and buffer
    // resources built from them stay in SGPRs
    mb0 = wave_uniform(tm * (F_TILE / 32));
    nb0 = wave_uniform(tn * (F_TILE / 32));
  };

  // ---- copy side.  The copy stream is the compute stream shifted by
  // F_NBUF stages: while stage st of the current tile is consumed, the
  // copies of stage st + 4 are issued -- of the current tile if st + 4 < S,
  // else of the next turn's tile (the launch gives a workgroup several tiles
  // only when S >= 4, so the copies never run more than one tile ahead);
  // past the last tile the last stage is repeated (never consumed).  For a
  // stage, wave w copies the two 1 KB blocks (both MFMA steps) of
  // activation row blocks 2w, 2w + 1 and of weight row blocks 2w, 2w + 1 (8
  // copies), the scales of the same row blocks (2 copies of 4 bytes per
  // lane: lanes 0-31 row block 2w, lanes 32-63 row block 2w + 1), and a
  // quarter of the tile's bias (1 copy; every stage copies the same bytes
  // into the tile's bias buffer).  Row blocks past the matrix repeat its last
  // block (their outputs are never stored).  All of it is branch-free, so
  // the stage bodies stay single basic blocks the scheduler can interleave.
  struct CopySrc {
    const uint8_t *x0, *x1, *w0, *w1;   // first block of each of the wave's row blocks
    uint32_t dk;                        // byte distance to the second block
    const uint8_t *sx, *sw;             // scale bytes of row block 2w (lanes 32-63 add sdx / sdw)
    uint32_t sdx, sdw;
    const uint8_t* b;                   // this wave's quarter of the bias
    uint32_t bias_lds;
  };
  // cur: blocks of the tile being consumed (turn seq); nxt: of turn seq + 1
  auto copy_src = [&](int st, int seq, int mb0, int nb0, int nmb0, int nnb0) __attribute__((always_inline)) {
    CopySrc c;
    const int cg = st + F_NBUF;
    const bool in_next = cg >= S;
    const bool has_next = seq + 1 < my_tiles;
    const int cst = in_next ? (has_next ? cg - S : S - 1) : cg;
    const bool use_next = in_next && has_next;
    const int cmb0 = use_next ? nmb0 : mb0, cnb0 = use_next ? nnb0 : nb0;
    const int cturn = use_next ? seq + 1 : seq;
    const bool lr = SLAB && cst < RS;
    const int xa = min(cmb0 + 2 * wave, last_ablk), xb = min(cmb0 + 2 * wave + 1, last_ablk);
    const int wa = min(cnb0 + 2 * wave, last_bblk), wb = min(cnb0 + 2 * wave + 1, last_bblk);
    // low-rank stage: ranks 32 cst .. +31 = blocks 2 cst, 2 cst + 1; with an
    // odd number of 16-rank blocks the last stage repeats its first block
    // (the weight operand of that step is zeroed on the compute side)
    const long lt = 2L * cst;
    const int ks = lr ? 0 : cst - RS;             // FP4 stage (low-rank stages copy unused scales of stage 0)
    const long ft = 2L * ks;
    c.x0 = lr ? tbb + ((xa * static_cast<long>(RK) + lt) << 10) : acodes + ((xa * KB64 + ft) << 10);
    c.x1 = lr ? tbb + ((xb * static_cast<long>(RK) + lt) << 10) : acodes + ((xb * KB64 + ft) << 10);
    c.w0 = lr ? l2b + ((wa * static_cast<long>(RK) + lt) << 10) : wcodes + ((wa * KB64 + ft) << 10);
    c.w1 = lr ? l2b + ((wb * static_cast<long>(RK) + lt) << 10) : wcodes + ((wb * KB64 + ft) << 10);
    c.dk = (lr && 2 * cst + 1 >= RK) ? 0u : 1024u;
    c.sx = ascales + (static_cast<long>(xa) * KS + ks) * 128;
    c.sw = wscales + (static_cast<long>(wa) * KS + ks) * 128;
    // byte distance to the second row block's scales (0 when it is clamped onto the first)
    c.sdx = static_cast<uint32_t>(xb - xa) * KS * 128;
    c.sdw = static_cast<uint32_t>(wb - wa) * KS * 128;
    c.b = biasb + (has_bias ? (min(cnb0 * 32 + wave * 64, N - 64) * 4) : 0);
    c.bias_lds = lds0 + F_BIAS + (cturn & 1) * 1024 + wave * 256;
    return c;
  };
  const uint32_t lane4 = (lane & 31) * 4, upper = lane >> 5;
  // copy q (0..10) of a stage into ring buffer rb
  auto copy = [&](const CopySrc& c, uint32_t rb, int q) __attribute__((always_inline)) {
    if (q < 8) {
      // bit 2 weight, bit 1 second row block, bit 0 second MFMA step
      const uint8_t* base = (q & 4) ? ((q & 2) ? c.w1 : c.w0) : ((q & 2) ? c.x1 : c.x0);
      const uint32_t dst = lds0 + rb * F_STAGE + ((q & 4) ? F_WB : F_XB) + wave * 4096 + (q & 3) * 1024;
      dma16(base, lane16 + ((q & 1) ? c.dk : 0u), dst);
    } else if (q < 10) {
      // activation (q = 8) / weight (q = 9) scales of row blocks 2w, 2w + 1
      dma4s(q == 8 ? c.sx : c.sw, lane4 + upper * (q == 8 ? c.sdx : c.sdw), lds0 + F_SC + rb * 2048 + (q - 8) * 1024 + wave * 256);
    } else {
      // bias floats 64 w .. 64 w + 63 of the tile
      dma4s(c.b, lane * 4, c.bias_lds);
    }
  };

  // ---- compute side.  Operands of one MFMA step: weight blocks i = 0..3
  // (tile columns 128 wn + 32 i ..), activation blocks j = 0..3 (tile rows
  // 128 wm + 32 j ..); the weights are the MFMA's A operand, so lane l of
  // accumulator (i, j) holds output row 32 j + l % 32 and columns
  // 32 i + 8 (v / 4) + 4 (l / 32) + v % 4.
  struct Ops {
    u32x4 w[4], x[4];
  };
  const uint32_t rx = F_XB + wm * 8192 + lane16, rw = F_WB + wn * 8192 + lane16;
  const uint32_t rsx = F_SC + wm * 512 + lane * 2, rsw = F_SC + 1024 + wn * 512 + lane * 2;
  // piece p of MFMA step kk of ring buffer rb, in the order the MFMAs first
  // need them: weight 0, activations 0..3, weights 1..3
  auto read_piece = [&](Ops& o, uint32_t rb, int kk, int p) __attribute__((always_inline)) {
    const uint32_t base = rb * F_STAGE + kk * 1024;
    if (p == 0 || p >= 5) {
      const int i = p == 0 ? 0 : p - 4;
      o.w[i] = *reinterpret_cast<const u32x4*>(smem + rw + base + i * 2048);
    } else {
      const int j = p - 1;
      o.x[j] = *reinterpret_cast<const u32x4*>(smem + rx + base + j * 2048);
    }
  };
  // scales of ring buffer rb: byte kk of each value is MFMA step kk's
  auto read_scale = [&](uint32_t (&sx)[4], uint32_t (&sw)[4], uint32_t rb, int p) __attribute__((always_inline)) {
    if (p < 4) sx[p] = *reinterpret_cast<const uint16_t*>(smem + rsx + rb * 2048 + p * 128);
    else sw[p - 4] = *reinterpret_cast<const uint16_t*>(smem + rsw + rb * 2048 + (p - 4) * 128);
  };

  f32x16 acc[4][4];
  // MFMA t of step kk: weight block i = t / 4, activation block j = t % 4
  auto mfma = [&](const Ops& o, const uint32_t (&sx)[4], const uint32_t (&sw)[4], int t, auto KK, auto LR,
                  uint32_t wmask) __attribute__((always_inline)) {
    constexpr int kk = decltype(KK)::value;
    const int i = t >> 2, j = t & 3;
    const f32x16 c = acc[i][j];
    if constexpr (decltype(LR)::value) {
      u32x4 w = o.w[i];
      if constexpr (kk == 1) w &= wmask;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                         __builtin_bit_cast(bf16x8, o.x[j]), c, 0, 0, 0);
    } else {
      const i32x8 av = i32x8{(int)o.w[i].x, (int)o.w[i].y, (int)o.w[i].z, (int)o.w[i].w, 0, 0, 0, 0};
      const i32x8 bv = i32x8{(int)o.x[j].x, (int)o.x[j].y, (int)o.x[j].z, (int)o.x[j].w, 0, 0, 0, 0};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, kk, (int)sw[i], kk, (int)sx[j]);
    }
  };

  // One stage G (ring buffer rb = G % 4; stage st of the tile of turn seq),
  // a single basic block.  Step 0: 16 MFMAs on R0 with the reads of step 1
  // into R1.  Wait + barrier: this wave's copies of stage G + 1 are complete
  // once at most the F_NCOPY copies of each of stages G + 2 and G + 3 are
  // outstanding (in the first stages of a tile the previous tile's
  // epilogue stores come after those copies, so the same count also waits
  // for the older stores); lgkmcnt(0) completes this wave's reads of stage
  // G; the barrier then publishes stage G + 1 and releases stage G's buffer.
  // Step 1: 16 MFMAs on R1 with the copies of stage G + 4 (into rb), the
  // reads of stage G + 1 step 0 into R0 and of its scales.
  static_assert(F_NCOPY == 11, "the wait counts below assume 11 copies per wave per stage");
  struct Tile {
    int seq, mb0, nb0, nmb0, nnb0;
  };
  auto stage = [&](Ops& R0, uint32_t (&sx)[4], uint32_t (&sw)[4], const Tile& tl, int st, long G, uint32_t wmask,
                   auto LR) __attribute__((always_inline)) {
    const uint32_t rb = static_cast<uint32_t>(G & (F_NBUF - 1));
    const uint32_t rn = static_cast<uint32_t>((G + 1) & (F_NBUF - 1));
    const CopySrc c = copy_src(st, tl.seq, tl.mb0, tl.nb0, tl.nmb0, tl.nnb0);
    Ops R1;
#pragma unroll
    for (int t = 0; t < 16; t++) {
      mfma(R0, sx, sw, t, std::integral_constant<int, 0>{}, LR, wmask);
      if (t < 8) read_piece(R1, rb, 1, t);
      __builtin_amdgcn_sched_barrier(0);
    }
    SVDQ_VM_BARRIER(22);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t nsx[4], nsw[4];
#pragma unroll
    for (int t = 0; t < 16; t++) {
      mfma(R1, sx, sw, t, std::integral_constant<int, 1>{}, LR, wmask);
      if (t < 11) copy(c, rb, t);
      if (t >= 2 && t < 10) read_piece(R0, rn, 0, t - 2);
      if (t >= 8) read_scale(nsx, nsw, rn, t - 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      sx[q] = nsx[q];
      sw[q] = nsw[q];
    }
  };

  // Accumulators of the tile of turn seq start at its bias (copied into
  // bias buffer seq % 2 with the copies of the tile's stages, the first of
  // which completed at the barrier before the tile's first stage), so the
  // epilogue only rounds: acc[i][j][v] = b[128 wn + 32 i + 8 (v / 4) + 4 lh + v % 4].
  auto init_acc = [&](int seq) __attribute__((always_inline)) {
    if (has_bias) {
      const float* bl = reinterpret_cast<const float*>(smem + F_BIAS + (seq & 1) * 1024) + wn * 128 + 4 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        f32x4 b4[4];
#pragma unroll
        for (int gq = 0; gq < 4; gq++) b4[gq] = *reinterpret_cast<const f32x4*>(bl + 32 * i + 8 * gq);
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int v = 0; v < 16; v++) acc[i][j][v] = b4[v >> 2][v & 3];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
    }
  };

  // Epilogue of the tile at (mb0, nb0): per 32-row x 64-column (bf16) or
  // 32 x 32 (fp32) slice, the lanes write their values, rounded, into this
  // wave's 4 KB staging area (16-byte chunks XOR-swizzled by row), then read
  // whole rows back and store them 16 bytes per lane.  Rows past M and
  // columns past N get an offset past the buffer resource and are dropped,
  // so every store instruction issues (the waits count them).
  auto epilogue = [&](int mb0, int nb0) __attribute__((always_inline)) {
    // lane indices recomputed through an opaque move, so that the compiler
    // does not hoist the epilogue's per-lane addresses out of the tile loop
    int lane_e;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_e) : "v"(lane));
    const int l32 = lane_e & 31, lh = lane_e >> 5;
    constexpr int OB = OUT == SVDQ_OUT_F32 ? 4 : 2;
    uint8_t* stg = smem + F_EPI + wave * 4096;
    const long m0 = static_cast<long>(mb0) * 32;
    const long colw = static_cast<long>(nb0) * 32 + wn * 128;     // the wave's first column
    const uint32_t rowb = static_cast<uint32_t>(N * OB);            // output row bytes
    const int valid_rows = static_cast<int>(min(static_cast<long>(M) - m0, static_cast<long>(F_TILE)));
    const uint32_t nrec = static_cast<uint32_t>(valid_rows) * rowb;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(Yout) + m0 * rowb, 0, static_cast<int>(nrec), 0x00020000);
    // read-back: lane reads chunk (lane % 8) of slice rows lane / 8 + 8 r
    const int rrow = lane_e >> 3, rch = lane_e & 7;
    constexpr int NSL = OUT == SVDQ_OUT_F32 ? 4 : 2;        // column slices of the wave's 128 columns
    constexpr int SLW = 128 / NSL;                          // slice width in columns
    constexpr int NII = SLW / 32;
#pragma unroll
    for (int sl = 0; sl < NSL; sl++) {
      const long c0 = colw + sl * SLW;
      const bool cols_ok = c0 < N;                          // N % 64 == 0: a whole slice is in or out
#pragma unroll
      for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int ii = 0; ii < NII; ii++) {
          const int i = sl * NII + ii;
#pragma unroll
          for (int gq = 0; gq < 4; gq++) {
            const f32x4 y = acc_read4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
            if constexpr (OUT == SVDQ_OUT_F32) {
              const int ch = 2 * gq + lh;                   // 16-byte chunk of the 128-byte slice row
              *reinterpret_cast<f32x4*>(stg + l32 * 128 + ((ch ^ (l32 & 7)) << 4)) = y;
            } else {
              const int ch = 4 * ii + gq;                   // 16-byte chunk; lh picks its 8-byte half
              typedef float f32x2 __attribute__((ext_vector_type(2)));
              typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
              typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
              // round to nearest even (v_cvt_pk_bf16_f32)
              const bf16x2 p0 = __builtin_convertvector(f32x2{y.x, y.y}, bf16x2);
              const bf16x2 p1 = __builtin_convertvector(f32x2{y.z, y.w}, bf16x2);
              *reinterpret_cast<u32x2*>(stg + l32 * 128 + ((ch ^ (l32 & 7)) << 4) + lh * 8) =
                  u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
        const int trow0 = wm * 128 + j * 32;                // first slice row in the tile
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int row = rrow + 8 * r;
          const u32x4 d = *reinterpret_cast<const u32x4*>(stg + row * 128 + ((rch ^ (row & 7)) << 4));
          const uint32_t off = cols_ok && trow0 + row < valid_rows
                                   ? static_cast<uint32_t>(trow0 + row) * rowb + static_cast<uint32_t>(c0 * OB) + rch * 16
                                   : nrec;
          __builtin_amdgcn_raw_buffer_store_b128(d, yr, static_cast<int>(off), 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
        // one slice at a time: keeps the compiler from reading all the
        // accumulators out at once (the register pressure would spill)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- prologue: stages 0 .. 3 of the first tile in flight, stage 0
  // published and read
  Tile tl;
  tl.seq = 0;
  tile_blocks(0, tl.mb0, tl.nb0);
  tile_blocks(min(1, my_tiles - 1), tl.nmb0, tl.nnb0);
#pragma unroll 1
  for (int p = 0; p < F_NBUF; p++) {
    // the copies of stage p are those issued while stage p - 4 is consumed
    const CopySrc c = copy_src(p - F_NBUF, 0, tl.mb0, tl.nb0, tl.nmb0, tl.nnb0);
#pragma unroll
    for (int q = 0; q < F_NCOPY; q++) copy(c, p, q);
  }
  // stage 0 complete: the copies of stages 1 .. 3 may stay in flight
  SVDQ_VM_BARRIER(33);
  Ops oa;
  uint32_t sx[4], sw[4];
#pragma unroll
  for (int p = 0; p < 8; p++) read_piece(oa, 0, 0, p);
#pragma unroll
  for (int p = 0; p < 8; p++) read_scale(sx, sw, 0, p);

  long G = 0;
  const uint32_t last_mask = (RK & 1) ? 0u : ~0u;    // zero weight operand in the odd half of the last low-rank stage
#pragma unroll 1
  for (int seq = 0; seq < my_tiles; seq++) {
    if (seq > 0) {
      tl.seq = seq;
      tl.mb0 = tl.nmb0;
      tl.nb0 = tl.nnb0;
      tile_blocks(min(seq + 1, my_tiles - 1), tl.nmb0, tl.nnb0);
    }
    init_acc(seq);
#pragma unroll 1
    for (int st = 0; st < RS; st++) {
      stage(oa, sx, sw, tl, st, G, st == RS - 1 ? last_mask : ~0u, std::true_type{});
      G++;
    }
#pragma unroll 1
    for (int st = RS; st < S; st++) {
      stage(oa, sx, sw, tl, st, G, ~0u, std::false_type{});
      G++;
    }
    epilogue(tl.mb0, tl.nb0);
  }
  // no copy may still be writing this workgroup's LDS when it exits
  SVDQ_VM_BARRIER(0);
}
// Compute units of the current device (cached per device): the persistent
// kernel launches at most one workgroup per CU.
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

hipError_t launch_gemm_fp4(bool slab, int out_dtype, const GemmArgs& g, hipStream_t st) {
  const int tiles = ((g.M + F_TILE - 1) / F_TILE) * ((g.N + F_TILE - 1) / F_TILE);
  // a workgroup walks several tiles only when a tile has at least 4 stages,
  // so that the copies never run more than one tile ahead
  const int stages = (slab ? (g.rank / 16 + 1) / 2 : 0) + g.K / 128;
  dim3 grid(stages >= 4 ? std::min(tiles, cu_count()) : tiles), block(256);
  const bool f32 = out_dtype == SVDQ_OUT_F32;
#define SVDQ_F(S, O) hipLaunchKernelGGL((gemm_fp4_kernel<S, O>), grid, block, 0, st, g)
  if (slab) { if (f32) SVDQ_F(true, SVDQ_OUT_F32); else SVDQ_F(true, SVDQ_OUT_BF16); }
  else      { if (f32) SVDQ_F(false, SVDQ_OUT_F32); else SVDQ_F(false, SVDQ_OUT_BF16); }
#undef SVDQ_F
  return hipGetLastError();
}

}  // namespace svdq
