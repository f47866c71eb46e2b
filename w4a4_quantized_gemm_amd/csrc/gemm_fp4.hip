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
//    G + 3 are issued during the first MFMA step of stage G, into the buffer
//    stage G - 1 released, and the stream continues across tile boundaries;
//  - one wait + barrier per stage, between its two MFMA steps: it publishes
//    stage G + 1 and releases stage G's buffer.  Operand reads run one MFMA
//    step ahead of the MFMAs, interleaved with them by scheduling fences;
//  - a wave per SIMD issues about one instruction per 4 cycles and an MFMA
//    takes 32, so every instruction besides the MFMAs counts: the copy
//    addresses are per-run scalar bases plus one per-lane offset that grows
//    by a constant each stage, and four copies share one m0 through the
//    copy's immediate offset (it moves the global and the LDS address alike);
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
constexpr int F_NBUF = 4;                         // stage ring depth
constexpr int F_AHEAD = 3;                        // stage G + 3 is copied while stage G is consumed
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
// issue order, together with the epilogue's stores).  A copy reads
// sbase + voff + OFF (64-bit scalar base, 32-bit per-lane offset, immediate
// OFF) and writes LDS at m0 + OFF + 16 l (4 l) for lane l: the immediate
// offset moves both addresses.  An LDS copy needs one wait state after a
// scalar write of m0: the stage bodies keep an MFMA between set_m0 and the
// first copy that reads it (scheduling fences fix that order), and the
// prologue waits explicitly (set_m0_nop).  Nothing else in these
// kernels uses m0 (the compiler warns that a reserved register in a clobber
// list may not be preserved, which these copies do not rely on: m0 is always
// written right before the copies that read it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void set_m0(uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0" ::"s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void set_m0_nop(uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(lds) : "memory", "m0");
}
template <int OFF>
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff) {
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(voff), "s"(sbase), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff) {
  asm volatile("global_load_lds_dword %0, %1 offset:%2" ::"v"(voff), "s"(sbase), "i"(OFF) : "memory");
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

// s_waitcnt lgkmcnt(0) (as a builtin, so the compiler knows this wave's LDS
// reads are complete), s_waitcnt vmcnt(n), then s_barrier; also a compiler
// memory barrier
constexpr int LGKM0 = 0xC07F;     // s_waitcnt encoding: lgkmcnt(0), vmcnt and expcnt unconstrained
#define SVDQ_VM_BARRIER(n)                  \
  do {                                      \
    __builtin_amdgcn_s_waitcnt(LGKM0);      \
    asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_barrier" ::: "memory"); \
  } while (0)

}  // namespace

// GENERAL: any rank and K; otherwise rank/32 <= 3 low-rank stages and at
// least 3 FP4 stages per tile, where the copy descriptors change only at
// fixed stages of a tile (straight-line runs, no per-stage descriptor work).
template <bool SLAB, int OUT, bool GENERAL>
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
  // F_AHEAD stages: during stage st of the tile being consumed, the copies
  // of stage st + 3 are issued -- of the current tile if st + 3 < S, else of
  // the next turn's tile (the launch gives a workgroup several tiles only
  // when S >= 3, so the copies never run more than one tile ahead); past the
  // last tile the last stage is repeated (never consumed).  For a stage,
  // wave w copies the two 1 KB blocks (both MFMA steps) of activation row
  // blocks 2w, 2w + 1 and of weight row blocks 2w, 2w + 1 (8 copies), the
  // scales of the same row blocks (2 copies of 4 bytes per lane: lanes 0-31
  // row block 2w, lanes 32-63 row block 2w + 1) and a quarter of the tile's
  // bias (1 copy; every stage copies the same bytes into the tile's bias
  // buffer).  Row blocks past the matrix repeat its last block (their
  // outputs are never stored).
  //
  // A run of consecutive stages whose copies come from one tile and one kind
  // (low-rank or FP4) shares a descriptor of scalar bases; the per-lane
  // offsets grow by a constant each stage (0 when the last stage repeats).
  // Block copy q of a stage reads base + voff + 1024 q for the activation
  // (q = 0..3: row block 2w steps 0, 1, row block 2w + 1 steps 0, 1) and
  // writes m0 + 1024 q; the bases absorb the distance between the two row
  // blocks and, in the last low-rank stage of an odd number of 16-rank
  // blocks, repeat the first block for the second step (whose weight operand
  // the compute side zeroes).
  struct CopyDesc {
    const uint8_t *x[4], *w[4];         // bases of block copies q = 0..3
    const uint8_t *sx, *sw;             // scale bases (sw minus 1024: its copy has OFF 1024)
    const uint8_t* b;                   // this wave's quarter of the tile's bias
    uint32_t bias_lds;                  // its LDS destination
    uint32_t inc, sinc;                 // per-stage growth of voff / the scale offsets
  };
  struct CopyOff {
    uint32_t v, vsx, vsw;               // per-lane offsets: blocks, activation / weight scales
  };
  const uint32_t lane4 = (lane & 31) * 4, upper = lane >> 5;
  // descriptor of a run starting at stage cst of the tile (mb0, nb0) of turn
  // `turn`; rep: the run repeats that stage
  auto make_desc = [&](int mb0, int nb0, int turn, int cst, bool rep, CopyDesc& d, CopyOff& o)
      __attribute__((always_inline)) {
    const bool lr = SLAB && cst < RS;
    const int xa = min(mb0 + 2 * wave, last_ablk), xb = min(mb0 + 2 * wave + 1, last_ablk);
    const int wa = min(nb0 + 2 * wave, last_bblk), wb = min(nb0 + 2 * wave + 1, last_bblk);
    const long rstride = lr ? RK : KB64;          // 1 KB blocks per row block of this kind
    const uint8_t* xm = lr ? tbb : acodes;
    const uint8_t* wmx = lr ? l2b : wcodes;
    // second step of the stage: the next block, or the same one (odd low-rank tail)
    const long dk = (lr && 2 * cst + 1 >= RK) ? 0 : 1024;
    const uint8_t* xa0 = xm + ((xa * rstride) << 10);
    const uint8_t* xb0 = xm + ((xb * rstride) << 10);
    const uint8_t* wa0 = wmx + ((wa * rstride) << 10);
    const uint8_t* wb0 = wmx + ((wb * rstride) << 10);
    d.x[0] = xa0;
    d.x[1] = xa0 + dk - 1024;
    d.x[2] = xb0 - 2048;
    d.x[3] = xb0 + dk - 3072;
    d.w[0] = wa0;
    d.w[1] = wa0 + dk - 1024;
    d.w[2] = wb0 - 2048;
    d.w[3] = wb0 + dk - 3072;
    const int ks = lr ? 0 : cst - RS;             // FP4 stage (low-rank stages copy unused scales of stage 0)
    d.sx = ascales + static_cast<long>(xa) * KS * 128;
    d.sw = wscales + static_cast<long>(wa) * KS * 128 - 1024;
    d.b = biasb + (has_bias ? (min(nb0 * 32 + wave * 64, N - 64) * 4) : 0);
    d.bias_lds = lds0 + F_BIAS + (turn & 1) * 1024 + wave * 256;
    d.inc = rep ? 0u : 2048u;
    d.sinc = (rep || lr) ? 0u : 128u;
    o.v = lane16 + static_cast<uint32_t>(lr ? cst : ks) * 2048u;
    o.vsx = lane4 + upper * static_cast<uint32_t>((xb - xa) * KS * 128) + static_cast<uint32_t>(ks) * 128u;
    o.vsw = lane4 + upper * static_cast<uint32_t>((wb - wa) * KS * 128) + static_cast<uint32_t>(ks) * 128u;
  };
  // copy items of a stage into ring buffer rc, one group per MFMA slot t of
  // the stage's first step: each m0 write sits one slot before the copies
  // that read it (the MFMA between them is the wait state the copy needs)
  auto copy_slot = [&](const CopyDesc& d, const CopyOff& o, uint32_t rc, int t) __attribute__((always_inline)) {
    // one copy per slot: bursts of copies stall the issuing wave
    switch (t) {
      case 0: set_m0(lds0 + rc * F_STAGE + F_XB + wave * 4096); break;
      case 1: dma16<0>(d.x[0], o.v); break;
      case 2: dma16<1024>(d.x[1], o.v); break;
      case 3: dma16<2048>(d.x[2], o.v); break;
      case 4: dma16<3072>(d.x[3], o.v); set_m0(lds0 + rc * F_STAGE + F_WB + wave * 4096); break;
      case 5: dma16<0>(d.w[0], o.v); break;
      case 6: dma16<1024>(d.w[1], o.v); break;
      case 7: dma16<2048>(d.w[2], o.v); break;
      case 8: dma16<3072>(d.w[3], o.v); set_m0(lds0 + F_SC + rc * 2048 + wave * 256); break;
      case 9: dma4<0>(d.sx, o.vsx); break;
      case 10: dma4<1024>(d.sw, o.vsw); set_m0(d.bias_lds); break;
      case 11: dma4<0>(d.b, lane * 4u); break;
      default: break;
    }
  };
  // the same copies outside a stage (prologue): explicit wait states
  auto copy_all = [&](const CopyDesc& d, const CopyOff& o, uint32_t rc) __attribute__((always_inline)) {
    set_m0_nop(lds0 + rc * F_STAGE + F_XB + wave * 4096);
    dma16<0>(d.x[0], o.v); dma16<1024>(d.x[1], o.v); dma16<2048>(d.x[2], o.v); dma16<3072>(d.x[3], o.v);
    set_m0_nop(lds0 + rc * F_STAGE + F_WB + wave * 4096);
    dma16<0>(d.w[0], o.v); dma16<1024>(d.w[1], o.v); dma16<2048>(d.w[2], o.v); dma16<3072>(d.w[3], o.v);
    set_m0_nop(lds0 + F_SC + rc * 2048 + wave * 256);
    dma4<0>(d.sx, o.vsx); dma4<1024>(d.sw, o.vsw);
    set_m0_nop(d.bias_lds);
    dma4<0>(d.b, lane * 4u);
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
  auto read_piece = [&](Ops& o, uint32_t ax, uint32_t aw, int kk, int p) __attribute__((always_inline)) {
    if (p == 0 || p >= 5) {
      const int i = p == 0 ? 0 : p - 4;
      o.w[i] = *reinterpret_cast<const u32x4*>(smem + aw + kk * 1024 + i * 2048);
    } else {
      const int j = p - 1;
      o.x[j] = *reinterpret_cast<const u32x4*>(smem + ax + kk * 1024 + j * 2048);
    }
  };
  // scales: byte kk of each value is MFMA step kk's
  auto read_scale = [&](uint32_t (&sx)[4], uint32_t (&sw)[4], uint32_t asx, uint32_t asw, int p)
      __attribute__((always_inline)) {
    if (p < 4) sx[p] = *reinterpret_cast<const uint16_t*>(smem + asx + p * 128);
    else sw[p - 4] = *reinterpret_cast<const uint16_t*>(smem + asw + (p - 4) * 128);
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

  // One stage G (ring buffer rb = G % 4), a single basic block.
  //  step 0: 16 MFMAs on R0 (stage G, step 0), with the reads of step 1 into
  //          R1 and the 15 copy items of stage G + 3 into ring buffer
  //          (G + 3) % 4 -- stage G - 1's, released by the previous barrier;
  //  wait + barrier: this wave's copies of stage G + 1 are complete once at
  //          most the F_NCOPY copies of each of stages G + 2 and G + 3 are
  //          outstanding (in the first stages of a tile the previous tile's
  //          epilogue stores come after those copies, so the same count also
  //          waits for the older stores); lgkmcnt(0) completes this wave's
  //          reads of stage G; the barrier then publishes stage G + 1 and
  //          releases stage G's buffer;
  //  step 1: 16 MFMAs on R1 with the reads of stage G + 1 step 0 into R0 and
  //          of its scales.
  static_assert(F_NCOPY == 11, "the wait counts below assume 11 copies per wave per stage");
  // (sx, sw): this stage's scales; (nsx, nsw): where the next stage's go
  auto stage = [&](Ops& R0, const uint32_t (&sx)[4], const uint32_t (&sw)[4], uint32_t (&nsx)[4],
                   uint32_t (&nsw)[4], long G, const CopyDesc& d, CopyOff& o, uint32_t wmask, auto LR)
      __attribute__((always_inline)) {
    const uint32_t rb = static_cast<uint32_t>(G & (F_NBUF - 1));
    const uint32_t rn = static_cast<uint32_t>((G + 1) & (F_NBUF - 1));
    const uint32_t rc = static_cast<uint32_t>((G + F_AHEAD) & (F_NBUF - 1));
    const uint32_t ax = rx + rb * F_STAGE, aw = rw + rb * F_STAGE;
    Ops R1;
#pragma unroll
    for (int t = 0; t < 16; t++) {
      mfma(R0, sx, sw, t, std::integral_constant<int, 0>{}, LR, wmask);
      __builtin_amdgcn_sched_barrier(0);
      if (t < 8) read_piece(R1, ax, aw, 1, t);
      copy_slot(d, o, rc, t);
      __builtin_amdgcn_sched_barrier(0);
    }
    SVDQ_VM_BARRIER(22);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t nx = rx + rn * F_STAGE, nw = rw + rn * F_STAGE;
    const uint32_t nsxa = rsx + rn * 2048, nswa = rsw + rn * 2048;
#pragma unroll
    for (int t = 0; t < 16; t++) {
      mfma(R1, sx, sw, t, std::integral_constant<int, 1>{}, LR, wmask);
      if (t < 8) read_piece(R0, nx, nw, 0, t);
      if (t < 8) read_scale(nsx, nsw, nsxa, nswa, t);
      __builtin_amdgcn_sched_barrier(0);
    }
    o.v += d.inc;
    o.vsx += d.sinc;
    o.vsw += d.sinc;
  };
  // n consecutive stages of one kind and descriptor (the next stage's scales
  // are read into (nsx, nsw) and moved into place after each stage)
  auto run = [&](Ops& R0, uint32_t (&sx)[4], uint32_t (&sw)[4], long& G, int n, const CopyDesc& d, CopyOff& o,
                 uint32_t wmask_last, auto LR) __attribute__((always_inline)) {
#pragma unroll 1
    for (; n > 0; n--, G++) {
      uint32_t nsx[4], nsw[4];
      stage(R0, sx, sw, nsx, nsw, G, d, o, n == 1 ? wmask_last : ~0u, LR);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        sx[q] = nsx[q];
        sw[q] = nsw[q];
      }
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

  // Epilogue of the tile at (mb0, nb0) whose last stage was G: per 32-row x
  // 64-column (bf16) or 32 x 32 (fp32) slice, the lanes write their values,
  // rounded, into a 4 KB staging slot (16-byte chunks XOR-swizzled by row),
  // then whole rows are read back and stored 16 bytes per lane.  Two slots
  // per wave alternate, so a slice's writes, read-back and stores overlap
  // the next slice's: this wave's part of the F_EPI area, and this wave's
  // quarter of ring buffer G % 4, which stage G released and nothing writes
  // before the copies issued in the next stage (the barrier at the end keeps
  // every wave's read-back ahead of those copies).  Rows past M and columns
  // past N get an offset past the buffer resource and are dropped, so every
  // store instruction issues (the waits count them).
  auto epilogue = [&](int mb0, int nb0, long G) __attribute__((always_inline)) {
    // lane indices recomputed through an opaque move, so that the compiler
    // does not hoist the epilogue's per-lane addresses out of the tile loop
    int lane_e;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_e) : "v"(lane));
    const int l32 = lane_e & 31, lh = lane_e >> 5;
    constexpr int OB = OUT == SVDQ_OUT_F32 ? 4 : 2;
    uint8_t* const slot[2] = {smem + F_EPI + wave * 4096,
                              smem + static_cast<uint32_t>(G & (F_NBUF - 1)) * F_STAGE + wave * 4096};
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
    constexpr int NQ = NSL * 4;                             // slices: (column slice, 32-row block)
    auto write_slice = [&](int q) __attribute__((always_inline)) {
      const int sl = q >> 2, j = q & 3;
      uint8_t* stg = slot[q & 1];
#pragma unroll
      for (int ii = 0; ii < NII; ii++) {
        const int i = sl * NII + ii;
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
          const f32x4 y = acc_read4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
          if constexpr (OUT == SVDQ_OUT_F32) {
            const int ch = 2 * gq + lh;                     // 16-byte chunk of the 128-byte slice row
            *reinterpret_cast<f32x4*>(stg + l32 * 128 + ((ch ^ (l32 & 7)) << 4)) = y;
          } else {
            const int ch = 4 * ii + gq;                     // 16-byte chunk; lh picks its 8-byte half
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
    };
    auto read_slice = [&](int q, u32x4 (&d)[4]) __attribute__((always_inline)) {
      const uint8_t* stg = slot[q & 1];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int row = rrow + 8 * r;
        d[r] = *reinterpret_cast<const u32x4*>(stg + row * 128 + ((rch ^ (row & 7)) << 4));
      }
    };
    auto store_slice = [&](int q, const u32x4 (&d)[4]) __attribute__((always_inline)) {
      const int sl = q >> 2, j = q & 3;
      const long c0 = colw + sl * SLW;
      const bool cols_ok = c0 < N;                          // N % 64 == 0: a whole slice is in or out
      const int trow0 = wm * 128 + j * 32;                  // first slice row in the tile
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int row = rrow + 8 * r;
        const uint32_t off = cols_ok && trow0 + row < valid_rows
                                 ? static_cast<uint32_t>(trow0 + row) * rowb + static_cast<uint32_t>(c0 * OB) + rch * 16
                                 : nrec;
        __builtin_amdgcn_raw_buffer_store_b128(d[r], yr, static_cast<int>(off), 0, 0);
      }
    };
    write_slice(0);
#pragma unroll
    for (int q = 1; q <= NQ; q++) {
      // slice q - 1 is read back while slice q is written (other slot),
      // then stored
      u32x4 dq[4];
      read_slice(q - 1, dq);
      if (q < NQ) write_slice(q);
      store_slice(q - 1, dq);
      // a slice at a time: keeps the compiler from reading all the
      // accumulators out at once (the register pressure would spill)
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave's read-back of ring buffer G % 4 precedes the copies into it
    __builtin_amdgcn_s_barrier();
  };

  // ---- prologue: the copies of stages 0 .. 2 of the first tile, stage 0
  // published and read
  int mb0, nb0, nmb0, nnb0;
  tile_blocks(0, mb0, nb0);
  tile_blocks(min(1, my_tiles - 1), nmb0, nnb0);
  CopyDesc d;
  CopyOff o;
#pragma unroll 1
  for (int p = 0; p < F_AHEAD; p++) {
    // (first tile: S >= 3 whenever it has a successor; otherwise repeat its last stage)
    make_desc(mb0, nb0, 0, min(p, S - 1), p >= S, d, o);
    copy_all(d, o, p);
  }
  // stage 0 complete: the copies of stages 1 and 2 may stay in flight
  SVDQ_VM_BARRIER(22);
  Ops oa;
  uint32_t sx[4], sw[4];
#pragma unroll
  for (int p = 0; p < 8; p++) read_piece(oa, rx, rw, 0, p);
#pragma unroll
  for (int p = 0; p < 8; p++) read_scale(sx, sw, rsx, rsw, p);

  long G = 0;
  const uint32_t last_mask = (RK & 1) ? 0u : ~0u;    // zero weight operand in the odd half of the last low-rank stage
#pragma unroll 1
  for (int seq = 0; seq < my_tiles; seq++) {
    if (seq > 0) {
      mb0 = nmb0;
      nb0 = nnb0;
      tile_blocks(min(seq + 1, my_tiles - 1), nmb0, nnb0);
    }
    init_acc(seq);
    const bool has = seq + 1 < my_tiles;         // else the copies repeat the last stage
    if constexpr (!GENERAL) {
      // A, B: stages [0, S - 3), copies of this tile's FP4 stages from stage 3
      make_desc(mb0, nb0, seq, F_AHEAD, false, d, o);
      if constexpr (SLAB) run(oa, sx, sw, G, RS, d, o, last_mask, std::true_type{});
      run(oa, sx, sw, G, S - F_AHEAD - RS, d, o, ~0u, std::false_type{});
      // C: copies of the next tile's low-rank stages (the odd tail stage,
      // with its own second-step bases, separately)
      if constexpr (SLAB) {
        if (RS > 1) {
          if (has) make_desc(nmb0, nnb0, seq + 1, 0, false, d, o);
          else make_desc(mb0, nb0, seq, S - 1, true, d, o);
          run(oa, sx, sw, G, RS - 1, d, o, ~0u, std::false_type{});
        }
        if (RS > 0) {
          if (has) make_desc(nmb0, nnb0, seq + 1, RS - 1, false, d, o);
          else make_desc(mb0, nb0, seq, S - 1, true, d, o);
          run(oa, sx, sw, G, 1, d, o, ~0u, std::false_type{});
        }
      }
      // D: copies of the next tile's FP4 stages
      if (has) make_desc(nmb0, nnb0, seq + 1, RS, false, d, o);
      else make_desc(mb0, nb0, seq, S - 1, true, d, o);
      run(oa, sx, sw, G, F_AHEAD - RS, d, o, ~0u, std::false_type{});
    } else {
      // any shape: a descriptor per stage
#pragma unroll 1
      for (int st = 0; st < S; st++) {
        const int cg = st + F_AHEAD;
        const bool c_next = cg >= S;
        const bool hs = !c_next || has;
        const int cst = !hs ? S - 1 : (c_next ? cg - S : cg);
        make_desc(c_next && hs ? nmb0 : mb0, c_next && hs ? nnb0 : nb0, c_next && hs ? seq + 1 : seq, cst, !hs, d, o);
        if (SLAB && st < RS) run(oa, sx, sw, G, 1, d, o, st == RS - 1 ? last_mask : ~0u, std::true_type{});
        else run(oa, sx, sw, G, 1, d, o, ~0u, std::false_type{});
      }
    }
    epilogue(mb0, nb0, G - 1);
  }
  // no copy may still be writing this workgroup's LDS when it exits
  SVDQ_VM_BARRIER(0);
}

// Compute units of the current device (cached per device): the persistent
// kernel launches at most one workgroup per CU.
int device_cu_count() {
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
  // a workgroup walks several tiles only when a tile has at least 3 stages,
  // so that the copies (3 stages ahead) never run more than one tile ahead
  const int stages = (slab ? (g.rank / 16 + 1) / 2 : 0) + g.K / 128;
  dim3 grid(stages >= 3 ? std::min(tiles, device_cu_count()) : tiles), block(256);
  const bool f32 = out_dtype == SVDQ_OUT_F32;
  const int rs = slab ? (g.rank / 16 + 1) / 2 : 0;
  const bool general = rs > 3 || stages < rs + 3;
#define SVDQ_F(S, O, GEN) hipLaunchKernelGGL((gemm_fp4_kernel<S, O, GEN>), grid, block, 0, st, g)
#define SVDQ_F2(S, O) do { if (general) SVDQ_F(S, O, true); else SVDQ_F(S, O, false); } while (0)
  if (slab) { if (f32) SVDQ_F2(true, SVDQ_OUT_F32); else SVDQ_F2(true, SVDQ_OUT_BF16); }
  else      { if (f32) SVDQ_F2(false, SVDQ_OUT_F32); else SVDQ_F2(false, SVDQ_OUT_BF16); }
#undef SVDQ_F2
#undef SVDQ_F
  return hipGetLastError();
}

}  // namespace svdq
