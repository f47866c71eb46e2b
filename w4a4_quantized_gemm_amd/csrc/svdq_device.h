// Device-side helpers shared by the HIP kernels of libsvdq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

namespace svdq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// A value the compiler cannot see is uniform across the wave, made scalar.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round-half-even of the exact quotient x / s for s > 0 with |x / s| <= 16,
// given r = 1/s correctly rounded.  y = x * r is within 2^-19 of x / s, so
// rint(y) is the answer unless y is within 2^-18 of a half-integer; then the
// sign of x - (q +- 1/2) s, which one fma gives exactly, decides.
__device__ __forceinline__ float rne_quotient(float x, float s, float r) {
  const float y = x * r;
  float q = __builtin_rintf(y);
  if (__builtin_fabsf(y - q) > 0.5f - 0x1p-18f) {
    const float dhi = __builtin_fmaf(-(q + 0.5f), s, x);
    const float dlo = __builtin_fmaf(-(q - 0.5f), s, x);
    const bool odd = (static_cast<int>(q) & 1) != 0;
    if (dhi > 0.f || (dhi == 0.f && odd)) q += 1.f;
    else if (dlo < 0.f || (dlo == 0.f && odd)) q -= 1.f;
  }
  return q;
}

// Smallest e with a <= 6 * 2^e for a finite a >= 0, clamped to [-127, 127];
// a = 0 (or below 2^-126) gives -127.  Exact integer arithmetic on the bits:
// a = 1.f * 2^(eb-127); 6 * 2^e >= a  <=>  e >= eb - 129 + (1.f > 1.5).
__device__ __forceinline__ int e8m0_exponent(float a) {
  const uint32_t b = __float_as_uint(a);
  const int eb = static_cast<int>((b >> 23) & 0xFFu);
  if (eb == 0) return -127;
  const int e = eb - 129 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 4-bit float (E2M1) code of y, |y| <= 6: nearest of 0, .5, 1, 1.5, 2, 3, 4,
// 6 with ties to the even code; a value that rounds to zero gives +0.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float m = __builtin_fabsf(y);
  uint32_t idx = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
                 (m >= 3.5f) + (m > 5.0f);
  return idx | ((y < 0.f && idx != 0u) ? 8u : 0u);
}

// Bits of INT4 code q (|q| <= 7) in the 32-bit word that holds codes
// k .. k + 7 (k % 8 == 0), for code j = 0..7 of the word.  Each code is the
// byte (q < 0) << 7 | |q|, the E4M3 bits of q * 2^-9 (a subnormal; zero is
// +0); codes 0-3 fill bits 7 and 0-2 of bytes 0-3, codes 4-7 the same byte
// positions rotated left by 4 bits.  So word & 0x87878787 and
// rotr(word, 4) & 0x87878787 are the E4M3 bytes of codes 0-3 and 4-7.
__host__ __device__ inline uint32_t int4_code_bits(int q, int j) {
  const uint32_t b = (q < 0 ? 0x80u : 0u) | static_cast<uint32_t>(q < 0 ? -q : q);
  const int sh = j < 4 ? 8 * j : 8 * (j - 4) + 4;
  return sh == 0 ? b : (b << sh) | (b >> (32 - sh));
}

// Byte offset of the 16-byte chunk holding codes k .. k + 31 (k % 32 == 0)
// of row `row` in a code matrix with K codes per row, stored in MFMA
// operand-block order (1 KB blocks of 32 rows x 64 codes, lane-ordered).
__device__ __forceinline__ long code_chunk_offset(long row, int k, int K) {
  return ((row >> 5) * (K >> 6) + (k >> 6)) * 1024 + (((row & 31) + (((k >> 5) & 1) << 5)) << 4);
}

// Byte offset of the E8M0 scale of (row `row`, group k / 32) of an FP4 scale
// matrix in operand-block order: for each 32-row block and 128-wide K stage,
// 128 bytes; the 2-byte slot of MFMA lane (row % 32) + 32 ((k / 32) % 2)
// holds the scales of the stage's two 64-wide steps, (k / 64) % 2.
__device__ __forceinline__ long fp4_scale_offset(long row, int k, int K) {
  return ((row >> 5) * (K >> 7) + (k >> 7)) * 128 + (((row & 31) + (((k >> 5) & 1) << 5)) << 1) + ((k >> 6) & 1);
}

// Element offset of (row i, column t) of a bf16 matrix with `cols` columns
// (cols % 16 == 0) in MFMA operand-block order: 1 KB blocks of 32 rows x 16
// columns; inside a block, the 16-byte slot of lane (i % 32) + 32 * ((t % 16) / 8)
// holds columns 8 * (t / 8) .. + 7 of row i.
__device__ __forceinline__ long bf16_block_index(long i, int t, int cols) {
  return (((i >> 5) * (cols >> 4) + (t >> 4)) << 9) + (((i & 31) + (((t >> 3) & 1) << 5)) << 3) + (t & 7);
}

// Element offset of L1t[t][k] (t < R, R % 16 == 0, k < K) in the
// down-projection operand order: per 128-wide K chunk c = k / 128, column
// block nb = t / 16 and step j = (k % 32) / 8, a 1 KB block (blocks ordered
// by c, then nb, then j) whose 16-byte slot of lane (t % 16) + 16 ((k % 128) / 32)
// holds k - k % 8 .. + 7, the B operand of a 16x16x32 bf16 MFMA.
__host__ __device__ __forceinline__ long l1_operand_index(int t, long k, int R) {
  return ((((k >> 7) * (R >> 4) + (t >> 4)) * 4 + ((k >> 3) & 3)) << 9) + (((t & 15) + (((k >> 5) & 3) << 4)) << 3) +
         (k & 7);
}

// Direct global -> LDS copies (global_load_lds), written as inline asm so
// that the compiler's own wait insertion neither sees them nor adds
// conservative waits before LDS reads; every wait on them is explicit
// (s_waitcnt vmcnt counts them in issue order, together with any other
// vector memory operation of the wave).  A copy reads sbase + voff + OFF
// (64-bit scalar base, 32-bit per-lane offset, immediate OFF) and writes LDS
// at m0 + OFF + 16 l (4 l) for lane l: the immediate offset moves both
// addresses.  A copy needs one wait state after a scalar write of m0
// (set_m0_nop provides it; set_m0 leaves it to the caller).  Nothing else in
// these kernels uses m0 (the compiler warns that a reserved register in a
// clobber list may not be preserved, which these copies do not rely on: m0
// is always written right before the copies that read it).
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

// s_waitcnt lgkmcnt(0) (as a builtin, so the compiler knows this wave's LDS
// reads are complete), s_waitcnt vmcnt(n), then s_barrier; also a compiler
// memory barrier
constexpr int LGKM0 = 0xC07F;     // s_waitcnt encoding: lgkmcnt(0), vmcnt and expcnt unconstrained
#define SVDQ_VM_BARRIER(n)                  \
  do {                                      \
    __builtin_amdgcn_s_waitcnt(svdq::LGKM0); \
    asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_barrier" ::: "memory"); \
  } while (0)

// Workgroup (or persistent turn) id b -> output tile (tm, tn).  The hardware
// deals workgroups round-robin to the 8 XCDs, so b % 8 is the XCD and b / 8
// its j-th workgroup; each XCD works through its own set of tiles, so that
// its L2 serves the operand data its resident workgroups share.
//  map 1 (column strips; tiles_n % 8 == 0): XCD x owns tile columns
//    [x w, (x + 1) w), w = tiles_n / 8, and walks them row by row: its slice
//    of the weight codes stays in its L2 while the activation rows stream;
//  map 2 (row strips; tiles_m % 8 == 0): the same with rows and columns
//    exchanged;
//  map 0: XCD x takes a contiguous range of the tiles in 4-row groups
//    walked column by column.
// The launch picks the map whose resident slice is smaller (and fits an L2).
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int map, int& tm, int& tn) {
  constexpr int NXCD = 8, GROUP_TM = 4;
  const int x = b % NXCD, j = b / NXCD;
  if (map == 1) {
    const int w = tiles_n / NXCD;
    tm = j / w;
    tn = x * w + j % w;
    return;
  }
  if (map == 2) {
    const int h = tiles_m / NXCD;
    tn = j / h;
    tm = x * h + j % h;
    return;
  }
  const int T = tiles_m * tiles_n;
  const int q = T / NXCD, rem = T % NXCD;
  const int t = x * q + (x < rem ? x : rem) + j;
  const int per_group = GROUP_TM * tiles_n;
  const int grp = t / per_group;
  const int first = grp * GROUP_TM;
  const int gm = min(GROUP_TM, tiles_m - first);
  const int w = t - grp * per_group;
  tm = first + w % gm;
  tn = w / gm;
}

}  // namespace svdq
