/*
 * svdq_peaks.h - C ABI of libsvdq_peaks: microbenchmarks that measure the
 * MI355X (gfx950) throughput ceilings the layer's kernels are judged
 * against (matrix-core rates per operand type, HBM streaming bandwidth).
 * A measurement aid next to libsvdq, not part of the layer: nothing in the
 * layer calls it.  The datasheet peaks are dense-MFMA and HBM figures; these
 * probes report what simple, unobstructed loops reach on the device, with
 * constant and with random operand bits (the clock drops when the operands
 * toggle).
 *
 * Conventions as in svdq.h: host pointers unless named d_*, status codes
 * (0 = success), the current HIP device, synchronous calls (each launches,
 * times with HIP events on `stream` and waits).
 */
#ifndef SVDQ_PEAKS_H
#define SVDQ_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core probe kinds: the 32 x 32 block-scaled MFMA with E2M1 (FP4),
 * E2M3 (FP6) or E4M3 (FP8) operands, the int8 32x32x32 MFMA, the bf16
 * 32x32x16 MFMA and the f16 32x32x8 MFMA. */
typedef enum {
  SVDQ_PEAK_FP4 = 0,
  SVDQ_PEAK_FP6 = 1,
  SVDQ_PEAK_FP8 = 2,
  SVDQ_PEAK_INT8 = 3,
  SVDQ_PEAK_BF16 = 4,
  SVDQ_PEAK_F16 = 5
} svdq_peak_kind;

/* Every SIMD of the device runs `iters` rounds of 8 independent MFMAs of the
 * kind (4 waves per workgroup of 256 threads, `workgroups` workgroups, one
 * per compute unit gives one wave per SIMD); random_operands != 0 fills the
 * operand registers with
 * pseudo-random bits (valid codes of the format), else with a constant.
 * `workgroups` = 0 means one per compute unit.
 * *tops receives the dense operations per second / 1e12 (2 per
 * multiply-add), *ms the kernel time.  d_sink (256 floats per workgroup,
 * with workgroups = 0 meaning one per compute unit) receives a value derived
 * from the results so that nothing is optimized away.  Returns 0, 1 (invalid
 * argument) or 5 (HIP error). */
int svdq_peak_mfma(int kind, int iters, int workgroups, int random_operands, void* d_sink, double* tops, double* ms,
                   void* stream);

/* HBM streaming probe over caller buffers of `bytes` each (16-byte aligned,
 * a multiple of 16; larger than the 256 MB Infinity Cache to measure HBM):
 * mode 0 reads d_src (a checksum goes to d_dst's first 16 bytes), mode 1
 * copies d_src to d_dst.  *gbs receives bytes moved (read + written) per
 * second / 1e9, *ms the kernel time. */
int svdq_peak_hbm(int mode, const void* d_src, void* d_dst, size_t bytes, double* gbs, double* ms, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_PEAKS_H */
