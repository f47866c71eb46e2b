// Launchers of the libsvdq HIP kernels (internal; host-callable).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "svdq.h"
#include "svdq_internal.h"

namespace svdq {

struct ActArgs {
  const uint16_t* X;      // M x K bf16
  int M, K, rank;
  const float* inv_lam;   // K
  const uint16_t* l1t;    // rank x K bf16
  uint8_t* codes;         // M x K/2
  void* scales;           // M x K/g (fp16 bits or E8M0 bytes)
  uint16_t* Tb;           // M x rank bf16
  float* tpart;           // kMaxKParts x M x rank fp32 partial T (workspace), or null: K is not split
  const float* rowstat = nullptr;  // norm-fused pass: M x {mean, 1/std}; inv_lam then holds gamma', beta' (2K)
};

// Compute units of the current device (cached per device).
int device_cu_count();

// quant: write codes + scales; down: write Tb.
hipError_t launch_act(int fmt, bool quant, bool down, const ActArgs& a, hipStream_t st);
// Row mean and 1/sqrt(var + eps) of X (M x {mu, rho}) and the norm's affine
// with the smoothing folded in (gamma' then beta', 2K floats).
hipError_t launch_norm_stats(const uint16_t* X, int M, int K, float eps, const uint16_t* gamma, const uint16_t* beta,
                             const float* inv_lam, float* rowstat, float* fold, hipStream_t st);
hipError_t launch_absmax(const uint16_t* X, int M, int K, float* out, bool accumulate, hipStream_t st);

struct GemmArgs {
  const uint8_t* acodes;  // M x K/2
  const void* ascales;    // M x K/g
  const uint8_t* wcodes;  // N x K/2
  const void* wscales;    // K/g x N
  const uint16_t* Tb;     // M x rank (slab A operand), may be null if rank == 0 or !slab
  const uint16_t* l2t;    // N x rank (slab B operand)
  const float* bias;      // N or null
  void* Y;                // M x N, bf16 bits or fp32
  int M, K, N, rank;
  int xcd_map;            // tile -> XCD assignment (tile_of), set by the launch
  // INT4 GEMM: workspace for the fp32 partial tiles of a K split (at most
  // kGemmSplitItems 128 x 128 tiles), or null: K is not split
  float* ypart;
  int kparts;             // set by the launch (1: no split)
};

// The tile -> XCD map for a GEMM of tiles_m x tiles_n tiles over M x K
// activations and N x K weights (4-bit codes): column strips when the weight
// slice per XCD is the smaller one and fits in an L2, row strips in the
// opposite case, else contiguous 4-row groups.
int gemm_xcd_map(int M, int N, int K, int tiles_m, int tiles_n);

// slab: append the rank-r bf16 K-slab Tb L2b before the epilogue.
hipError_t launch_gemm(int fmt, bool slab, int out_dtype, const GemmArgs& g, hipStream_t st);
// the FP4 variant (persistent, block-scaled MFMA); launch_gemm dispatches to it
hipError_t launch_gemm_fp4(bool slab, int out_dtype, const GemmArgs& g, hipStream_t st);

struct W4A16Args {
  const uint16_t* X;      // M x K bf16 (M <= kW4A16MaxM)
  int M, K, N;
  const float* inv_lam;   // K
  const uint8_t* wcodes;  // N x K/2 (operand-block order)
  const void* wscales;
  const float* bias;      // N or null
  void* Y;                // M x N
  int out_f32;
  void* pieces;           // workspace: the bf16 pieces of x_hat in MFMA A-operand order (K * 64 * w4a16_planes(M) bytes)
};
// The weight-only 4-bit layer (rank 0 blob), small M.
hipError_t launch_w4a16(int fmt, const W4A16Args& a, hipStream_t st);

// Unfused up-projection: Y = round(Y + Tb L2b) in place.
hipError_t launch_up(int out_dtype, const uint16_t* Tb, const uint16_t* l2t, void* Y, int M, int N,
                     int rank, hipStream_t st);

}  // namespace svdq
