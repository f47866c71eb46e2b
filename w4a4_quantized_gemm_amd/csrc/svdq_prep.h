// Offline-preparation internals (host side).
#pragma once

#include <cstdint>
#include <vector>

#include "svdq.h"

namespace svdq {

struct PrepOptions {
  int oversample = 64;    // extra subspace columns beyond the rank
  int iterations = 32;    // subspace (power) iterations
  uint64_t seed = 0x5344;  // seed of the Gaussian start block
};

// Smoothing factors lambda32 (the real a^alpha / w^(1 - alpha) rounded once
// to fp32; 1 where a channel's maximum is 0 or with no_smoothing) and
// inv32 = fp32(1 / lambda32), from host copies of the activation and weight
// channel maxima.
void smoothing_lambda(const float* a, const float* w, int K, float alpha, bool no_smoothing, float* lam, float* inv);

// Symmetric eigendecomposition by cyclic Jacobi rotations.  A is n x n
// row-major and is overwritten.  On return w holds the eigenvalues in
// descending order and V (n x n row-major) the matching eigenvectors as
// columns.
void jacobi_eigh(int n, std::vector<double>& A, std::vector<double>& V, std::vector<double>& w);

// Upper Cholesky factor U of A^-1 (A^-1 = U^T U) of a symmetric positive
// definite n x n row-major A; false if A is not positive definite.
bool cholesky_upper_of_inverse(int n, std::vector<double> A, std::vector<double>& U);

}  // namespace svdq

#include <hip/hip_runtime.h>

namespace svdq {
// Calibration activations for GPTQ on the residual (bf16 M x K, device).
struct GptqArgs {
  const uint16_t* X;
  int M;
  double damp;
};
svdq_status prepare_impl(const svdq_layer_desc& d, const uint16_t* W, const float* act_absmax,
                         const uint16_t* bias, const uint16_t* L1, const uint16_t* L2, uint8_t* blob,
                         hipStream_t st, const PrepOptions& opt, const GptqArgs* gptq = nullptr);
svdq_status merge_impl(const svdq_layer_desc& d, const uint8_t* old_blob, const uint16_t* A, const uint16_t* B,
                       int re, uint8_t* blob, hipStream_t st);
}  // namespace svdq
