// Offline preparation of one SVDQuant layer (runs once per layer).
//
//   w_j   = max_n |W[j, n]|;  lambda_j = a_j^alpha / w_j^(1-alpha)
//           (quantization handbook, SmoothQuant section), fp64 -> fp32,
//           inv_lambda = fp32(1 / lambda32)
//   W_hat = lambda32 * W in fp64 (exact)
//   top-r SVD of W_hat (SVDQuant walkthrough eq. (5), handbook SVDQuant
//           section: L1 = U_r Sigma_r, L2 = V_r^T) by randomized subspace
//           iteration: the products with W_hat run in an fp64 GEMM kernel,
//           the small (r+p) x (r+p) eigenproblems of the orthonormalization
//           and the Rayleigh-Ritz step run on the host (cyclic Jacobi)
//   R     = W_hat - sum_t L1b[:, t] L2b[t, :]  (fp64, t increasing)
//   group quantization of R along K for every output column; packing into
//   the blob (codes N x K/2, scales N x K/g).
#include <cmath>
#include <cstring>
#include <random>
#include <vector>

#include "svdq_device.h"
#include "svdq_internal.h"
#include "svdq_prep.h"

namespace svdq {

// ---------------------------------------------------------------- fp64 helpers

// Round a finite double to a binary format with `mbits` fraction bits and
// `ebits` exponent bits (IEEE-style bias, gradual underflow, overflow to
// infinity), nearest-even, directly from the double (no intermediate fp32).
__device__ uint32_t f64_round_bits(double d, int mbits, int ebits) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(d));
  const uint32_t sign_bit = static_cast<uint32_t>(b >> 63) << (mbits + ebits);
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if ((mag >> 52) == 0) return sign_bit;  // zero (double subnormals are far below every target)
  const int e = static_cast<int>(mag >> 52) - 1023;
  const uint64_t m = (mag & ((1ull << 52) - 1)) | (1ull << 52);
  const int bias = (1 << (ebits - 1)) - 1;
  const int emin = 1 - bias;
  const int shift = 52 - mbits + (e < emin ? emin - e : 0);
  uint64_t kept = 0;
  if (shift < 64) {
    kept = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (kept & 1ull))) kept++;
  }
  uint32_t bits;
  if (e < emin) bits = static_cast<uint32_t>(kept);
  else bits = (static_cast<uint32_t>(e + bias) << mbits) + static_cast<uint32_t>(kept - (1ull << mbits));
  const uint32_t inf = ((1u << ebits) - 1u) << mbits;
  if (bits > inf) bits = inf;
  return sign_bit | bits;
}

// fp16 bits of the INT4 group scale A / 7, rounded to nearest even and
// saturated at the largest finite fp16 value (65504, bits 0x7BFF) instead of
// overflowing to infinity; codes then clamp to +-7.
__device__ __forceinline__ uint32_t int4_scale_bits(double a) {
  const uint32_t b = f64_round_bits(a / 7.0, 10, 5);
  return b > 0x7BFFu ? 0x7BFFu : b;
}

__device__ __forceinline__ double half_bits_to_f64(uint32_t h) {
  return static_cast<double>(__half2float(__ushort_as_half(static_cast<unsigned short>(h))));
}

// Round-half-even of the exact quotient x / s (s > 0 with at most 11
// significant bits, |x / s| <= 16): candidate from the fp64 quotient, then
// the exact sign of x - (q +- 1/2) s from one fma decides ties and near-ties.
__device__ __forceinline__ double rne_quotient_f64(double x, double s) {
  double q = rint(x / s);
  const double dhi = fma(-(q + 0.5), s, x);
  const double dlo = fma(-(q - 0.5), s, x);
  const bool odd = (static_cast<long long>(q) & 1ll) != 0;
  if (dhi > 0.0 || (dhi == 0.0 && odd)) q += 1.0;
  else if (dlo < 0.0 || (dlo == 0.0 && odd)) q -= 1.0;
  return q;
}

// Smallest e with a <= 6 * 2^e (a >= 0 finite), clamped to [-127, 127].
__device__ __forceinline__ int e8m0_exponent_f64(double a) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(a));
  const int eb = static_cast<int>((b >> 52) & 0x7FF);
  if (eb == 0) return -127;
  const int e = eb - 1025 + ((b & ((1ull << 52) - 1)) > (1ull << 51) ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ uint32_t e2m1_code_f64(double y) {
  const double m = fabs(y);
  uint32_t idx = (m > 0.25) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5) + (m > 5.0);
  return idx | ((y < 0.0 && idx != 0u) ? 8u : 0u);
}

// ---------------------------------------------------------------- kernels

__global__ void row_absmax_kernel(const uint16_t* __restrict__ W, int N, float* __restrict__ wmax) {
  __shared__ uint32_t red[256];
  const long j = blockIdx.x;
  uint32_t m = 0;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const uint32_t b = W[j * N + n] & 0x7FFFu;
    m = b > m ? b : m;
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = red[threadIdx.x] > red[threadIdx.x + s] ? red[threadIdx.x] : red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) wmax[j] = __uint_as_float(red[0] << 16);
}

__global__ void what_kernel(const uint16_t* __restrict__ W, const float* __restrict__ lam, int K, int N,
                            double* __restrict__ What) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(K) * N) return;
  const long j = idx / N;
  What[idx] = static_cast<double>(lam[j]) * static_cast<double>(__uint_as_float(static_cast<uint32_t>(W[idx]) << 16));
}

// C[M x N] = op(A)[M x K] * B[K x N] (row-major), op(A)[i][k] = TA ? A[k][i] : A[i][k].
template <bool TA>
__global__ __launch_bounds__(256) void dgemm_kernel(int M, int N, int K, const double* __restrict__ A, int lda,
                                                    const double* __restrict__ B, int ldb, double* __restrict__ C,
                                                    int ldc) {
  __shared__ double sA[16][65];
  __shared__ double sB[16][65];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const long m0 = static_cast<long>(blockIdx.y) * 64, n0 = static_cast<long>(blockIdx.x) * 64;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = tid + q * 256;
      if (!TA) {
        const int i = e >> 4, k = e & 15;
        const long gi = m0 + i, gk = k0 + k;
        sA[k][i] = (gi < M && gk < K) ? A[gi * lda + gk] : 0.0;
      } else {
        const int k = e >> 6, i = e & 63;
        const long gi = m0 + i, gk = k0 + k;
        sA[k][i] = (gi < M && gk < K) ? A[gk * lda + gi] : 0.0;
      }
      const int k = e >> 6, j = e & 63;
      const long gk = k0 + k, gj = n0 + j;
      sB[k][j] = (gk < K && gj < N) ? B[gk * ldb + gj] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; k++) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; u++) a[u] = sA[k][ty * 4 + u];
#pragma unroll
      for (int u = 0; u < 4; u++) b[u] = sB[k][tx * 4 + u];
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int v = 0; v < 4; v++) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const long gi = m0 + ty * 4 + u, gj = n0 + tx * 4 + v;
      if (gi < M && gj < N) C[gi * ldc + gj] = acc[u][v];
    }
}

// bf16(L1[j][t]) from an fp64 K x r matrix, into the down-projection
// operand order (l1_operand_index)
__global__ void store_l1t_kernel(const double* __restrict__ L1, int K, int r, uint16_t* __restrict__ l1t) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(K) * r) return;
  const long j = idx / r;
  const int t = static_cast<int>(idx % r);
  l1t[l1_operand_index(t, j, r)] = static_cast<uint16_t>(f64_round_bits(L1[idx], 7, 8));
}

// l2t = bf16(L2t) from an fp64 N x r matrix, stored in operand-block order
__global__ void store_l2t_kernel(const double* __restrict__ L2t, long count, int r, uint16_t* __restrict__ l2t) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= count) return;
  l2t[bf16_block_index(idx / r, static_cast<int>(idx % r), r)] = static_cast<uint16_t>(f64_round_bits(L2t[idx], 7, 8));
}

// Caller-supplied factors: L1 (K x r, row-major) -> l1t in the
// down-projection operand order
__global__ void store_given_l1_kernel(const uint16_t* __restrict__ L1, int K, int r, uint16_t* __restrict__ l1t) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(K) * r) return;
  l1t[l1_operand_index(static_cast<int>(idx % r), idx / r, r)] = L1[idx];
}

// Caller-supplied factors: L2 (r x N, row-major) -> l2t (N x r, operand-block order)
__global__ void store_given_l2_kernel(const uint16_t* __restrict__ L2, int r, int N, uint16_t* __restrict__ l2t) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(r) * N) return;
  l2t[bf16_block_index(idx % N, static_cast<int>(idx / N), r)] = L2[idx];
}

// R = W_hat - sum_t L1b[j][t] L2b[t][n], in place, t increasing.
__global__ void residual_kernel(double* __restrict__ What, const uint16_t* __restrict__ l1t,
                                const uint16_t* __restrict__ l2t, int K, int N, int r) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(K) * N) return;
  const long j = idx / N, n = idx % N;
  double s = 0.0;
  for (int t = 0; t < r; t++) {
    const double a = __uint_as_float(static_cast<uint32_t>(l1t[l1_operand_index(t, j, r)]) << 16);
    const double b = __uint_as_float(static_cast<uint32_t>(l2t[bf16_block_index(n, t, r)]) << 16);
    s = fma(a, b, s);  // the product of two bf16 numbers is exact in fp64
  }
  What[idx] = What[idx] - s;
}

// One thread per (output column n, K group g); n varies fastest.
template <int FMT>
__global__ void wquant_kernel(const double* __restrict__ R, int K, int N, uint8_t* __restrict__ wcodes,
                              void* __restrict__ wscales) {
  constexpr int G = FMT == SVDQ_INT4_G64_FP16 ? 64 : 32;
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long groups = K / G;
  if (idx >= groups * N) return;
  const long g = idx / N, n = idx % N;
  const double* col = R + g * G * static_cast<long>(N) + n;
  double a = 0.0;
  for (int k = 0; k < G; k++) a = fmax(a, fabs(col[static_cast<long>(k) * N]));
  uint32_t words[G / 8];
#pragma unroll
  for (int w = 0; w < G / 8; w++) words[w] = 0u;
  if constexpr (FMT == SVDQ_INT4_G64_FP16) {
    const uint32_t sbits = int4_scale_bits(a);
    const double s = half_bits_to_f64(sbits);
    if (s > 0.0) {
      for (int k = 0; k < G; k++) {
        double q = rne_quotient_f64(col[static_cast<long>(k) * N], s);
        q = fmin(fmax(q, -7.0), 7.0);
        words[k >> 3] |= int4_code_bits(static_cast<int>(q), k & 7);
      }
    }
    reinterpret_cast<uint16_t*>(wscales)[n * groups + g] = static_cast<uint16_t>(sbits);
  } else {
    const int e = e8m0_exponent_f64(a);
    for (int k = 0; k < G; k++) {
      const double y = ldexp(col[static_cast<long>(k) * N], -e);
      words[k >> 3] |= e2m1_code_f64(y) << (4 * (k & 7));
    }
    reinterpret_cast<uint8_t*>(wscales)[fp4_scale_offset(n, static_cast<int>(g * G), K)] = static_cast<uint8_t>(e + 127);
  }
#pragma unroll
  for (int w = 0; w < G / 32; w++)
    *reinterpret_cast<u32x4*>(wcodes + code_chunk_offset(n, static_cast<int>(g * G + 32 * w), K)) =
        u32x4{words[4 * w], words[4 * w + 1], words[4 * w + 2], words[4 * w + 3]};
}

// Merged low-rank factors for an extra branch dW = A B (A: K x re, B: re x
// N, bf16 row-major): columns t < r of L1 and rows t < r of L2 are the old
// blob's, the new ones are bf16(lambda32[k] A[k][t - r]) (the product is
// exact in fp64, rounded once) and B[t - r][n].  Thread per element of the
// merged factor, in the stored orders (l1_operand_index, bf16_block_index).
__global__ void merge_l1_kernel(const uint16_t* __restrict__ old_l1t, const float* __restrict__ lam,
                                const uint16_t* __restrict__ A, int K, int r, int re, uint16_t* __restrict__ l1t) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int R = r + re;
  if (idx >= static_cast<long>(K) * R) return;
  const long k = idx / R;
  const int t = static_cast<int>(idx % R);
  uint16_t v;
  if (t < r) {
    v = old_l1t[l1_operand_index(t, k, r)];
  } else {
    const double a = __uint_as_float(static_cast<uint32_t>(A[k * re + (t - r)]) << 16);
    v = static_cast<uint16_t>(f64_round_bits(static_cast<double>(lam[k]) * a, 7, 8));
  }
  l1t[l1_operand_index(t, k, R)] = v;
}

__global__ void merge_l2_kernel(const uint16_t* __restrict__ old_l2t, const uint16_t* __restrict__ B, int N, int r,
                                int re, uint16_t* __restrict__ l2t) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int R = r + re;
  if (idx >= static_cast<long>(N) * R) return;
  const long n = idx / R;
  const int t = static_cast<int>(idx % R);
  const uint16_t v = t < r ? old_l2t[bf16_block_index(n, t, r)] : B[static_cast<long>(t - r) * N + n];
  l2t[bf16_block_index(n, t, R)] = v;
}

// GPTQ on the residual (the walkthrough's Table 3 row on GPTQ): the rows
// (input channels) of R are quantized in order; the rounding error of row k,
// divided by U[k][k], is taken off the later rows with weights U[k][k+1:],
// U the upper Cholesky factor of H^-1, H = x_hat^T x_hat of calibration
// activations (damped).  A group's scales come from the current rows when k
// reaches its first row.  The quantization of one value is the round-to-
// nearest path's (wquant_kernel), so a diagonal H reproduces it exactly.

// x_hat of the calibration activations in fp64: fp32(x * inv_lambda), as the
// runtime computes it.
__global__ void xhat64_kernel(const uint16_t* __restrict__ X, const float* __restrict__ inv, long MK, int K,
                              double* __restrict__ out) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= MK) return;
  const float x = __uint_as_float(static_cast<uint32_t>(X[idx]) << 16);
  out[idx] = static_cast<double>(x * inv[idx % K]);
}

// Scales of the group starting at row k, one thread per column: fp16 bits
// (INT4) or the E8M0 byte (FP4).
template <int FMT>
__global__ void gptq_scale_kernel(const double* __restrict__ R, int k, int N, uint32_t* __restrict__ sc) {
  constexpr int G = FMT == SVDQ_INT4_G64_FP16 ? 64 : 32;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  double a = 0.0;
  for (int j = 0; j < G; j++) a = fmax(a, fabs(R[static_cast<long>(k + j) * N + n]));
  sc[static_cast<long>(k / G) * N + n] =
      FMT == SVDQ_INT4_G64_FP16 ? int4_scale_bits(a) : static_cast<uint32_t>(e8m0_exponent_f64(a) + 127);
}

// Row k: codes and the error (value - dequantized code) / U[k][k].
template <int FMT>
__global__ void gptq_row_kernel(const double* __restrict__ R, int k, int N, const uint32_t* __restrict__ sc, double ukk,
                                uint8_t* __restrict__ codes, double* __restrict__ err) {
  constexpr int G = FMT == SVDQ_INT4_G64_FP16 ? 64 : 32;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const double w = R[static_cast<long>(k) * N + n];
  const uint32_t sb = sc[static_cast<long>(k / G) * N + n];
  double deq;
  if constexpr (FMT == SVDQ_INT4_G64_FP16) {
    const double s = half_bits_to_f64(sb);
    double q = 0.0;
    if (s > 0.0) q = fmin(fmax(rne_quotient_f64(w, s), -7.0), 7.0);
    deq = q * s;
    codes[static_cast<long>(k) * N + n] = static_cast<uint8_t>(static_cast<int>(q) & 0xFF);
  } else {
    const int e = static_cast<int>(sb) - 127;
    const uint32_t c = e2m1_code_f64(ldexp(w, -e));
    const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    deq = ldexp((c & 8u) ? -grid[c & 7u] : grid[c & 7u], e);
    codes[static_cast<long>(k) * N + n] = static_cast<uint8_t>(c);
  }
  err[n] = (w - deq) / ukk;
}

// R[i][n] -= U[k][i] err[n] for the rows i > k.
__global__ void gptq_update_kernel(double* __restrict__ R, int k, int K, int N, const double* __restrict__ urow,
                                   const double* __restrict__ err) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(K - k - 1) * N) return;
  const long i = k + 1 + idx / N;
  const int n = static_cast<int>(idx % N);
  R[i * N + n] -= urow[i] * err[n];
}

// Packs the GPTQ codes and scales into the blob layout (the layout
// wquant_kernel writes); one thread per (output column n, K group g).
template <int FMT>
__global__ void gptq_pack_kernel(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ sc, int K, int N,
                                 uint8_t* __restrict__ wcodes, void* __restrict__ wscales) {
  constexpr int G = FMT == SVDQ_INT4_G64_FP16 ? 64 : 32;
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long groups = K / G;
  if (idx >= groups * N) return;
  const long g = idx / N, n = idx % N;
  uint32_t words[G / 8];
#pragma unroll
  for (int w = 0; w < G / 8; w++) words[w] = 0u;
  for (int k = 0; k < G; k++) {
    const uint8_t c = codes[(g * G + k) * N + n];
    if constexpr (FMT == SVDQ_INT4_G64_FP16)
      words[k >> 3] |= int4_code_bits(static_cast<int8_t>(c), k & 7);
    else
      words[k >> 3] |= static_cast<uint32_t>(c & 0xF) << (4 * (k & 7));
  }
  const uint32_t sb = sc[g * N + n];
  if constexpr (FMT == SVDQ_INT4_G64_FP16)
    reinterpret_cast<uint16_t*>(wscales)[n * groups + g] = static_cast<uint16_t>(sb);
  else
    reinterpret_cast<uint8_t*>(wscales)[fp4_scale_offset(n, static_cast<int>(g * G), K)] = static_cast<uint8_t>(sb);
#pragma unroll
  for (int w = 0; w < G / 32; w++)
    *reinterpret_cast<u32x4*>(wcodes + code_chunk_offset(n, static_cast<int>(g * G + 32 * w), K)) =
        u32x4{words[4 * w], words[4 * w + 1], words[4 * w + 2], words[4 * w + 3]};
}

__global__ void bias_kernel(const uint16_t* __restrict__ b, int N, float* __restrict__ out) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N) out[n] = __uint_as_float(static_cast<uint32_t>(b[n]) << 16);
}

// ---------------------------------------------------------------- host side

namespace {

struct DevBuf {
  void* p = nullptr;
  hipError_t alloc(size_t bytes) { return hipMalloc(&p, bytes ? bytes : 16); }
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
  double* d() const { return static_cast<double*>(p); }
};

#define SVDQ_TRY(x)                          \
  do {                                       \
    hipError_t e_ = (x);                     \
    if (e_ != hipSuccess) return SVDQ_ERR_HIP; \
  } while (0)

inline unsigned blocks_for(long n, int per = 256) { return static_cast<unsigned>((n + per - 1) / per); }

hipError_t dgemm(bool ta, int M, int N, int K, const double* A, int lda, const double* B, int ldb, double* C,
                 int ldc, hipStream_t st) {
  dim3 grid((N + 63) / 64, (M + 63) / 64), block(256);
  if (ta) hipLaunchKernelGGL(dgemm_kernel<true>, grid, block, 0, st, M, N, K, A, lda, B, ldb, C, ldc);
  else hipLaunchKernelGGL(dgemm_kernel<false>, grid, block, 0, st, M, N, K, A, lda, B, ldb, C, ldc);
  return hipGetLastError();
}

// Y (n x b, device) <- Y W with W = V diag(d)^-1/2 from the eigenpairs of
// G = Y^T Y; directions with d <= 1e-28 max(d) are dropped (set to zero).
// Two passes give columns orthonormal to fp64 precision.
svdq_status orthonormalize(double* Y, double* tmp, double* G, int n, int b, hipStream_t st) {
  std::vector<double> Gh(static_cast<size_t>(b) * b), V, w, Wm(static_cast<size_t>(b) * b);
  for (int pass = 0; pass < 2; pass++) {
    SVDQ_TRY(dgemm(true, b, b, n, Y, b, Y, b, G, b, st));
    SVDQ_TRY(hipMemcpyAsync(Gh.data(), G, Gh.size() * sizeof(double), hipMemcpyDeviceToHost, st));
    SVDQ_TRY(hipStreamSynchronize(st));
    jacobi_eigh(b, Gh, V, w);
    const double dmax = w.empty() ? 0.0 : w[0];
    for (int i = 0; i < b; i++)
      for (int c = 0; c < b; c++) {
        const double dc = w[c];
        Wm[static_cast<size_t>(i) * b + c] = (dc > 1e-28 * dmax && dc > 0.0) ? V[static_cast<size_t>(i) * b + c] / std::sqrt(dc) : 0.0;
      }
    SVDQ_TRY(hipMemcpyAsync(G, Wm.data(), Wm.size() * sizeof(double), hipMemcpyHostToDevice, st));
    SVDQ_TRY(dgemm(false, n, b, b, Y, b, G, b, tmp, b, st));
    SVDQ_TRY(hipMemcpyAsync(Y, tmp, static_cast<size_t>(n) * b * sizeof(double), hipMemcpyDeviceToDevice, st));
    SVDQ_TRY(hipStreamSynchronize(st));
  }
  return SVDQ_OK;
}

}  // namespace

template <int FMT>
svdq_status gptq_impl(const svdq_layer_desc& d, double* R, const float* inv, const GptqArgs& gq, uint8_t* wcodes,
                      void* wscales, hipStream_t st) {
  constexpr int G = FMT == SVDQ_INT4_G64_FP16 ? 64 : 32;
  const int K = d.K, N = d.N, Mc = gq.M;
  DevBuf xh, H;
  SVDQ_TRY(xh.alloc(sizeof(double) * static_cast<size_t>(Mc) * K));
  SVDQ_TRY(H.alloc(sizeof(double) * static_cast<size_t>(K) * K));
  const long MK = static_cast<long>(Mc) * K;
  hipLaunchKernelGGL(xhat64_kernel, dim3(blocks_for(MK)), dim3(256), 0, st, gq.X, inv, MK, K, xh.d());
  SVDQ_TRY(hipGetLastError());
  SVDQ_TRY(dgemm(true, K, K, Mc, xh.d(), K, xh.d(), K, H.d(), K, st));
  std::vector<double> Hh(static_cast<size_t>(K) * K), U;
  SVDQ_TRY(hipMemcpyAsync(Hh.data(), H.p, Hh.size() * sizeof(double), hipMemcpyDeviceToHost, st));
  SVDQ_TRY(hipStreamSynchronize(st));
  // a channel the calibration never activates gets 1 on the diagonal; then
  // damp * mean(diag) on every diagonal entry
  double mean = 0.0;
  for (int k = 0; k < K; k++) {
    double& h = Hh[static_cast<size_t>(k) * K + k];
    if (h == 0.0) h = 1.0;
    mean += h;
  }
  mean /= K;
  for (int k = 0; k < K; k++) Hh[static_cast<size_t>(k) * K + k] += gq.damp * mean;
  if (!cholesky_upper_of_inverse(K, Hh, U)) return SVDQ_ERR_INVALID_ARGUMENT;
  DevBuf dU, codes, sc, err;
  SVDQ_TRY(dU.alloc(sizeof(double) * static_cast<size_t>(K) * K));
  SVDQ_TRY(codes.alloc(static_cast<size_t>(K) * N));
  SVDQ_TRY(sc.alloc(sizeof(uint32_t) * static_cast<size_t>(K / G) * N));
  SVDQ_TRY(err.alloc(sizeof(double) * N));
  SVDQ_TRY(hipMemcpyAsync(dU.p, U.data(), U.size() * sizeof(double), hipMemcpyHostToDevice, st));
  uint8_t* cd = static_cast<uint8_t*>(codes.p);
  uint32_t* scd = static_cast<uint32_t*>(sc.p);
  for (int k = 0; k < K; k++) {
    if (k % G == 0) {
      hipLaunchKernelGGL(gptq_scale_kernel<FMT>, dim3(blocks_for(N)), dim3(256), 0, st, R, k, N, scd);
      SVDQ_TRY(hipGetLastError());
    }
    hipLaunchKernelGGL(gptq_row_kernel<FMT>, dim3(blocks_for(N)), dim3(256), 0, st, R, k, N, scd,
                       U[static_cast<size_t>(k) * K + k], cd, err.d());
    SVDQ_TRY(hipGetLastError());
    if (k + 1 < K) {
      hipLaunchKernelGGL(gptq_update_kernel, dim3(blocks_for(static_cast<long>(K - k - 1) * N)), dim3(256), 0, st, R, k,
                         K, N, dU.d() + static_cast<size_t>(k) * K, err.d());
      SVDQ_TRY(hipGetLastError());
    }
  }
  hipLaunchKernelGGL(gptq_pack_kernel<FMT>, dim3(blocks_for(static_cast<long>(K / G) * N)), dim3(256), 0, st, cd, scd,
                     K, N, wcodes, wscales);
  SVDQ_TRY(hipGetLastError());
  SVDQ_TRY(hipStreamSynchronize(st));
  return SVDQ_OK;
}

svdq_status prepare_impl(const svdq_layer_desc& d, const uint16_t* W, const float* act_absmax,
                         const uint16_t* bias, const uint16_t* L1, const uint16_t* L2, uint8_t* blob,
                         hipStream_t st, const PrepOptions& opt, const GptqArgs* gptq) {
  const int K = d.K, N = d.N, r = d.rank;
  const svdq_blob_layout L = layout_of(d);
  float* lam = reinterpret_cast<float*>(blob + L.lambda);
  float* inv = reinterpret_cast<float*>(blob + L.inv_lambda);
  uint16_t* l1t = reinterpret_cast<uint16_t*>(blob + L.l1t);
  uint16_t* l2t = reinterpret_cast<uint16_t*>(blob + L.l2t);
  const bool nosmooth = (d.flags & SVDQ_F_NO_SMOOTHING) != 0;

  // smoothing factors
  DevBuf wmax;
  SVDQ_TRY(wmax.alloc(sizeof(float) * K));
  hipLaunchKernelGGL(row_absmax_kernel, dim3(K), dim3(256), 0, st, W, N, static_cast<float*>(wmax.p));
  SVDQ_TRY(hipGetLastError());
  SVDQ_TRY(hipGetLastError());
  {
    // the factors themselves on the host (K values; the preparation is
    // synchronous anyway)
    std::vector<float> ha(K, 0.0f), hw(K), hl(K), hi(K);
    if (!nosmooth) SVDQ_TRY(hipMemcpyAsync(ha.data(), act_absmax, sizeof(float) * K, hipMemcpyDeviceToHost, st));
    SVDQ_TRY(hipMemcpyAsync(hw.data(), wmax.p, sizeof(float) * K, hipMemcpyDeviceToHost, st));
    SVDQ_TRY(hipStreamSynchronize(st));
    smoothing_lambda(ha.data(), hw.data(), K, d.alpha, nosmooth, hl.data(), hi.data());
    SVDQ_TRY(hipMemcpyAsync(lam, hl.data(), sizeof(float) * K, hipMemcpyHostToDevice, st));
    SVDQ_TRY(hipMemcpyAsync(inv, hi.data(), sizeof(float) * K, hipMemcpyHostToDevice, st));
    SVDQ_TRY(hipStreamSynchronize(st));
  }

  // W_hat in fp64
  const long KN = static_cast<long>(K) * N;
  DevBuf what;
  SVDQ_TRY(what.alloc(sizeof(double) * KN));
  hipLaunchKernelGGL(what_kernel, dim3(blocks_for(KN)), dim3(256), 0, st, W, lam, K, N, what.d());
  SVDQ_TRY(hipGetLastError());

  // low-rank factors
  if (r > 0) {
    if (d.flags & SVDQ_F_FACTORS_GIVEN) {
      hipLaunchKernelGGL(store_given_l1_kernel, dim3(blocks_for(static_cast<long>(K) * r)), dim3(256), 0, st, L1, K, r, l1t);
      SVDQ_TRY(hipGetLastError());
      hipLaunchKernelGGL(store_given_l2_kernel, dim3(blocks_for(static_cast<long>(r) * N)), dim3(256), 0, st, L2, r, N, l2t);
      SVDQ_TRY(hipGetLastError());
    } else {
      const int b = r + opt.oversample > (K < N ? K : N) ? (K < N ? K : N) : r + opt.oversample;
      DevBuf Q, Qt, Z, Zt, G, Om;
      SVDQ_TRY(Q.alloc(sizeof(double) * K * b));
      SVDQ_TRY(Qt.alloc(sizeof(double) * K * b));
      SVDQ_TRY(Z.alloc(sizeof(double) * N * b));
      SVDQ_TRY(Zt.alloc(sizeof(double) * N * b));
      SVDQ_TRY(G.alloc(sizeof(double) * b * b));
      SVDQ_TRY(Om.alloc(sizeof(double) * N * b));
      {
        std::mt19937_64 gen(opt.seed);
        std::normal_distribution<double> nd(0.0, 1.0);
        std::vector<double> om(static_cast<size_t>(N) * b);
        for (auto& x : om) x = nd(gen);
        SVDQ_TRY(hipMemcpyAsync(Om.p, om.data(), om.size() * sizeof(double), hipMemcpyHostToDevice, st));
        SVDQ_TRY(hipStreamSynchronize(st));
      }
      svdq_status s;
      SVDQ_TRY(dgemm(false, K, b, N, what.d(), N, Om.d(), b, Q.d(), b, st));
      if ((s = orthonormalize(Q.d(), Qt.d(), G.d(), K, b, st)) != SVDQ_OK) return s;
      for (int it = 0; it < opt.iterations; it++) {
        SVDQ_TRY(dgemm(true, N, b, K, what.d(), N, Q.d(), b, Z.d(), b, st));
        if ((s = orthonormalize(Z.d(), Zt.d(), G.d(), N, b, st)) != SVDQ_OK) return s;
        SVDQ_TRY(dgemm(false, K, b, N, what.d(), N, Z.d(), b, Q.d(), b, st));
        if ((s = orthonormalize(Q.d(), Qt.d(), G.d(), K, b, st)) != SVDQ_OK) return s;
      }
      // Rayleigh-Ritz: B^T = W_hat^T Q (N x b); H = B B^T = U diag(sigma^2) U^T
      SVDQ_TRY(dgemm(true, N, b, K, what.d(), N, Q.d(), b, Z.d(), b, st));
      SVDQ_TRY(dgemm(true, b, b, N, Z.d(), b, Z.d(), b, G.d(), b, st));
      std::vector<double> H(static_cast<size_t>(b) * b), V, w;
      SVDQ_TRY(hipMemcpyAsync(H.data(), G.p, H.size() * sizeof(double), hipMemcpyDeviceToHost, st));
      SVDQ_TRY(hipStreamSynchronize(st));
      jacobi_eigh(b, H, V, w);
      // Wl = U_r diag(sigma_r) (b x r), Wr = U_r diag(1/sigma_r) (b x r)
      std::vector<double> Wl(static_cast<size_t>(b) * r), Wr(static_cast<size_t>(b) * r);
      const double tiny = (w.empty() ? 0.0 : w[0]) * 1e-28;
      for (int i = 0; i < b; i++)
        for (int c = 0; c < r; c++) {
          const double sig = w[c] > tiny && w[c] > 0.0 ? std::sqrt(w[c]) : 0.0;
          const double u = V[static_cast<size_t>(i) * b + c];
          Wl[static_cast<size_t>(i) * r + c] = u * sig;
          Wr[static_cast<size_t>(i) * r + c] = sig > 0.0 ? u / sig : 0.0;
        }
      DevBuf dWl, dWr, dL1, dL2t;
      SVDQ_TRY(dWl.alloc(sizeof(double) * b * r));
      SVDQ_TRY(dWr.alloc(sizeof(double) * b * r));
      SVDQ_TRY(dL1.alloc(sizeof(double) * K * r));
      SVDQ_TRY(dL2t.alloc(sizeof(double) * N * r));
      SVDQ_TRY(hipMemcpyAsync(dWl.p, Wl.data(), Wl.size() * sizeof(double), hipMemcpyHostToDevice, st));
      SVDQ_TRY(hipMemcpyAsync(dWr.p, Wr.data(), Wr.size() * sizeof(double), hipMemcpyHostToDevice, st));
      SVDQ_TRY(dgemm(false, K, r, b, Q.d(), b, dWl.d(), r, dL1.d(), r, st));
      SVDQ_TRY(dgemm(false, N, r, b, Z.d(), b, dWr.d(), r, dL2t.d(), r, st));
      hipLaunchKernelGGL(store_l1t_kernel, dim3(blocks_for(static_cast<long>(K) * r)), dim3(256), 0, st, dL1.d(), K, r, l1t);
      SVDQ_TRY(hipGetLastError());
      hipLaunchKernelGGL(store_l2t_kernel, dim3(blocks_for(static_cast<long>(N) * r)), dim3(256), 0, st, dL2t.d(),
                         static_cast<long>(N) * r, r, l2t);
      SVDQ_TRY(hipGetLastError());
      SVDQ_TRY(hipStreamSynchronize(st));
    }
    hipLaunchKernelGGL(residual_kernel, dim3(blocks_for(KN)), dim3(256), 0, st, what.d(), l1t, l2t, K, N, r);
    SVDQ_TRY(hipGetLastError());
  }

  // residual quantization + packing
  uint8_t* wcodes = blob + L.wcodes;
  void* wscales = blob + L.wscales;
  const long groups = static_cast<long>(K / group_of(d.fmt)) * N;
  if (gptq) {
    const svdq_status gs = d.fmt == SVDQ_INT4_G64_FP16 ? gptq_impl<SVDQ_INT4_G64_FP16>(d, what.d(), inv, *gptq, wcodes, wscales, st)
                                                      : gptq_impl<SVDQ_FP4_E2M1_G32_E8M0>(d, what.d(), inv, *gptq, wcodes, wscales, st);
    if (gs != SVDQ_OK) return gs;
  } else if (d.fmt == SVDQ_INT4_G64_FP16)
    hipLaunchKernelGGL(wquant_kernel<SVDQ_INT4_G64_FP16>, dim3(blocks_for(groups)), dim3(256), 0, st, what.d(), K, N,
                       wcodes, wscales);
  else
    hipLaunchKernelGGL(wquant_kernel<SVDQ_FP4_E2M1_G32_E8M0>, dim3(blocks_for(groups)), dim3(256), 0, st, what.d(), K,
                       N, wcodes, wscales);
  SVDQ_TRY(hipGetLastError());

  if (d.flags & SVDQ_F_HAS_BIAS) {
    hipLaunchKernelGGL(bias_kernel, dim3(blocks_for(N)), dim3(256), 0, st, bias, N,
                       reinterpret_cast<float*>(blob + L.bias));
    SVDQ_TRY(hipGetLastError());
  }

  // header last
  BlobHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kMagic;
  h.version = kVersion;
  h.fmt = d.fmt;
  h.K = K;
  h.N = N;
  h.rank = r;
  h.flags = d.flags;
  h.group = group_of(d.fmt);
  h.alpha = d.alpha;
  h.layout = L;
  SVDQ_TRY(hipMemcpyAsync(blob, &h, sizeof(h), hipMemcpyHostToDevice, st));
  SVDQ_TRY(hipStreamSynchronize(st));
  return SVDQ_OK;
}

svdq_status merge_impl(const svdq_layer_desc& d, const uint8_t* old_blob, const uint16_t* A, const uint16_t* B,
                       int re, uint8_t* blob, hipStream_t st) {
  svdq_layer_desc dn = d;
  dn.rank = d.rank + re;
  const svdq_blob_layout Lo = layout_of(d), Ln = layout_of(dn);
  const int K = d.K, N = d.N, r = d.rank;
  // sections that do not depend on the rank are copied as they are
  SVDQ_TRY(hipMemcpyAsync(blob + Ln.lambda, old_blob + Lo.lambda, 4ul * K, hipMemcpyDeviceToDevice, st));
  SVDQ_TRY(hipMemcpyAsync(blob + Ln.inv_lambda, old_blob + Lo.inv_lambda, 4ul * K, hipMemcpyDeviceToDevice, st));
  SVDQ_TRY(hipMemcpyAsync(blob + Ln.wcodes, old_blob + Lo.wcodes, static_cast<size_t>(N) * K / 2,
                          hipMemcpyDeviceToDevice, st));
  SVDQ_TRY(hipMemcpyAsync(blob + Ln.wscales, old_blob + Lo.wscales,
                          static_cast<size_t>(K / group_of(d.fmt)) * N * scale_bytes_of(d.fmt), hipMemcpyDeviceToDevice,
                          st));
  if (d.flags & SVDQ_F_HAS_BIAS)
    SVDQ_TRY(hipMemcpyAsync(blob + Ln.bias, old_blob + Lo.bias, 4ul * N, hipMemcpyDeviceToDevice, st));
  hipLaunchKernelGGL(merge_l1_kernel, dim3(blocks_for(static_cast<long>(K) * dn.rank)), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(old_blob + Lo.l1t),
                     reinterpret_cast<const float*>(old_blob + Lo.lambda), A, K, r, re,
                     reinterpret_cast<uint16_t*>(blob + Ln.l1t));
  SVDQ_TRY(hipGetLastError());
  hipLaunchKernelGGL(merge_l2_kernel, dim3(blocks_for(static_cast<long>(N) * dn.rank)), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(old_blob + Lo.l2t), B, N, r, re,
                     reinterpret_cast<uint16_t*>(blob + Ln.l2t));
  SVDQ_TRY(hipGetLastError());
  BlobHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kMagic;
  h.version = kVersion;
  h.fmt = dn.fmt;
  h.K = K;
  h.N = N;
  h.rank = dn.rank;
  h.flags = dn.flags;
  h.group = group_of(dn.fmt);
  h.alpha = dn.alpha;
  h.layout = Ln;
  // header last, from host memory: the call returns after the stream has
  // drained
  SVDQ_TRY(hipMemcpyAsync(blob, &h, sizeof(h), hipMemcpyHostToDevice, st));
  SVDQ_TRY(hipStreamSynchronize(st));
  return SVDQ_OK;
}

}  // namespace svdq
