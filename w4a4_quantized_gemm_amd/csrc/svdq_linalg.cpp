// Host-side numerics of the offline preparation (no HIP): the smoothing
// factors, a small dense symmetric eigensolver for the SVD, and the Cholesky
// factor GPTQ uses.
#include <quadmath.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

namespace svdq {

// lambda_j = a_j^alpha / w_j^(1 - alpha) (the handbook's SmoothQuant
// section) rounded once to fp32: evaluated as exp(alpha ln a - (1 - alpha)
// ln w) in binary128 (relative error near 2^-110), whose single rounding to
// fp32 is the correctly rounded value unless the real lambda lies within
// about 2^-100 of an fp32 rounding midpoint.  1 / lambda32 is rounded to
// fp64 and then fp32, which equals its correctly rounded fp32 value (53 >=
// 2 * 24 + 2).  Channels with a zero maximum keep lambda = 1.
void smoothing_lambda(const float* a, const float* w, int K, float alpha, bool no_smoothing, float* lam, float* inv) {
  const __float128 al = alpha;
  for (int j = 0; j < K; j++) {
    float l = 1.0f;
    if (!no_smoothing && a[j] > 0.0f && w[j] > 0.0f)
      l = static_cast<float>(expq(al * logq(static_cast<__float128>(a[j])) -
                                  (1 - al) * logq(static_cast<__float128>(w[j]))));
    lam[j] = l;
    inv[j] = static_cast<float>(1.0 / static_cast<double>(l));
  }
}

void jacobi_eigh(int n, std::vector<double>& A, std::vector<double>& V, std::vector<double>& w) {
  V.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; i++) V[static_cast<size_t>(i) * n + i] = 1.0;
  auto a = [&](int i, int j) -> double& { return A[static_cast<size_t>(i) * n + j]; };
  double diag2 = 0.0;
  for (int i = 0; i < n; i++) diag2 += a(i, i) * a(i, i);
  for (int sweep = 0; sweep < 100; sweep++) {
    double off = 0.0, tot = diag2;
    for (int p = 0; p < n; p++)
      for (int q = p + 1; q < n; q++) off += a(p, q) * a(p, q);
    tot = 0.0;
    for (int i = 0; i < n; i++) tot += a(i, i) * a(i, i);
    if (off <= 1e-32 * (tot + 2.0 * off) || off == 0.0) break;
    for (int p = 0; p < n; p++) {
      for (int q = p + 1; q < n; q++) {
        const double apq = a(p, q);
        if (apq == 0.0) continue;
        const double theta = (a(q, q) - a(p, p)) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; k++) {  // columns p, q
          const double akp = a(k, p), akq = a(k, q);
          a(k, p) = c * akp - s * akq;
          a(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < n; k++) {  // rows p, q
          const double apk = a(p, k), aqk = a(q, k);
          a(p, k) = c * apk - s * aqk;
          a(q, k) = s * apk + c * aqk;
        }
        a(p, q) = 0.0;
        a(q, p) = 0.0;
        for (int k = 0; k < n; k++) {
          double& vkp = V[static_cast<size_t>(k) * n + p];
          double& vkq = V[static_cast<size_t>(k) * n + q];
          const double x = vkp, y = vkq;
          vkp = c * x - s * y;
          vkq = s * x + c * y;
        }
      }
    }
  }
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int x, int y) { return a(x, x) > a(y, y); });
  std::vector<double> Vs(static_cast<size_t>(n) * n);
  w.resize(n);
  for (int c = 0; c < n; c++) {
    w[c] = a(order[c], order[c]);
    for (int k = 0; k < n; k++) Vs[static_cast<size_t>(k) * n + c] = V[static_cast<size_t>(k) * n + order[c]];
  }
  V.swap(Vs);
}

// Upper Cholesky factor U of A^-1 (A^-1 = U^T U) for a symmetric positive
// definite n x n row-major A, as GPTQ needs it: A = L L^T (lower Cholesky),
// L^-1 by forward substitution, A^-1 = L^-T L^-1, then A^-1 = G G^T and
// U = G^T.  Returns false if A is not numerically positive definite.  U is
// n x n row-major (zeros below the diagonal).
static bool cholesky_lower(int n, std::vector<double>& A) {
  for (int j = 0; j < n; j++) {
    double* aj = &A[static_cast<size_t>(j) * n];
    double d = aj[j];
    for (int k = 0; k < j; k++) d -= aj[k] * aj[k];
    if (!(d > 0.0)) return false;
    d = std::sqrt(d);
    aj[j] = d;
    for (int i = j + 1; i < n; i++) {
      double* ai = &A[static_cast<size_t>(i) * n];
      double v = ai[j];
      for (int k = 0; k < j; k++) v -= ai[k] * aj[k];
      ai[j] = v / d;
    }
  }
  for (int i = 0; i < n; i++)
    for (int j = i + 1; j < n; j++) A[static_cast<size_t>(i) * n + j] = 0.0;
  return true;
}

bool cholesky_upper_of_inverse(int n, std::vector<double> A, std::vector<double>& U) {
  if (!cholesky_lower(n, A)) return false;
  // Li = L^-1 (lower), column by column: L Li[:, c] = e_c
  std::vector<double> Li(static_cast<size_t>(n) * n, 0.0);
  for (int c = 0; c < n; c++) {
    for (int i = c; i < n; i++) {
      const double* li = &A[static_cast<size_t>(i) * n];
      double v = i == c ? 1.0 : 0.0;
      for (int k = c; k < i; k++) v -= li[k] * Li[static_cast<size_t>(k) * n + c];
      Li[static_cast<size_t>(i) * n + c] = v / li[i];
    }
  }
  // Ainv = Li^T Li: Ainv[i][j] = sum_{k >= max(i, j)} Li[k][i] Li[k][j]
  std::vector<double> Ai(static_cast<size_t>(n) * n, 0.0);
  for (int k = 0; k < n; k++) {
    const double* lk = &Li[static_cast<size_t>(k) * n];
    for (int i = 0; i <= k; i++) {
      const double v = lk[i];
      if (v == 0.0) continue;
      double* ai = &Ai[static_cast<size_t>(i) * n];
      for (int j = 0; j <= k; j++) ai[j] += v * lk[j];
    }
  }
  if (!cholesky_lower(n, Ai)) return false;
  U.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; i++)
    for (int j = i; j < n; j++) U[static_cast<size_t>(i) * n + j] = Ai[static_cast<size_t>(j) * n + i];
  return true;
}

}  // namespace svdq
