// Host fp64 parts of the offline calibration (OSCAR, gist.science nl/fr
// technical summaries, section 2.2.A): order and signs of the eigenbasis of
// the covariance targets, the composite rotation R = U H P_br, and the clip
// quantile.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "calib_host.h"

namespace oscar {

// Eigenbasis from an eigen-decomposition V, w (V row-major, columns are
// eigenvectors; from the device Jacobi iteration): eigenvalues descending and
// each column's largest-magnitude entry positive (first index on ties).  U
// row-major, columns = vectors.
void sorted_basis(const std::vector<double> &V, const std::vector<double> &w, int n, std::vector<double> &U) {
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
  U.assign(size_t(n) * n, 0.0);
  for (int j = 0; j < n; ++j) {
    const int src = order[j];
    int arg = 0;
    double best = -1.0;
    for (int i = 0; i < n; ++i) {
      const double m = std::fabs(V[size_t(i) * n + src]);
      if (m > best) {
        best = m;
        arg = i;
      }
    }
    const double sgn = V[size_t(arg) * n + src] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i) U[size_t(i) * n + j] = sgn * V[size_t(i) * n + src];
  }
}

static int bitrev7(int i) {
  int r = 0;
  for (int b = 0; b < 7; ++b) r |= ((i >> b) & 1) << (6 - b);
  return r;
}

// R = U H P_br with H the normalised Sylvester Hadamard matrix and
// P_br[i][j] = 1 iff i = bitrev(j), so (M P_br)[i][j] = M[i][bitrev(j)].
void compose_rotation(const std::vector<double> &U, std::vector<double> &R) {
  const int n = 128;
  const double h = 1.0 / std::sqrt(double(n));
  std::vector<double> UH(size_t(n) * n);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      double s = 0.0;
      for (int k = 0; k < n; ++k) s += U[size_t(i) * n + k] * ((__builtin_popcount(k & j) & 1) ? -h : h);
      UH[size_t(i) * n + j] = s;
    }
  R.assign(size_t(n) * n, 0.0);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) R[size_t(i) * n + j] = UH[size_t(i) * n + bitrev7(j)];
}

// Quantile with linear interpolation between order statistics (type 7).
double quantile_linear(std::vector<double> &x, double p) {
  const size_t n = x.size();
  const double h = double(n - 1) * p;
  size_t lo = size_t(std::floor(h));
  if (lo >= n - 1) return *std::max_element(x.begin(), x.end());
  std::nth_element(x.begin(), x.begin() + lo, x.end());
  const double a = x[lo];
  const double b = *std::min_element(x.begin() + lo + 1, x.end());
  const double t = h - double(lo);
  return t >= 0.5 ? b - (b - a) * (1.0 - t) : a + (b - a) * t;
}

}  // namespace oscar
