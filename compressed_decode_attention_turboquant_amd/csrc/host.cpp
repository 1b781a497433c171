// Host-side pieces of the method: the Beta Lloyd-Max codebook and the tier plan.
//
// Codebook [Ablation, Statistical Inference, and Validation for KV-Cache
// Compression, technical summary, "Experimental setup": a data-oblivious Beta
// Lloyd-Max codebook follows the random Walsh-Hadamard transform].  The
// quantised variable is one coordinate Y of a uniformly random unit vector in
// R^d, density proportional to (1 - y^2)^((d-3)/2) on [-1, 1].  With the
// substitution y = sin(theta) the cell mass and first moment become
//     mass   ~ int cos^(d-2)(theta) d theta
//     moment ~ int sin(theta) cos^(d-2)(theta) d theta
// on [asin a, asin b]; both integrands are smooth, so composite
// Gauss-Legendre quadrature reaches double precision.  Lloyd's two
// conditions are iterated to the fixed point.
//
// Tier plan [Tamarin (HSQ) summary, section 2, "Three-tier architecture"]:
// L1 = sinks + recent window + reader marks + a short trailing remainder;
// groups of N over the rest, in position order.
#include <algorithm>
#include <cmath>
#include <vector>

#include "hsq_internal.h"

namespace hsq {
namespace {

constexpr int kGL = 20;  // Gauss-Legendre points per panel

struct GaussLegendre {
  double x[kGL], w[kGL];
  GaussLegendre() {
    // Newton iteration on P_n for the n roots (Golub-Welsch-free classic form).
    const int n = kGL;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre& gl() {
  static const GaussLegendre g;
  return g;
}

// int_{t0}^{t1} cos^p(t) * (moment ? sin t : 1) dt by composite Gauss-Legendre
// with panels no wider than h.
double integrate(double t0, double t1, double p, bool moment, double h) {
  if (t1 <= t0) return 0.0;
  const GaussLegendre& g = gl();
  int panels = std::max(1, (int)std::ceil((t1 - t0) / h));
  double width = (t1 - t0) / panels, sum = 0.0;
  for (int k = 0; k < panels; ++k) {
    double a = t0 + k * width, mid = a + 0.5 * width, half = 0.5 * width;
    double acc = 0.0;
    for (int i = 0; i < kGL; ++i) {
      double t = mid + half * g.x[i];
      double c = std::cos(t);
      double f = (c > 0.0) ? std::exp(p * std::log(c)) : (p == 0.0 ? 1.0 : 0.0);
      if (moment) f *= std::sin(t);
      acc += g.w[i] * f;
    }
    sum += acc * half;
  }
  return sum;
}

}  // namespace

int codebook(int d, int bits, float* centroids, float* thresholds) {
  const int L = 1 << bits;
  const double p = d - 2.0;              // cos power after y = sin(theta)
  const double h = 0.25 / std::sqrt((double)d);
  const double sigma = 1.0 / std::sqrt((double)d);
  std::vector<double> c(L), t(L - 1), e(L + 1);
  // start: uniform cells over +-3 sigma, conditional means from there
  for (int j = 0; j < L - 1; ++j) t[j] = std::min(0.99, 3.0 * sigma) * (2.0 * (j + 1) / L - 1.0);
  auto centroids_of = [&](const std::vector<double>& thr, std::vector<double>& out) {
    e[0] = -M_PI / 2;
    e[L] = M_PI / 2;
    for (int j = 0; j < L - 1; ++j) e[j + 1] = std::asin(std::max(-1.0, std::min(1.0, thr[j])));
    for (int j = 0; j < L; ++j) {
      double m0 = integrate(e[j], e[j + 1], p, false, h);
      double m1 = integrate(e[j], e[j + 1], p, true, h);
      out[j] = m0 > 0.0 ? m1 / m0 : 0.5 * (std::sin(e[j]) + std::sin(e[j + 1]));
    }
  };
  centroids_of(t, c);
  std::vector<double> cn(L);
  for (int it = 0; it < 20000; ++it) {
    for (int j = 0; j < L - 1; ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
    centroids_of(t, cn);
    double delta = 0.0, cmax = 0.0;
    for (int j = 0; j < L; ++j) {
      delta = std::max(delta, std::fabs(cn[j] - c[j]));
      cmax = std::max(cmax, std::fabs(cn[j]));
    }
    c.swap(cn);
    if (delta <= 2e-14 * cmax) break;
  }
  // exact odd symmetry: middle threshold 0, zero goes to the lower cell
  for (int j = 0; j < L / 2; ++j) {
    double m = 0.5 * (c[L - 1 - j] - c[j]);
    c[L - 1 - j] = m;
    c[j] = -m;
  }
  // stored codebook: the fixed point's centroids and its thresholds (the
  // fp64 midpoints), each rounded to the nearest fp32, so the stored tables
  // satisfy both Lloyd conditions to fp32 rounding
  for (int j = 0; j < L; ++j) centroids[j] = (float)c[j];
  for (int j = 0; j < L - 1; ++j) thresholds[j] = (float)(0.5 * (c[j] + c[j + 1]));
  return HSQ_OK;
}

}  // namespace hsq

extern "C" int hsq_codebook(int d, int bits, float* centroids, float* thresholds) {
  if (!centroids || !thresholds) return hsq::fail(HSQ_ERR_ARG, "hsq_codebook: null output");
  if (d < 3 || d > 4096) return hsq::fail(HSQ_ERR_ARG, "hsq_codebook: d must be in [3, 4096]");
  if (bits < 1 || bits > 4) return hsq::fail(HSQ_ERR_ARG, "hsq_codebook: bits must be in [1, 4]");
  return hsq::codebook(d, bits, centroids, thresholds);
}

extern "C" int hsq_tier_plan(int T, int n_sink, int n_recent, const int32_t* marked, int n_marked,
                             int group_n, int32_t* l1_pos, int* n1, int32_t* group_pos,
                             int* n_groups) {
  if (T < 1 || n_sink < 0 || n_recent < 0 || n_marked < 0 || group_n < 1)
    return hsq::fail(HSQ_ERR_ARG, "hsq_tier_plan: bad sizes");
  if (n_marked > 0 && !marked) return hsq::fail(HSQ_ERR_ARG, "hsq_tier_plan: marked is null");
  if (!n1 || !n_groups) return hsq::fail(HSQ_ERR_ARG, "hsq_tier_plan: null count output");
  std::vector<uint8_t> l1(T, 0);
  for (int i = 0; i < std::min(n_sink, T); ++i) l1[i] = 1;
  for (int i = std::max(T - n_recent, 0); i < T; ++i) l1[i] = 1;
  for (int i = 0; i < n_marked; ++i) {
    if (marked[i] < 0 || marked[i] >= T)
      return hsq::fail(HSQ_ERR_ARG, "hsq_tier_plan: marked position out of range");
    l1[marked[i]] = 1;
  }
  std::vector<int32_t> rest;
  rest.reserve(T);
  for (int i = 0; i < T; ++i)
    if (!l1[i]) rest.push_back(i);
  const int ng = (int)(rest.size() / group_n);
  for (size_t i = (size_t)ng * group_n; i < rest.size(); ++i) l1[rest[i]] = 1;
  int cnt = 0;
  for (int i = 0; i < T; ++i)
    if (l1[i]) {
      if (l1_pos) l1_pos[cnt] = i;
      ++cnt;
    }
  if (group_pos)
    for (int i = 0; i < ng * group_n; ++i) group_pos[i] = rest[i];
  *n1 = cnt;
  *n_groups = ng;
  return HSQ_OK;
}
