// NF4 level table and decision thresholds, built on the host.
//
// [QLoRA / infivelines.com]: NF4 places its 16 levels at quantiles of a
// normal distribution so each level is about equally likely to be used.
// The format fixes an exact zero and the range [-1, 1], so the 16 levels
// are 8 above zero and 7 below: each side at normal quantiles of evenly
// spaced probabilities between 1/2 (excluded) and p_max, where p_max is the
// mean of the outermost equal-mass bin centres for 15 and 16 levels,
// ((1 - 1/30) + (1 - 1/32)) / 2.  Dividing by the quantile of p_max makes
// the end levels exactly -1 and +1.  Levels are built in double precision
// and rounded once to fp32.
//
// The normal quantile here is this library's own: Newton's method on
// Phi(x) = erfc(-x/sqrt 2)/2 using libm's erfc, started at 0.  For p >= 1/2
// Phi is concave on [0, inf), so the iterates rise monotonically to the
// root; iteration stops when a step no longer moves x.
//
// Thresholds: a code is the index of the nearest fp32 level, ties to the
// lower level.  For fp32 u that is "u > midpoint", and the fp32 threshold
// that decides it exactly is the midpoint rounded towards -infinity.

#include <cmath>
#include <cstdint>
#include <mutex>

#include "nf4_table.h"

namespace qlora {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_pdf(double x) {
  static const double inv_sqrt_2pi = 0.39894228040143267794;
  return inv_sqrt_2pi * std::exp(-0.5 * x * x);
}

// Quantile of the standard normal for p in [1/2, 1).
double normal_quantile_upper(double p) {
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double step = (normal_cdf(x) - p) / normal_pdf(x);
    const double nx = x - step;
    if (nx == x || !(std::fabs(step) > 0.0)) break;
    // once converged, Newton can oscillate between neighbouring doubles;
    // keep the one with the smaller residual
    if (it > 50 && std::fabs(normal_cdf(nx) - p) >= std::fabs(normal_cdf(x) - p))
      break;
    x = nx;
  }
  return x;
}

Nf4Table g_table;
std::once_flag g_once;

void build() {
  const double p_max = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  const double top = normal_quantile_upper(p_max);
  double lv[16];
  int n = 0;
  // negative side, most negative first: 7 probabilities from p_max
  for (int i = 0; i < 7; ++i) {
    const double p = p_max - (p_max - 0.5) * i / 7.0;
    lv[n++] = -normal_quantile_upper(p);
  }
  lv[n++] = 0.0;
  // positive side, ascending: 8 probabilities from just above 1/2 to p_max
  for (int i = 7; i >= 0; --i) {
    const double p = p_max - (p_max - 0.5) * i / 8.0;
    lv[n++] = normal_quantile_upper(p);
  }
  for (int i = 0; i < 16; ++i) g_table.level[i] = static_cast<float>(lv[i] / top);
  for (int i = 0; i < 15; ++i) {
    const double mid = (static_cast<double>(g_table.level[i]) +
                        static_cast<double>(g_table.level[i + 1])) / 2.0;
    float t = static_cast<float>(mid);
    if (static_cast<double>(t) > mid) t = std::nextafter(t, -INFINITY);
    g_table.threshold[i] = t;
  }
}

}  // namespace

const Nf4Table& nf4_table() {
  std::call_once(g_once, build);
  return g_table;
}

}  // namespace qlora
