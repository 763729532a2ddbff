// Host construction of the NF4 tables (QLoRA, Heng's Blog, section
// "Contribution 1: 4-bit NormalFloat (NF4)"): 16 values at standard-normal
// quantiles with equal probability mass per bin, 8 for the negative half and 9
// for the positive half, the duplicated 0 dropped, scaled into [-1, 1].
//
// The standard-normal quantile (only probabilities >= 1/2 are needed, the
// negative half uses symmetry) is obtained by bisection on the upper tail
// erfc(x / sqrt(2)) / 2 to full float64 resolution. Levels are
// rounded to float32; threshold t_i is the largest float32 not above the
// exact midpoint of q_i and q_{i+1}, so that counting thresholds strictly
// below x picks the nearest level with ties to the lower index.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "lq_internal.h"

namespace lq {
namespace {

// Truncation probability of the outermost quantile (not given on the page;
// 1 - (1/32 + 1/30)/2 is the value the NF4 construction is usually quoted
// with).
const double kDelta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);

// Upper tail Q(x) = 1 - Phi(x) = erfc(x / sqrt(2)) / 2, accurate for x > 0.
double normal_upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }

// Phi^-1(p) for p in [1/2, 1): the x >= 0 with Q(x) = 1 - p (1 - p is exact
// there), by bisection until the bracket is two adjacent doubles, then the
// endpoint whose tail is nearer.
double normal_quantile_upper(double p) {
  if (p == 0.5) return 0.0;
  const double q = 1.0 - p;
  double lo = 0.0, hi = 40.0;
  for (int it = 0; it < 2000; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_upper_tail(mid) > q) lo = mid; else hi = mid;
  }
  return (std::fabs(normal_upper_tail(lo) - q) <= std::fabs(normal_upper_tail(hi) - q)) ? lo : hi;
}

float largest_f32_not_above(double m) {
  float f = (float)m;
  if ((double)f > m) f = std::nextafterf(f, -INFINITY);
  return f;
}

Tables build() {
  Tables t{};
  const double scale = normal_quantile_upper(kDelta);
  double vals[16];
  int n = 0;
  vals[n++] = 0.0;
  for (int j = 1; j <= 8; ++j)  // positive half: 9 quantiles, the first is 0
    vals[n++] = normal_quantile_upper(0.5 + (kDelta - 0.5) * ((double)j / 8.0)) / scale;
  for (int j = 1; j <= 7; ++j)  // negative half: 8 quantiles, the first is 0
    vals[n++] = -normal_quantile_upper(0.5 + (kDelta - 0.5) * ((double)j / 7.0)) / scale;
  // insertion sort, ascending
  for (int i = 1; i < 16; ++i)
    for (int k = i; k > 0 && vals[k] < vals[k - 1]; --k) {
      const double tmp = vals[k]; vals[k] = vals[k - 1]; vals[k - 1] = tmp;
    }
  for (int i = 0; i < 16; ++i) {
    t.levels[i] = (float)vals[i];
    t.lv.q[i] = t.levels[i];
  }
  for (int i = 0; i < 15; ++i)
    t.thresholds[i] = largest_f32_not_above(((double)t.levels[i] + (double)t.levels[i + 1]) / 2.0);

  // 33 bins of width 1/16 over [-1, 1 + 1/16), each widened by 2^-20.
  const double eps = std::ldexp(1.0, -20);
  for (int j = 0; j < 33; ++j) {
    const double lo = j / 16.0 - 1.0, hi = lo + 1.0 / 16.0;
    int base = 0, inside = 0;
    float T = 4.0f;
    for (int i = 0; i < 15; ++i) {
      const double ti = t.thresholds[i];
      if (ti < lo - eps) ++base;
      else if (ti <= hi + eps) { T = t.thresholds[i]; ++inside; }
    }
    if (inside > 1) {
      std::fprintf(stderr, "lq: NF4 thresholds closer than the search bins\n");
      std::abort();
    }
    t.lut.T[j] = T;
    t.lut.base[j] = base;
  }
  return t;
}

// NormalFloat levels of width b in float64, ascending in [-1, 1]: with
// h = 2^(b-1) and delta_b = 1 - (1/(2 * 2^b) + 1/(2 * (2^b - 1)))/2 (delta_4 is
// NF4's), h + 1 quantiles at probabilities 1/2 .. delta_b in equal steps on the
// positive half and h on the negative half, divided by Phi^-1(delta_b), the
// shared 0 kept once. Width 1 is {-1, +1}. These start the per-channel
// learner (LowRA, section 5: NormalFloat thresholds at 2 and 4 bits, 0 at 1
// bit; width 3 and delta_b for widths below 4 are not given there).
void nf_levels_f64(int bits, double* out) {
  if (bits == 1) {
    out[0] = -1.0;
    out[1] = 1.0;
    return;
  }
  const int n = 1 << bits, half = n / 2;
  const double delta = 1.0 - 0.5 * (1.0 / (2.0 * n) + 1.0 / (2.0 * (n - 1)));
  const double scale = normal_quantile_upper(delta);
  int c = 0;
  out[c++] = 0.0;
  for (int j = 1; j <= half; ++j)
    out[c++] = normal_quantile_upper(0.5 + (delta - 0.5) * ((double)j / (double)half)) / scale;
  for (int j = 1; j <= half - 1; ++j)
    out[c++] = -normal_quantile_upper(0.5 + (delta - 0.5) * ((double)j / (double)(half - 1))) / scale;
  for (int i = 1; i < n; ++i)
    for (int k = i; k > 0 && out[k] < out[k - 1]; --k) {
      const double tmp = out[k]; out[k] = out[k - 1]; out[k - 1] = tmp;
    }
}

LloydInit build_lloyd_init() {
  LloydInit li{};
  for (int b = 1; b <= 4; ++b) {
    const int n = 1 << b;
    nf_levels_f64(b, li.L[b - 1]);
    for (int i = 0; i + 1 < n; ++i) li.T[b - 1][i] = (li.L[b - 1][i] + li.L[b - 1][i + 1]) / 2.0;
  }
  return li;
}

}  // namespace

const LloydInit& lloyd_init() {
  static LloydInit li;
  static std::once_flag once;
  std::call_once(once, [] { li = build_lloyd_init(); });
  return li;
}

const Tables& tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] { t = build(); });
  return t;
}

}  // namespace lq
