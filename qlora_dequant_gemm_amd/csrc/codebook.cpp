// NF4 codebook and decision thresholds, derived on the host in fp64.
//
// Levels: "A 65B fine-tune on the GPU you already have", figure 3 (sixteen
// levels at quantiles of the zero-centred normal, equal mass per bin, dense
// near zero); "QLoRA and Quantized Training", section "The idea".
// Level i is the N(0,1) quantile at probability (i + 1/2)/16 -- the median of
// the i-th of 16 equal-mass bins -- divided by the largest one so that the
// levels span [-1, 1], then rounded to the nearest fp32. The positive half is
// computed and the negative half is its exact negation.
//
// Thresholds: code = number of thresholds strictly below v picks the nearest
// level with ties going to the lower index when threshold j is the largest
// fp32 that does not exceed the exact midpoint of levels j and j+1 (for an
// fp32 v, v > RD(m) <=> v > m). The midpoint of two fp32 values in [-1, 1] is
// exact in fp64.
#include <cmath>
#include <mutex>

#include "codebook.hpp"

namespace qnf4 {
namespace {

// Upper-tail probability of N(0,1): Q(x) = P(Z > x) = erfc(x / sqrt 2) / 2.
double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }

// x > 0 with Q(x) = q, for 0 < q < 1/2: bisection on the monotone tail, then
// Newton steps (dQ/dx = -phi(x)). Working in the upper tail keeps q, and so x,
// accurate to a few ulps.
double upper_quantile(double q) {
  double lo = 0.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (upper_tail(mid) > q) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  const double inv_sqrt_2pi = 0.39894228040143267794;
  for (int i = 0; i < 4; ++i) {
    double f = upper_tail(x) - q;
    double d = -inv_sqrt_2pi * std::exp(-0.5 * x * x);
    double nx = x - f / d;
    if (!(nx > 0.0) || nx == x) break;
    x = nx;
  }
  return x;
}

float round_down_f32(double m) {
  float f = static_cast<float>(m);            // nearest
  if (static_cast<double>(f) > m) f = std::nextafter(f, -INFINITY);
  return f;
}

Codebook g_cb;
bool g_ok = false;
std::once_flag g_once;

void derive() {
  // positive levels: probabilities (8.5 .. 15.5)/16, i.e. upper tails (7.5 .. 0.5)/16
  double z[8];
  for (int i = 0; i < 8; ++i) z[i] = upper_quantile((7.5 - i) / 16.0);
  const double top = z[7];
  for (int i = 0; i < 8; ++i) {
    float v = static_cast<float>(z[i] / top);
    g_cb.L[8 + i] = v;
    g_cb.L[7 - i] = -v;
  }
  for (int j = 0; j < 15; ++j) {
    double m = (static_cast<double>(g_cb.L[j]) + static_cast<double>(g_cb.L[j + 1])) / 2.0;
    g_cb.T[j] = round_down_f32(m);
  }
  g_cb.pad = 0.0f;
  bool ok = g_cb.L[0] == -1.0f && g_cb.L[15] == 1.0f;
  for (int j = 0; j < 15; ++j) ok = ok && g_cb.L[j] < g_cb.L[j + 1] && g_cb.T[j] >= g_cb.L[j] && g_cb.T[j] < g_cb.L[j + 1];
  // The quantize kernel's cell lookup (cell(v) = floor(64 v + 64.5)) needs
  // every threshold well inside its cell and at most one threshold per cell.
  int prev_cell = -1;
  for (int j = 0; j < 15; ++j) {
    const double pos = static_cast<double>(g_cb.T[j]) * 64.0 + 64.5;
    const double frac = pos - std::floor(pos);
    const int cell = static_cast<int>(std::floor(pos));
    ok = ok && frac > 64.0 * kCellMargin && frac < 1.0 - 64.0 * kCellMargin && cell > prev_cell;
    prev_cell = cell;
  }
  g_ok = ok;
}

}  // namespace

const Codebook* codebook() {
  std::call_once(g_once, derive);
  return g_ok ? &g_cb : nullptr;
}

}  // namespace qnf4
