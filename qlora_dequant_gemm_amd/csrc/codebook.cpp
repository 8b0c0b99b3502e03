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
//
// The other formats ("QLoRA Explained", "The three ideas behind QLoRA": NF4
// beats the standard 4-bit integer and float formats on normal weights; "A 65B
// fine-tune on the GPU you already have", figure 3): INT4 = the 16 evenly
// spaced levels (2i - 15) / 15; FP4 = the E2M1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6
// divided by 6, with -0 and +0 as codes 7 and 8 (the threshold between them is
// 0, so v <= 0 takes -0 and v > 0 takes +0).
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

Codebook g_cb[kNumFormats];
bool g_ok[kNumFormats] = {false, false, false};
std::once_flag g_once;

// positive half of each format's levels, fp64 (index 8 + i)
void positive_levels(int format, double (&p)[8]) {
  if (format == kNF4) {
    // probabilities (8.5 .. 15.5)/16, i.e. upper tails (7.5 .. 0.5)/16
    double z[8];
    for (int i = 0; i < 8; ++i) z[i] = upper_quantile((7.5 - i) / 16.0);
    for (int i = 0; i < 8; ++i) p[i] = z[i] / z[7];
  } else if (format == kINT4) {
    for (int i = 0; i < 8; ++i) p[i] = (2.0 * (8 + i) - 15.0) / 15.0;
  } else {
    const double e2m1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (int i = 0; i < 8; ++i) p[i] = e2m1[i] / 6.0;
  }
}

bool derive_one(int format, Codebook& cb) {
  double p[8];
  positive_levels(format, p);
  for (int i = 0; i < 8; ++i) {
    const float v = static_cast<float>(p[i]);
    cb.L[8 + i] = v;
    cb.L[7 - i] = -v;                          // exact negation (FP4: -0 at 7)
  }
  for (int j = 0; j < 15; ++j) {
    double m = (static_cast<double>(cb.L[j]) + static_cast<double>(cb.L[j + 1])) / 2.0;
    cb.T[j] = round_down_f32(m);
    if (cb.T[j] == 0.0f) cb.T[j] = 0.0f;       // +0
  }
  cb.pad = 0.0f;
  bool ok = cb.L[0] == -1.0f && cb.L[15] == 1.0f;
  for (int j = 0; j < 15; ++j) {
    const bool zeros = cb.L[j] == 0.0f && cb.L[j + 1] == 0.0f && std::signbit(cb.L[j]) && !std::signbit(cb.L[j + 1]);
    ok = ok && (cb.L[j] < cb.L[j + 1] || zeros) && cb.T[j] >= cb.L[j] && (cb.T[j] < cb.L[j + 1] || zeros);
  }
  // The quantize kernel's cell lookup (cell(v) = floor(64 v + 64.5)) needs
  // every threshold well inside its cell and at most one threshold per cell.
  int prev_cell = -1;
  for (int j = 0; j < 15; ++j) {
    const double pos = static_cast<double>(cb.T[j]) * 64.0 + 64.5;
    const double frac = pos - std::floor(pos);
    const int cell = static_cast<int>(std::floor(pos));
    ok = ok && frac > 64.0 * kCellMargin && frac < 1.0 - 64.0 * kCellMargin && cell > prev_cell;
    prev_cell = cell;
  }
  return ok;
}

void derive() {
  for (int f = 0; f < kNumFormats; ++f) g_ok[f] = derive_one(f, g_cb[f]);
}

}  // namespace

const Codebook* codebook(int format) {
  if (format < 0 || format >= kNumFormats) return nullptr;
  std::call_once(g_once, derive);
  return g_ok[format] ? &g_cb[format] : nullptr;
}

}  // namespace qnf4
