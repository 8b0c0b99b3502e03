// NF4 codebook shared by the host layer and the kernels (passed by value as a
// kernel argument, so the kernels read it from scalar registers).
#pragma once

namespace qnf4 {

struct Codebook {
  float L[16];   // levels, ascending; L[7 - i] == -L[8 + i]
  float T[15];   // T[j] = largest fp32 <= midpoint(L[j], L[j+1])
  float pad;
};

// Smallest distance (in normalised-weight units) required between a threshold
// and an edge of the quantize kernel's lookup cells.
constexpr double kCellMargin = 1e-4;

// Derived once (thread-safe); nullptr if the derivation failed its checks.
const Codebook* codebook();

}  // namespace qnf4
