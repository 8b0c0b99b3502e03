// 16-level codebooks shared by the host layer and the kernels (passed by value
// as a kernel argument, so the kernels read it from scalar registers): NF4, and
// the evenly spaced INT4 and the E2M1 FP4 levels the pages compare it with.
#pragma once

namespace qnf4 {

enum Format { kNF4 = 0, kINT4 = 1, kFP4 = 2, kNumFormats = 3 };

struct Codebook {
  float L[16];   // levels, ascending (FP4: -0 then +0 at 7, 8); L[7 - i] == -L[8 + i]
  float T[15];   // T[j] = largest fp32 <= midpoint(L[j], L[j+1])
  float pad;
};

// Smallest distance (in normalised-weight units) required between a threshold
// and an edge of the quantize kernel's lookup cells.
constexpr double kCellMargin = 1e-4;

// Derived once per format (thread-safe); nullptr if the derivation failed its
// checks or the format is unknown.
const Codebook* codebook(int format = kNF4);

}  // namespace qnf4
