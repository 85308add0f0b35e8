// sk_check.h -- input screening of a solve (SK_CHECK_FINITE; library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

// Bits ORed into the device word *bad by launch_check_inputs.
enum InputCheckBits : unsigned {
  kBadPoints = 1u,      // a coordinate of x or y is NaN or infinite
  kBadWeights = 2u,     // a weight is NaN, infinite or negative
  kPositiveA = 4u,      // some a_i > 0
  kPositiveB = 8u,      // some b_j > 0
  kBadPotentials = 16u  // a starting potential is NaN or infinite
};

// Clears *bad, then screens x, y (n x d and m x d as stored), a, b and, when
// f is non-null, the starting potentials f (n) and g (m).
hipError_t launch_check_inputs(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                               const float* a, const float* b, const float* f, const float* g,
                               unsigned* bad, hipStream_t s);

}  // namespace sk
