// range_check.hpp — optional device check of the admissible input ranges.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>

namespace kda {

enum class RangeResult { InRange, OutOfRange, Capturing, HipError };

// Reads alpha[0..na), beta[0..nb) and theta[0..nt) on `stream` and reports
// whether every alpha lies in the mode's gate range (KDA: (0, 1]; CKDA:
// [-1, 1]), every beta in its write-strength range (KDA: [0, 1]; CKDA:
// [0, 2]) and every theta is finite; NaN is out of range.  Synchronises
// `stream`; refuses (Capturing) a stream under graph capture without
// enqueueing anything.  Null pointers with a zero count are allowed.
RangeResult check_ranges(const float* alpha, size_t na, const float* beta, size_t nb,
                         const float* theta, size_t nt, bool ckda, hipStream_t stream);

}  // namespace kda
