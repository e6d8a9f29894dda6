// Opt-in (SSD_DEBUG=1) device checks of caller preconditions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Validates seq_idx (non-decreasing, values in [0, num_seqs)) on `stream` and
// waits for the answer.  *first_bad = the lowest offending token index, or
// INT_MAX if there is none.
hipError_t check_seq_idx(const int32_t *seq, int L, int num_seqs, hipStream_t stream, int *first_bad);

}  // namespace ssd
