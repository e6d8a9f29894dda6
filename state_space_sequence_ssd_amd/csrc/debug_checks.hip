// Opt-in device checks of caller preconditions that host code cannot see
// (SSD_DEBUG=1 in the environment).  They run on the caller's stream before
// the kernels that rely on the precondition, and wait for their answer, so a
// bad argument is reported as an error instead of being read out of range.
#include <climits>

#include "debug_checks.h"

namespace ssd {

namespace {

__device__ int g_first_bad;  // lowest offending token index, INT_MAX if none

__global__ void reset_first_bad_kernel() { g_first_bad = INT_MAX; }

// seq_idx must be non-decreasing with values in [0, num_seqs).
__global__ void seq_idx_check_kernel(const int32_t *seq, int L, int num_seqs) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= L) return;
  const int v = seq[t];
  const bool bad = v < 0 || v >= num_seqs || (t > 0 && seq[t - 1] > v);
  if (bad) atomicMin(&g_first_bad, t);
}

}  // namespace

hipError_t check_seq_idx(const int32_t *seq, int L, int num_seqs, hipStream_t stream, int *first_bad) {
  *first_bad = INT_MAX;
  if (L <= 0) return hipSuccess;
  hipLaunchKernelGGL(reset_first_bad_kernel, dim3(1), dim3(1), 0, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seq_idx_check_kernel, dim3((L + 255) / 256), dim3(256), 0, stream, seq, L, num_seqs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(first_bad, HIP_SYMBOL(g_first_bad), sizeof(int), 0, hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace ssd
