// Internal launch interface between the C ABI layer (api.hip) and the kernels.
// Every launcher assumes the arguments were validated by api.hip and only
// enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kHeadDim = 64;     // P
constexpr int kDState = 128;     // N
constexpr int kChunk = 128;      // Q
constexpr int kConvWidth = 4;    // K
constexpr int kNumCU = 256;      // MI355X compute units (8 XCDs x 32)
constexpr int kNumXCD = 8;

struct ConvParams {
  int bf16;                       // 1: bf16 storage, 0: fp32
  int batch, L, CH;
  const void *x; int64_t x_sb, x_st;
  void *out; int64_t o_sb, o_st;
  const float *w, *bias;
  const int32_t *seq_idx; int num_seqs;
  const void *state_in; void *state_out;
};
hipError_t launch_conv1d_silu(const ConvParams &p, hipStream_t stream);

struct DecodeParams {
  int bf16;
  int batch, H, G;
  const void *xBC; int64_t xBC_sb;
  const void *dt; int64_t dt_sb;
  const float *dt_bias, *A, *D, *conv_w, *conv_b;
  void *conv_state;
  float *ssm_state;
  void *y; int64_t y_sb;
};
hipError_t launch_decode_step(const DecodeParams &p, hipStream_t stream);

// Work decomposition of one chunk-scan call.  A work item is one segment of
// one sequence; each (item, head) pair is one workgroup.
struct ScanPlan {
  int packed;           // sequences from seq_idx (batch == 1)
  int rows;             // batch rows or num_seqs
  int seg_len;          // tokens per segment (multiple of kChunk)
  int nseg;             // batch mode: segments per row
  int items;            // batch mode: exact count; packed: upper bound
  int segmented;        // segments may need an entry state from the pre-pass
  size_t ws_plan_off, ws_local_off, ws_entry_off, ws_decay_off, ws_bytes;
};

struct ScanParams {
  int bf16;
  int batch, L, H, G;
  const void *x; int64_t x_sb, x_st;
  const void *B; int64_t B_sb, B_st;
  const void *C; int64_t C_sb, C_st;
  const void *dt; int64_t dt_sb, dt_st;
  const float *dt_bias, *A, *D;
  const int32_t *seq_idx; int num_seqs;
  const float *init; float *final_state;
  void *y; int64_t y_sb, y_st;
};

// Host arithmetic only.
ScanPlan make_scan_plan(const ScanParams &p, int seg_chunks);
hipError_t launch_chunk_scan(const ScanParams &p, const ScanPlan &plan, void *workspace,
                             hipStream_t stream);

}  // namespace ssd
