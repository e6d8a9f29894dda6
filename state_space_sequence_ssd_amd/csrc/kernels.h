// Internal launch interface between the C ABI layer (api.hip) and the kernels.
// Every launcher assumes the arguments were validated by api.hip and only
// enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// hipFuncSetAttribute(MaxDynamicSharedMemorySize) once per (device, kernel)
// and size, not on every launch: a launch stays a plain stream operation
// (nothing else on the host), which also keeps it capturable in a graph.
hipError_t set_max_dynamic_lds(const void *fn, size_t bytes);

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
  int64_t s_st;  // elements per conv-state row (the state's full channel count)
};
hipError_t launch_conv1d_silu(const ConvParams &p, hipStream_t stream);
// the conv-state export alone (state_out from the last inputs of each sequence)
hipError_t launch_conv_state_out(const ConvParams &p, hipStream_t stream);

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

struct MimoParams {
  int bf16;
  int batch, H, G, R, trapezoid;
  const void *x; int64_t x_sb;
  const void *B; int64_t B_sb;
  const void *C; int64_t C_sb;
  const void *dt; int64_t dt_sb;
  const void *lam; int64_t lam_sb;
  const float *dt_bias, *A, *D;
  float *ssm_state;
  void *prev_x, *prev_B;
  void *y; int64_t y_sb;
};
size_t mimo_lds_bytes(int hpg, int R, bool trapezoid);
hipError_t launch_decode_mimo(const MimoParams &p, hipStream_t stream);

struct BwdParams {
  int bf16;
  int batch, L, H, G, nchunks;
  const void *x, *dt, *B, *C, *dy;      // contiguous (batch, L, H, P) / (batch, L, H) / (batch, L, G, N)
  const float *dt_bias, *A, *D, *init, *dfinal;
  void *dx, *ddt, *dB, *dC;
  float *ddt_bias, *dA, *dD, *dinit;
  float *ws_states, *ws_dB, *ws_dC, *ws_scalars;
};
struct BwdLayout {
  int nchunks;
  size_t states_off, dB_off, dC_off, scalars_off, bytes;
};
BwdLayout bwd_layout(int batch, int L, int H, int G);
size_t bwd_lds_bytes();
hipError_t launch_chunk_scan_bwd(const BwdParams &p, hipStream_t stream);

struct NormParams {
  int bf16;
  int batch, L, CH, gs, before;
  float eps;
  const void *y; int64_t y_sb, y_st;
  const void *z; int64_t z_sb, z_st;
  const float *w;
  void *out; int64_t o_sb, o_st;
};
hipError_t launch_gated_rmsnorm(const NormParams &p, hipStream_t stream);

// Work decomposition of one chunk-scan call.  A work item is one segment of
// one sequence; each (item, head) pair is one workgroup.
struct ScanPlan {
  int packed;           // sequences from seq_idx (batch == 1)
  int rows;             // batch rows or num_seqs
  int seg_len;          // tokens per segment (multiple of kChunk)
  int nseg;             // batch mode: segments per row
  int items;            // batch mode: exact count; packed: upper bound
  int segmented;        // segments may need an entry state from the pre-pass
  int quad;             // fp32 short batch rows: one quadratic-form launch, no workspace
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
  // bf16 chunk kernel only: x is the raw conv input of the x channels (head h
  // at columns h * headdim), and the kernel applies conv1d(4) + SiLU to it on
  // the way into its x tile.  conv_w / conv_b: the conv's taps and bias with
  // the x channels first (row h * headdim + p); conv_state: (rows, 3, conv_ch)
  // inputs before each sequence (x channels at column 0), or null (zeros).
  int xconv;
  const float *conv_w, *conv_b;
  const void *conv_state; int64_t conv_ch;
};

// y (M, N) = x (M, K) . w (N, K)^T in bf16 with fp32 accumulation (linear_bf16.hip).
struct LinearParams {
  int M, N, K;
  const void *x; int64_t x_st;  // row strides in elements
  const void *w; int64_t w_st;
  void *y; int64_t y_st;
};
hipError_t launch_linear_bf16(const LinearParams &p, hipStream_t stream);

// fp32 batch-row sequences up to this length run as one masked quadratic form
// (quad_scan_f32.hip) instead of the chunked kernels.
constexpr int kQuadMaxL = 1024;
hipError_t launch_quad_scan_f32(const ScanParams &p, hipStream_t stream);

// Host arithmetic only.
ScanPlan make_scan_plan(const ScanParams &p, int seg_chunks);
hipError_t launch_chunk_scan(const ScanParams &p, const ScanPlan &plan, void *workspace,
                             hipStream_t stream);

}  // namespace ssd
