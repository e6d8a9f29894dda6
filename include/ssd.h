/*
 * ssd.h -- C ABI of libssd.so: the Mamba-2 selective state-space (SSD)
 * layer's hot path on one AMD Instinct MI355X (gfx950).
 *
 * The layer (Mamba-2 mixer core):
 *   1. a depthwise causal conv1d of width 4 followed by SiLU on the x|B|C
 *      channels ("Nemotron-H style Hybrid Mamba-Transformer 3B feasibility
 *      study", sec. 1.4 "Mamba-2 configuration": conv_kernel 4, SiLU;
 *      "Nemotron-Mamba3 architecture" article, sec. 2.2: Conv1D before the
 *      scan);
 *   2. the selective scan, computed as a chunked SSD prefill (feasibility
 *      study sec. 1.4 / 2.6: chunk_size 128): per head h, a fixed-size state
 *      S (headdim x dstate) with a scalar-times-identity transition
 *      ("Mamba-3: an inference-first state space model", on Mamba-2's
 *      simplified transition):
 *          dt_t = softplus(dt_raw[t][h] + dt_bias[h])
 *          S_t  = exp(dt_t * A[h]) * S_{t-1} + dt_t * x_t (outer) B_t
 *          y_t  = S_t . C_t + D[h] * x_t
 *      B and C are shared by the heads of each of ngroups groups
 *      (feasibility study sec. 1.4: n_groups 8); head h reads group
 *      h / (nheads / ngroups).  dt, B and C depend on the token
 *      (selectivity: "AI Engineering EP6", sec. 6 principle 2).
 *   3. the single-token decode step, the same recurrence for one token
 *      with the conv window kept as state (decode is memory-bound:
 *      "Mamba-3" blog, same paragraph; "Bamba-9B" summary, inference
 *      efficiency section).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors) unless stated otherwise.  The caller allocates and owns every
 *     buffer, including the scan workspace.  The library never allocates
 *     device memory, never synchronises, and keeps no device state.
 *   - Strides are in ELEMENTS.  The innermost dimension of each tensor is
 *     unit-stride; the dimensions listed as "contiguous" are packed.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue
 *     kernels and return; device-side faults surface at the caller's next
 *     synchronisation.
 *   - Every argument check below is host code and runs before any HIP call,
 *     so an error return means nothing was enqueued.
 *   - Return 0 (SSD_OK) or an ssd_status code; ssd_last_error() then holds a
 *     message for the calling thread.
 *   - Input pointers of one call must not alias its output pointers (the
 *     decode step's conv_state / ssm_state are in/out by design).
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_VERSION 1

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1,       /* null required pointer, bad dims, H % G != 0 ... */
  SSD_ERR_UNSUPPORTED = 2,       /* headdim/dstate/width/chunk/dtype outside the built set */
  SSD_ERR_WORKSPACE_TOO_SMALL = 3,
  SSD_ERR_MISALIGNED = 4,        /* pointer or stride breaks the 16-byte vector access */
  SSD_ERR_HIP = 5                /* a launch failed; see ssd_last_error() */
} ssd_status;

typedef enum ssd_dtype {
  SSD_DTYPE_F32 = 0,
  SSD_DTYPE_BF16 = 1
} ssd_dtype;

/* ------------------------------------------------------------------------
 * ssd_conv1d_silu -- depthwise causal conv1d + SiLU.
 *
 *   u[t][c]   = bias[c] + sum_{k=0}^{width-1} weight[c][k] * v(t-(width-1)+k, c)
 *   out[t][c] = u[t][c] / (1 + exp(-u[t][c]))
 *
 * v(tau, c) is the input at token tau when tau lies in the same sequence as
 * t; otherwise the matching row of conv_state_in (if given), else 0.  So the
 * tap weight[c][width-1] multiplies the newest token (cross-correlation
 * order), and the left edge of every sequence is zero-padded unless a conv
 * state carries the previous inputs.
 *
 * Sequences: without seq_idx every batch row is one sequence (rows = batch).
 * With seq_idx (batch must be 1) token t belongs to sequence seq_idx[t];
 * seq_idx must be non-decreasing with values in [0, num_seqs) (rows =
 * num_seqs).  Sequences with no token are allowed.  This is a precondition:
 * by default it is not checked (a value out of range is read out of range).
 * With SSD_DEBUG=1 in the environment, ssd_conv1d_silu and
 * ssd_chunk_scan_fwd first check seq_idx on the device, wait for the
 * answer (a synchronising call) and return SSD_ERR_INVALID_ARG, naming the
 * first bad token, before any kernel reads by it.
 *
 * conv_state_in / conv_state_out: (rows, width-1, channels), contiguous,
 * same dtype as x.  Row r of a sequence's state is the input width-1-r
 * tokens before its first token.  conv_state_out receives the last width-1
 * inputs of each sequence (falling back on conv_state_in / zeros for
 * sequences shorter than width-1), ready for ssd_decode_step.
 *
 * Supported: width 4; dtype F32 or BF16; channels a multiple of 8;
 * x / out 16-byte aligned with token and batch strides multiples of 8.
 * out must not overlap x (no in-place conv).
 * ---------------------------------------------------------------------- */
typedef struct ssd_conv_args {
  uint32_t struct_size;          /* sizeof(ssd_conv_args) */
  int32_t dtype;                 /* ssd_dtype of x, out, conv states */
  int32_t batch, seqlen, channels, width;
  const void *x;  int64_t x_stride_batch, x_stride_token;      /* (batch, seqlen, channels) */
  void *out;      int64_t out_stride_batch, out_stride_token;  /* (batch, seqlen, channels) */
  const float *weight;           /* (channels, width) fp32, contiguous; required */
  const float *bias;             /* (channels) fp32 or NULL (= 0) */
  const int32_t *seq_idx;        /* (seqlen) int32 or NULL */
  int32_t num_seqs;              /* rows of the conv states when seq_idx is given */
  const void *conv_state_in;     /* (rows, width-1, channels) or NULL */
  void *conv_state_out;          /* (rows, width-1, channels) or NULL */
} ssd_conv_args;

int ssd_conv1d_silu(const ssd_conv_args *args, void *stream);

/* ------------------------------------------------------------------------
 * ssd_chunk_scan_fwd -- chunked SSD prefill of the selective scan above.
 *
 * Tensors (innermost two dims contiguous; strides for batch and token):
 *   x  (batch, seqlen, nheads, headdim)    head stride = headdim
 *   B  (batch, seqlen, ngroups, dstate)    group stride = dstate
 *   C  (batch, seqlen, ngroups, dstate)
 *   dt (batch, seqlen, nheads)             raw, before bias and softplus
 *   y  (batch, seqlen, nheads, headdim)    same dtype as x
 * so x, B and C may be views into one conv output of width
 * nheads*headdim + 2*ngroups*dstate (token stride = that width).
 *   dt_bias, A, D: (nheads) fp32; dt_bias and D may be NULL (= 0).
 *   initial_state / final_state: (rows, nheads, headdim, dstate) fp32,
 *   contiguous, state[p][n] multiplies B[n] x[p]; either may be NULL
 *   (initial = 0 / not written).  rows = batch, or num_seqs with seq_idx.
 *   seq_idx: as for ssd_conv1d_silu (batch must be 1).  Each sequence
 *   starts from its own initial_state row and ends in its final_state row;
 *   tokens of different sequences never interact.
 *
 * Precision: bf16 x/B/C/dt/y with fp32 state and accumulation (MFMA bf16
 * operands); fp32 inputs run an all-fp32 path.
 *
 * Supported: headdim 64, dstate 128, chunk_size 64, 128 or 256, dtype F32
 * or BF16.  chunk_size is the model's chunk length; the block (chunked) form
 * of the recurrence gives the same result for any chunk length, up to
 * rounding, so the kernels always work in their own tiles (128 tokens for
 * bf16, 64 for fp32).
 * x, B, C, y 16-byte aligned with strides multiples of 8 elements; token
 * strides below 2^22 elements (SSD_ERR_INVALID_ARG otherwise).
 *
 * seg_chunks: 0 = automatic (segments of whole kernel tiles, as many as
 * fill the GPU).  Otherwise each sequence is cut into segments of seg_chunks
 * 128-token tiles that run in parallel; the state entering each segment is
 * found by a short pre-pass (same result, more parallelism for few long
 * sequences).
 *
 * The workspace (device memory, at least ssd_chunk_scan_workspace_size()
 * bytes, 256-byte aligned, contents on entry irrelevant) holds the
 * per-segment states and the packed-sequence work list.  It may be NULL
 * when the size is 0.
 * ---------------------------------------------------------------------- */
typedef struct ssd_scan_args {
  uint32_t struct_size;          /* sizeof(ssd_scan_args) */
  int32_t dtype;                 /* ssd_dtype of x, B, C, dt, y */
  int32_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size;
  int32_t seg_chunks;            /* 0 = automatic */
  const void *x;  int64_t x_stride_batch, x_stride_token;
  const void *B;  int64_t B_stride_batch, B_stride_token;
  const void *C;  int64_t C_stride_batch, C_stride_token;
  const void *dt; int64_t dt_stride_batch, dt_stride_token;
  const float *dt_bias;          /* (nheads) or NULL */
  const float *A;                /* (nheads), required */
  const float *D;                /* (nheads) or NULL */
  const int32_t *seq_idx;        /* (seqlen) or NULL */
  int32_t num_seqs;
  const float *initial_state;    /* (rows, nheads, headdim, dstate) or NULL */
  float *final_state;            /* (rows, nheads, headdim, dstate) or NULL */
  void *y;        int64_t y_stride_batch, y_stride_token;
} ssd_scan_args;

/* Workspace bytes ssd_chunk_scan_fwd needs for these arguments (pure host
 * arithmetic; returns 0 for none, or (size_t)-1 if args are invalid). */
size_t ssd_chunk_scan_workspace_size(const ssd_scan_args *args);

int ssd_chunk_scan_fwd(const ssd_scan_args *args, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * ssd_decode_step -- one token of the recurrence for every batch row,
 * updating the states in place.
 *
 *   xBC (batch, conv_dim), conv_dim = nheads*headdim + 2*ngroups*dstate,
 *       channel order x (head-major), B (group-major), C (group-major).
 *       Raw (pre-conv) when conv_state != NULL, else already conv+SiLU'd.
 *   conv_state (batch, conv_width-1, conv_dim) contiguous, dtype of xBC,
 *       in/out: the window [conv_state rows, xBC] is convolved as in
 *       ssd_conv1d_silu, then conv_state becomes the window's last
 *       conv_width-1 rows (a shift by one token).
 *   conv_weight (conv_dim, conv_width) fp32, conv_bias (conv_dim) or NULL.
 *   dt (batch, nheads) raw; dt_bias, A, D (nheads) fp32 (dt_bias, D may be NULL).
 *   ssm_state (batch, nheads, headdim, dstate) fp32 contiguous, in/out.
 *   y (batch, nheads, headdim), dtype of xBC, batch stride y_stride_batch.
 *
 * Supported: headdim 64, dstate 128, conv_width 4, dtype F32 or BF16;
 * ssm_state 16-byte aligned; nheads / ngroups at most 254 (one workgroup
 * holds a group's conv outputs and y in LDS), SSD_ERR_UNSUPPORTED beyond.
 * ---------------------------------------------------------------------- */
typedef struct ssd_decode_args {
  uint32_t struct_size;          /* sizeof(ssd_decode_args) */
  int32_t dtype;                 /* ssd_dtype of xBC, dt, y, conv_state */
  int32_t batch, nheads, headdim, dstate, ngroups, conv_width;
  const void *xBC;  int64_t xBC_stride_batch;
  const void *dt;   int64_t dt_stride_batch;
  const float *dt_bias;          /* (nheads) or NULL */
  const float *A;                /* (nheads), required */
  const float *D;                /* (nheads) or NULL */
  const float *conv_weight;      /* (conv_dim, conv_width); required if conv_state */
  const float *conv_bias;        /* (conv_dim) or NULL */
  void *conv_state;              /* (batch, conv_width-1, conv_dim) in/out, or NULL */
  float *ssm_state;              /* (batch, nheads, headdim, dstate) in/out, required */
  void *y;          int64_t y_stride_batch;
} ssd_decode_args;

int ssd_decode_step(const ssd_decode_args *args, void *stream);

/* Message describing the last error on the calling thread ("" if none). */
const char *ssd_last_error(void);

/* SSD_VERSION of the built library. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
