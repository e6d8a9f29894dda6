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
 *     device memory and never synchronises; its only device state is the
 *     workspace array of ssd_chunk_scan_fwd_noalloc, reserved with the code
 *     object (below).
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
 * Passage: the Mamba-2 block's short causal convolution of kernel 4 with SiLU
 * on the x|B|C channels ("Nemotron-H style Hybrid Mamba-Transformer 3B
 * feasibility study", sec. 1.4 "Mamba-2 configuration"), applied before the
 * scan ("Nemotron-Mamba3 architecture" article, sec. 2.2).
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
 * Passages: the recurrence with a scalar-times-identity transition per head
 * ("Mamba-3: an inference-first state space model", the paragraph on
 * Mamba-2's simplified transition); its block (chunked) evaluation as a
 * masked matrix product, the state space duality ("AI Engineering EP6",
 * sec. 8 and 10); chunk 128 and n_groups 8 (feasibility study sec. 1.4);
 * states carried between calls for resumable, chunked prefill ("Bamba-9B"
 * summary, inference-efficiency section).
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
 * ssd_conv_scan_fwd -- the conv1d(4) + SiLU and the chunked scan of one
 * Mamba-2 mixer in one call: the short convolution fused into the scan's
 * prologue.
 *
 * Passages: Conv1D and the SSM merged into one operator to save kernel
 * launches and memory round trips ("Nemotron-Mamba3 architecture" article,
 * sec. 4.3, deployment notes on operator fusion); the conv and the scan
 * themselves as for ssd_conv1d_silu and ssd_chunk_scan_fwd above.
 *
 * The result is exactly that of ssd_conv1d_silu on xBC followed by
 * ssd_chunk_scan_fwd on the x | B | C column views of its output (and, for
 * bf16, bit for bit: the fused kernel repeats the conv's fp32 arithmetic in
 * the same order and rounds to bf16 where the conv would have stored it).
 * The post-conv x is never written to memory: the bf16 scan computes it
 * while loading its x tiles; the B and C channels (shared by the heads of a
 * group) are convolved once into the workspace.  fp32 runs the two steps
 * through the workspace.
 *
 *   xBC (batch, seqlen, conv_dim), conv_dim = nheads*headdim + 2*ngroups*dstate:
 *       the raw conv input, columns x | B | C (the in_proj output's slice);
 *       16-byte aligned, strides multiples of 8 elements.
 *   conv_weight (conv_dim, conv_width) fp32, required; conv_bias (conv_dim)
 *       fp32 or NULL.  conv_width must be 4.
 *   conv_state_in / conv_state_out (rows, conv_width-1, conv_dim) or NULL:
 *       as for ssd_conv1d_silu (conv_state_out is written after every read
 *       of conv_state_in, so the two may be the same buffer).
 *   dt, dt_bias, A, D, seq_idx, num_seqs, initial_state, final_state, y,
 *   chunk_size, seg_chunks: as for ssd_chunk_scan_fwd.
 *
 * The workspace (ssd_conv_scan_workspace_size() bytes, 256-byte aligned,
 * contents on entry irrelevant) holds the conv output of the B and C
 * channels (bf16; all channels for fp32) and the scan's own workspace.
 * Errors: as for the two calls it replaces (SSD_ERR_INVALID_ARG,
 * SSD_ERR_UNSUPPORTED, SSD_ERR_MISALIGNED, SSD_ERR_WORKSPACE_TOO_SMALL,
 * SSD_ERR_HIP), reported before any kernel is launched except SSD_ERR_HIP.
 * ---------------------------------------------------------------------- */
typedef struct ssd_conv_scan_args {
  uint32_t struct_size;          /* sizeof(ssd_conv_scan_args) */
  int32_t dtype;                 /* ssd_dtype of xBC, dt, y, conv states */
  int32_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size;
  int32_t seg_chunks;            /* 0 = automatic */
  int32_t conv_width;            /* 4 */
  const void *xBC; int64_t xBC_stride_batch, xBC_stride_token;
  const float *conv_weight;      /* (conv_dim, conv_width), required */
  const float *conv_bias;        /* (conv_dim) or NULL */
  const void *dt; int64_t dt_stride_batch, dt_stride_token;
  const float *dt_bias;          /* (nheads) or NULL */
  const float *A;                /* (nheads), required */
  const float *D;                /* (nheads) or NULL */
  const int32_t *seq_idx;        /* (seqlen) or NULL */
  int32_t num_seqs;
  const void *conv_state_in;     /* (rows, conv_width-1, conv_dim) or NULL */
  void *conv_state_out;          /* (rows, conv_width-1, conv_dim) or NULL */
  const float *initial_state;    /* (rows, nheads, headdim, dstate) or NULL */
  float *final_state;            /* (rows, nheads, headdim, dstate) or NULL */
  void *y;        int64_t y_stride_batch, y_stride_token;
} ssd_conv_scan_args;

/* Workspace bytes ssd_conv_scan_fwd needs (host arithmetic; (size_t)-1 if
 * args are invalid). */
size_t ssd_conv_scan_workspace_size(const ssd_conv_scan_args *args);

int ssd_conv_scan_fwd(const ssd_conv_scan_args *args, void *workspace,
                      size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * ssd_linear -- the mixer's linear projections: y = x w^T.
 *
 * Passages: in_proj takes each token's d_model features to the conv input
 * x|B|C, the gate z and dt; out_proj takes the gated, normalised y back to
 * d_model ("Nemotron-H style Hybrid Mamba-Transformer 3B feasibility
 * study", the Mamba-2 block's projection parameters; "Nemotron-Mamba3
 * architecture" article, sec. 2.2, the layer's projections around the conv
 * and the scan).
 *
 *   y[m][n] = sum_k x[m][k] * w[n][k]
 *   x (M, K), w (N, K) -- a torch Linear weight, (out, in) --, y (M, N);
 *   row-major with the given row strides (elements); x, w, y must not
 *   overlap.
 *
 * Precision: bf16 x, w, y; products and sums in fp32 (bf16 matrix cores),
 * one bf16 rounding of each output.
 * Supported: dtype BF16; K a positive multiple of 64; 16-byte aligned bases and row
 * strides multiples of 8 elements (below 2^22); N a multiple of 8.
 * Errors: SSD_ERR_INVALID_ARG (NULL pointer, negative dims, a row stride
 * below its row width), SSD_ERR_UNSUPPORTED (dtype, K), SSD_ERR_MISALIGNED,
 * SSD_ERR_HIP -- all but the last before any HIP call.
 * ---------------------------------------------------------------------- */
typedef struct ssd_linear_args {
  uint32_t struct_size;          /* sizeof(ssd_linear_args) */
  int32_t dtype;                 /* SSD_DTYPE_BF16 */
  int32_t M, N, K;
  const void *x; int64_t x_stride;
  const void *w; int64_t w_stride;
  void *y;       int64_t y_stride;
} ssd_linear_args;

int ssd_linear(const ssd_linear_args *args, void *stream);

/* ------------------------------------------------------------------------
 * ssd_chunk_scan_fwd_noalloc -- ssd_chunk_scan_fwd without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, kernels and results as ssd_chunk_scan_fwd.  The workspace
 * is a library-owned device array of SSD_NOALLOC_SCRATCH_BYTES (96 MiB) per
 * GPU, reserved when the library's code object is loaded on that GPU and
 * held until the process ends; its address is looked up on the calling
 * thread's current device (which must be the stream's device) on the first
 * call there.  The call allocates nothing.  That is enough for every
 * automatic segmentation (seg_chunks = 0 needs at most 1,533 (segment, head)
 * pairs of two 32 KiB states, 95.9 MiB, at 511 heads in one packed
 * sequence); a call that needs more (an explicit seg_chunks) returns
 * SSD_ERR_WORKSPACE_TOO_SMALL before any HIP call.
 *
 * All calls on one GPU share its array, and it keeps the last call's
 * contents (nothing in it needs to start at zero).  Calls that overlap on one
 * GPU -- on different streams, or from different host threads without
 * ordering between them -- race on it; serialise them (one stream, or events).
 * ---------------------------------------------------------------------- */
#define SSD_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)

int ssd_chunk_scan_fwd_noalloc(const ssd_scan_args *args, void *stream);

/* ------------------------------------------------------------------------
 * ssd_decode_step -- one token of the recurrence for every batch row,
 * updating the states in place.
 *
 * Passage: decoding applies the same recurrence one token at a time to a
 * fixed-size state, which makes it memory-bound ("Mamba-3" blog, the
 * paragraph on why the simplified transition ties decoding to memory
 * traffic; "Bamba-9B" summary, inference-efficiency section).
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
 * ssm_state 16-byte aligned; nheads / ngroups at most 250 (one workgroup
 * holds a group's conv outputs and y in 128 KiB of LDS:
 * 130 * (nheads / ngroups) + 256 floats), SSD_ERR_UNSUPPORTED beyond.
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

/* ------------------------------------------------------------------------
 * ssd_chunk_scan_bwd -- backward pass of the scan: the gradients of every
 * input for a loss L with dL/dy = dy (and dL/dfinal_state = d_final_state).
 *
 * Passage: the training workload of the layer needs its backward pass
 * ("Nemotron-H style Hybrid Mamba-Transformer 3B feasibility study", sec. 3.1,
 * forward/backward verification of the layer; sec. 7, Phase 2).
 *
 * Forward (as ssd_chunk_scan_fwd, batch rows only): dt_t = softplus(z_t),
 * z_t = dt[t] + dt_bias, a_t = exp(dt_t A), S_t = a_t S_{t-1} + dt_t x_t B_t^T,
 * y_t = S_t C_t + D x_t, S_{-1} = initial_state (or 0).  Outputs:
 *   dx (batch, seqlen, nheads, headdim), ddt = dL/d(dt raw) (batch, seqlen,
 *   nheads), dB, dC (batch, seqlen, ngroups, dstate): the dtype of x;
 *   d_dt_bias, dA, dD (nheads) fp32; d_initial_state (batch, nheads, headdim,
 *   dstate) fp32 or NULL.  Every output is overwritten.
 * Inputs x, dt, B, C, dy are contiguous in the layouts above (dy like x).
 * Arithmetic is fp32 (bf16 inputs widened), in chunks of 32 tokens.
 *
 * The workspace (ssd_chunk_scan_bwd_workspace_size bytes, 256-byte aligned)
 * holds the state entering every chunk and per-head partial sums: about
 * batch x nheads x (seqlen / 32 x 32 KiB + seqlen x 1 KiB).  With BF16
 * inputs the stored chunk states are rounded to bf16 (the forward pass's
 * own precision for the state in its state->output product) and use half
 * of their region; with F32 inputs they stay fp32.
 *
 * Supported: headdim 64, dstate 128, dtype F32 or BF16, batch rows (no
 * seq_idx); x, B, C, dy, dt and the states 16-byte aligned.
 * ---------------------------------------------------------------------- */
typedef struct ssd_scan_bwd_args {
  uint32_t struct_size;          /* sizeof(ssd_scan_bwd_args) */
  int32_t dtype;                 /* ssd_dtype of x, dt, B, C, dy and of dx, ddt, dB, dC */
  int32_t batch, seqlen, nheads, headdim, dstate, ngroups;
  const void *x, *dt, *B, *C, *dy;
  const float *dt_bias;          /* (nheads) or NULL */
  const float *A;                /* (nheads), required */
  const float *D;                /* (nheads) or NULL */
  const float *initial_state;    /* (batch, nheads, headdim, dstate) or NULL */
  const float *d_final_state;    /* (batch, nheads, headdim, dstate) or NULL (= 0) */
  void *dx, *ddt, *dB, *dC;
  float *d_dt_bias;              /* (nheads) or NULL (not written) */
  float *dA;                     /* (nheads), required */
  float *dD;                     /* (nheads) or NULL (not written) */
  float *d_initial_state;        /* (batch, nheads, headdim, dstate) or NULL */
} ssd_scan_bwd_args;

size_t ssd_chunk_scan_bwd_workspace_size(const ssd_scan_bwd_args *args);

int ssd_chunk_scan_bwd(const ssd_scan_bwd_args *args, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * ssd_gated_rmsnorm -- the gated RMSNorm that follows the scan in the
 * Mamba-2 mixer.
 *
 * Passage: Mamba-2 keeps an RMSNorm together with the output gate; the norm
 * may sit before or after the gate and be taken per group of channels or
 * over the whole width ("Mamba-3: an inference-first state space model",
 * the normalization paragraph and the later remark on the norm's placement
 * and grouped or plain type).
 *
 * Per token row and per group of group_size consecutive channels, with
 * SiLU(u) = u / (1 + e^-u) and rms(v) = sqrt(mean over the group of v^2 + eps):
 *   norm_before_gate = 0:  g = y * SiLU(z);  out = g / rms(g) * weight
 *   norm_before_gate = 1:  out = y / rms(y) * weight * SiLU(z)
 * z may be NULL (no gate).  Arithmetic in fp32; out rounded to the dtype.
 *
 *   y, z, out (batch, seqlen, channels), unit channel stride, strides in
 *   elements for batch and token (z may be a view into the in-projection
 *   output); weight (channels) fp32 contiguous, required.
 *
 * Supported: dtype F32 or BF16; channels a multiple of group_size;
 * group_size a multiple of 8 (bf16) or 4 (fp32) and at most 8192 (bf16) or
 * 4096 (fp32); y, z, out
 * and weight 16-byte aligned, strides multiples of the 16-byte vector;
 * eps finite and >= 0.  out must not overlap y or z.
 * ---------------------------------------------------------------------- */
typedef struct ssd_norm_args {
  uint32_t struct_size;          /* sizeof(ssd_norm_args) */
  int32_t dtype;                 /* ssd_dtype of y, z, out */
  int32_t batch, seqlen, channels, group_size, norm_before_gate;
  float eps;
  const void *y;  int64_t y_stride_batch, y_stride_token;
  const void *z;  int64_t z_stride_batch, z_stride_token;   /* NULL = no gate */
  const float *weight;
  void *out;      int64_t out_stride_batch, out_stride_token;
} ssd_norm_args;

int ssd_gated_rmsnorm(const ssd_norm_args *args, void *stream);

/* ------------------------------------------------------------------------
 * ssd_decode_step_mimo -- one decode token of the multi-input multi-output
 * (MIMO) SSM, optionally with an exponential-trapezoidal input term.
 *
 * Passage: "Mamba-3: an inference-first state space model" lists the changes
 * to Mamba-2: a more general recurrence from an exponential-trapezoidal
 * discretization, and MIMO instead of SISO, whose projection widens B and C
 * to rank R and adds parallel work to each update at almost no extra decode
 * latency.  The page states no formulas; this is the plainest reading, which
 * is the Mamba-2 decode step at R = 1 with the Euler form.  Per head h
 * (group g = h / (nheads / ngroups)), dt = softplus(dt_raw + dt_bias[h]),
 * a = exp(dt * A[h]), state S (headdim x dstate):
 *   trapezoid = 0:  S <- a S + dt X B^T
 *   trapezoid = 1:  S <- a S + (1 - lam) dt a Xp Bp^T + lam dt X B^T
 *   Y = S C + D[h] X
 * X (headdim x rank) is the head's input, B and C (dstate x rank) the
 * group's; Xp and Bp are the previous token's X and B, held in prev_x and
 * prev_B and replaced by X and B after the step.  lam per (row, head), NULL
 * = 1/2 (the trapezoid rule); lam = 1 gives the Euler form.
 *
 *   x, y     (batch, nheads, headdim, rank), batch strides in elements
 *   B, C     (batch, ngroups, dstate, rank), batch strides in elements
 *   dt, lam  (batch, nheads) raw, batch strides; dt_bias, A, D (nheads) fp32
 *   ssm_state (batch, nheads, headdim, dstate) fp32 contiguous, in/out
 *   prev_x (batch, nheads, headdim, rank), prev_B (batch, ngroups, dstate,
 *   rank): contiguous, dtype of x, in/out; required when trapezoid != 0.
 * No conv: the MIMO form drops the short convolution (the same page), so x,
 * B and C are the projections' outputs.  Inputs must not alias outputs.
 *
 * Supported: headdim 64, dstate 128, rank 1, 2, 4 or 8, dtype F32 or BF16,
 * ssm_state 16-byte aligned; nheads / ngroups small enough that the group's
 * X, previous X and Y (and B, C, Bp) fit in 160 KiB of LDS
 * (SSD_ERR_UNSUPPORTED beyond).
 * ---------------------------------------------------------------------- */
typedef struct ssd_mimo_decode_args {
  uint32_t struct_size;          /* sizeof(ssd_mimo_decode_args) */
  int32_t dtype;                 /* ssd_dtype of x, B, C, dt, lam, y, prev_x, prev_B */
  int32_t batch, nheads, headdim, dstate, ngroups, rank, trapezoid;
  const void *x;   int64_t x_stride_batch;
  const void *B;   int64_t B_stride_batch;
  const void *C;   int64_t C_stride_batch;
  const void *dt;  int64_t dt_stride_batch;
  const void *lam; int64_t lam_stride_batch;   /* NULL = 1/2 */
  const float *dt_bias;          /* (nheads) or NULL */
  const float *A;                /* (nheads), required */
  const float *D;                /* (nheads) or NULL */
  float *ssm_state;
  void *prev_x;
  void *prev_B;
  void *y;         int64_t y_stride_batch;
} ssd_mimo_decode_args;

int ssd_decode_step_mimo(const ssd_mimo_decode_args *args, void *stream);

/* Message describing the last error on the calling thread ("" if none). */
const char *ssd_last_error(void);

/* SSD_VERSION of the built library. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
