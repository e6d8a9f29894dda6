// C ABI of libssd.so (declared in include/ssd.h): argument validation,
// error reporting and dispatch to the gfx950 kernels.  Every check here is
// host arithmetic on the argument struct and runs before any HIP call.
#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>

#include "debug_checks.h"
#include "kernels.h"
#include "ssd.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return SSD_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dtype_size(int dt) { return dt == SSD_DTYPE_BF16 ? 2 : 4; }

// 16-byte vector access to rows of `tensor` needs a 16-byte aligned base and
// row strides that keep every row 16-byte aligned.
bool vec_ok(const void *p, int64_t s0, int64_t s1, int esize) {
  const int64_t per = 16 / esize;
  return aligned16(p) && s0 % per == 0 && s1 % per == 0;
}

// SSD_DEBUG=1: device checks of seq_idx before the kernels that index by it
// (a synchronising call; off by default, when nothing is checked on the device).
bool debug_checks() {
  const char *e = std::getenv("SSD_DEBUG");
  return e && e[0] == '1' && e[1] == 0;
}

int debug_check_seq_idx(const char *fn, const int32_t *seq, int L, int num_seqs, void *stream) {
  if (!seq || L <= 0 || !debug_checks()) return SSD_OK;
  int bad = INT_MAX;
  const hipError_t e = ssd::check_seq_idx(seq, L, num_seqs, reinterpret_cast<hipStream_t>(stream), &bad);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "%s: seq_idx check: %s", fn, hipGetErrorString(e));
  if (bad != INT_MAX)
    return fail(SSD_ERR_INVALID_ARG, "%s: seq_idx[%d] is outside [0, %d) or below its predecessor (SSD_DEBUG check)",
                fn, bad, num_seqs);
  return SSD_OK;
}

// ---------------------------------------------------------------------------
int check_scan(const ssd_scan_args *a, ssd::ScanParams &p) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: args is NULL");
  if (a->struct_size != sizeof(ssd_scan_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: struct_size %u != %zu", a->struct_size,
                sizeof(ssd_scan_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_chunk_scan_fwd: dtype %d not supported", a->dtype);
  if (a->batch < 1 || a->seqlen < 0 || a->nheads < 1 || a->ngroups < 1)
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: non-positive dims (batch %d seqlen %d nheads %d ngroups %d)",
                a->batch, a->seqlen, a->nheads, a->ngroups);
  if (a->nheads % a->ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: nheads %d not a multiple of ngroups %d", a->nheads,
                a->ngroups);
  // the model's chunk length does not change the result (the chunked form is
  // exact for any block length); the kernels always work in 128-token tiles
  if (a->headdim != ssd::kHeadDim || a->dstate != ssd::kDState ||
      (a->chunk_size != 64 && a->chunk_size != 128 && a->chunk_size != 256))
    return fail(SSD_ERR_UNSUPPORTED,
                "ssd_chunk_scan_fwd: built for headdim 64, dstate 128, chunk 64/128/256 (got %d, %d, %d)", a->headdim,
                a->dstate, a->chunk_size);
  if (a->seg_chunks < 0) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: seg_chunks < 0");
  if (!a->A) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: A is NULL");
  if (a->seqlen > 0 && (!a->x || !a->B || !a->C || !a->dt || !a->y))
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: x, B, C, dt and y are required");
  if (a->seq_idx) {
    if (a->batch != 1) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: seq_idx needs batch == 1");
    if (a->num_seqs < 1) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: num_seqs < 1 with seq_idx");
  }
  const int es = dtype_size(a->dtype);
  if (a->seqlen > 0) {
    if (!vec_ok(a->x, a->x_stride_batch, a->x_stride_token, es) || !vec_ok(a->B, a->B_stride_batch, a->B_stride_token, es) ||
        !vec_ok(a->C, a->C_stride_batch, a->C_stride_token, es) || !vec_ok(a->y, a->y_stride_batch, a->y_stride_token, es))
      return fail(SSD_ERR_MISALIGNED,
                  "ssd_chunk_scan_fwd: x, B, C, y need 16-byte aligned bases and strides that are multiples of %d elements",
                  16 / es);
    const int64_t xw = (int64_t)a->nheads * a->headdim, bw = (int64_t)a->ngroups * a->dstate;
    if (a->x_stride_token < xw || a->y_stride_token < xw || a->B_stride_token < bw || a->C_stride_token < bw ||
        a->dt_stride_token < a->nheads)
      return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: token strides smaller than the packed row width");
    // the kernels address one chunk's rows with 32-bit byte offsets
    const int64_t kMaxSt = int64_t(1) << 22;
    if (a->x_stride_token >= kMaxSt || a->y_stride_token >= kMaxSt || a->B_stride_token >= kMaxSt ||
        a->C_stride_token >= kMaxSt || a->dt_stride_token >= kMaxSt)
      return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_fwd: token strides must be below 2^22 elements");
  }
  if ((a->initial_state && !aligned16(a->initial_state)) || (a->final_state && !aligned16(a->final_state)))
    return fail(SSD_ERR_MISALIGNED, "ssd_chunk_scan_fwd: states must be 16-byte aligned");
  p = ssd::ScanParams{};
  p.bf16 = a->dtype == SSD_DTYPE_BF16;
  p.batch = a->batch; p.L = a->seqlen; p.H = a->nheads; p.G = a->ngroups;
  p.x = a->x; p.x_sb = a->x_stride_batch; p.x_st = a->x_stride_token;
  p.B = a->B; p.B_sb = a->B_stride_batch; p.B_st = a->B_stride_token;
  p.C = a->C; p.C_sb = a->C_stride_batch; p.C_st = a->C_stride_token;
  p.dt = a->dt; p.dt_sb = a->dt_stride_batch; p.dt_st = a->dt_stride_token;
  p.dt_bias = a->dt_bias; p.A = a->A; p.D = a->D;
  p.seq_idx = a->seq_idx; p.num_seqs = a->seq_idx ? a->num_seqs : a->batch;
  p.init = a->initial_state; p.final_state = a->final_state;
  p.y = a->y; p.y_sb = a->y_stride_batch; p.y_st = a->y_stride_token;
  return SSD_OK;
}

}  // namespace

extern "C" {

const char *ssd_last_error(void) { return g_err; }

int ssd_version(void) { return SSD_VERSION; }

int ssd_conv1d_silu(const ssd_conv_args *a, void *stream) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: args is NULL");
  if (a->struct_size != sizeof(ssd_conv_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: struct_size %u != %zu", a->struct_size, sizeof(ssd_conv_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_conv1d_silu: dtype %d not supported", a->dtype);
  if (a->batch < 1 || a->seqlen < 0 || a->channels < 1)
    return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: non-positive dims (batch %d seqlen %d channels %d)", a->batch,
                a->seqlen, a->channels);
  if (a->width != ssd::kConvWidth)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_conv1d_silu: built for width 4 (got %d)", a->width);
  if (a->channels % 8 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_conv1d_silu: channels %d not a multiple of 8", a->channels);
  if (!a->weight) return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: weight is NULL");
  if (a->seqlen > 0 && (!a->x || !a->out)) return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: x and out are required");
  if (a->seq_idx) {
    if (a->batch != 1) return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: seq_idx needs batch == 1");
    if (a->num_seqs < 1) return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: num_seqs < 1 with seq_idx");
  }
  const int es = dtype_size(a->dtype);
  if (a->seqlen > 0) {
    if (!vec_ok(a->x, a->x_stride_batch, a->x_stride_token, es) || !vec_ok(a->out, a->out_stride_batch, a->out_stride_token, es))
      return fail(SSD_ERR_MISALIGNED, "ssd_conv1d_silu: x/out need 16-byte aligned bases and strides multiple of %d",
                  16 / es);
    if (a->x_stride_token < a->channels || a->out_stride_token < a->channels)
      return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: token stride smaller than channels");
  }
  if (!aligned16(a->weight) || (a->conv_state_in && !aligned16(a->conv_state_in)) ||
      (a->conv_state_out && !aligned16(a->conv_state_out)))
    return fail(SSD_ERR_MISALIGNED, "ssd_conv1d_silu: weight and conv states must be 16-byte aligned");
  if (a->conv_state_out && a->seqlen > 0 && !a->x)
    return fail(SSD_ERR_INVALID_ARG, "ssd_conv1d_silu: conv_state_out needs x");
  ssd::ConvParams p{};
  p.bf16 = a->dtype == SSD_DTYPE_BF16;
  p.batch = a->batch; p.L = a->seqlen; p.CH = a->channels;
  p.x = a->x; p.x_sb = a->x_stride_batch; p.x_st = a->x_stride_token;
  p.out = a->out; p.o_sb = a->out_stride_batch; p.o_st = a->out_stride_token;
  p.w = a->weight; p.bias = a->bias;
  p.seq_idx = a->seq_idx; p.num_seqs = a->num_seqs;
  p.state_in = a->conv_state_in; p.state_out = a->conv_state_out;
  const int drc = debug_check_seq_idx("ssd_conv1d_silu", a->seq_idx, a->seqlen, a->num_seqs, stream);
  if (drc != SSD_OK) return drc;
  const hipError_t e = ssd::launch_conv1d_silu(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_conv1d_silu: %s", hipGetErrorString(e));
  return ok();
}

size_t ssd_chunk_scan_workspace_size(const ssd_scan_args *a) {
  ssd::ScanParams p;
  if (check_scan(a, p) != SSD_OK) return (size_t)-1;
  return ssd::make_scan_plan(p, a->seg_chunks).ws_bytes;
}

int ssd_chunk_scan_fwd(const ssd_scan_args *a, void *workspace, size_t ws_bytes, void *stream) {
  ssd::ScanParams p;
  const int rc = check_scan(a, p);
  if (rc != SSD_OK) return rc;
  const ssd::ScanPlan plan = ssd::make_scan_plan(p, a->seg_chunks);
  if (ws_bytes < plan.ws_bytes || (plan.ws_bytes > 0 && !workspace))
    return fail(SSD_ERR_WORKSPACE_TOO_SMALL, "ssd_chunk_scan_fwd: workspace needs %zu bytes, got %zu", plan.ws_bytes,
                ws_bytes);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(SSD_ERR_MISALIGNED, "ssd_chunk_scan_fwd: workspace must be 256-byte aligned");
  const int drc = debug_check_seq_idx("ssd_chunk_scan_fwd", a->seq_idx, a->seqlen, a->num_seqs, stream);
  if (drc != SSD_OK) return drc;
  const hipError_t e = ssd::launch_chunk_scan(p, plan, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_chunk_scan_fwd: %s", hipGetErrorString(e));
  return ok();
}

int ssd_decode_step(const ssd_decode_args *a, void *stream) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: args is NULL");
  if (a->struct_size != sizeof(ssd_decode_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: struct_size %u != %zu", a->struct_size, sizeof(ssd_decode_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step: dtype %d not supported", a->dtype);
  if (a->batch < 1 || a->nheads < 1 || a->ngroups < 1)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: non-positive dims");
  if (a->nheads % a->ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: nheads %d not a multiple of ngroups %d", a->nheads, a->ngroups);
  if (a->headdim != ssd::kHeadDim || a->dstate != ssd::kDState)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step: built for headdim 64, dstate 128 (got %d, %d)", a->headdim,
                a->dstate);
  if (a->conv_state && a->conv_width != ssd::kConvWidth)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step: built for conv_width 4 (got %d)", a->conv_width);
  if (!a->xBC || !a->dt || !a->A || !a->ssm_state || !a->y)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: xBC, dt, A, ssm_state and y are required");
  if (a->conv_state && !a->conv_weight)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: conv_state needs conv_weight");
  const int hpg = a->nheads / a->ngroups;
  if (2 * (int64_t)hpg * a->headdim + 2 * a->dstate + 2 * hpg > 32768)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step: nheads / ngroups = %d too large for one workgroup", hpg);
  if (!aligned16(a->ssm_state) || (a->conv_weight && !aligned16(a->conv_weight)))
    return fail(SSD_ERR_MISALIGNED, "ssd_decode_step: ssm_state and conv_weight must be 16-byte aligned");
  const int64_t conv_dim = (int64_t)a->nheads * a->headdim + 2 * (int64_t)a->ngroups * a->dstate;
  if (a->xBC_stride_batch < conv_dim || a->dt_stride_batch < a->nheads ||
      a->y_stride_batch < (int64_t)a->nheads * a->headdim)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step: batch strides smaller than the row width");
  ssd::DecodeParams p{};
  p.bf16 = a->dtype == SSD_DTYPE_BF16;
  p.batch = a->batch; p.H = a->nheads; p.G = a->ngroups;
  p.xBC = a->xBC; p.xBC_sb = a->xBC_stride_batch;
  p.dt = a->dt; p.dt_sb = a->dt_stride_batch;
  p.dt_bias = a->dt_bias; p.A = a->A; p.D = a->D;
  p.conv_w = a->conv_weight; p.conv_b = a->conv_bias;
  p.conv_state = a->conv_state; p.ssm_state = a->ssm_state;
  p.y = a->y; p.y_sb = a->y_stride_batch;
  const hipError_t e = ssd::launch_decode_step(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_decode_step: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
