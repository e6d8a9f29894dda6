// C ABI of libssd.so (declared in include/ssd.h): argument validation,
// error reporting and dispatch to the gfx950 kernels.  Every check here is
// host arithmetic on the argument struct and runs before any HIP call.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

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

// ---------------------------------------------------------------------------
// Library-owned scan workspace for ssd_chunk_scan_fwd_noalloc: one array per
// GPU, in device memory the code object reserves when it is loaded (each GPU
// that runs the library holds it until the process ends).  In host code the
// array's name is only a host-side stand-in; its device address on the
// current GPU comes from hipGetSymbolAddress, looked up once per device and
// kept, and only that address is ever passed to a kernel.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[SSD_NOALLOC_SCRATCH_BYTES];
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_chunk_scan_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_chunk_scan_fwd_noalloc: device %d beyond the %d this build tracks", dev,
                kMaxDevices);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(SSD_ERR_HIP, "ssd_chunk_scan_fwd_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SSD_OK;
}

}  // namespace

namespace ssd {
hipError_t set_max_dynamic_lds(const void *fn, size_t bytes) {
  static std::mutex mu;
  static constexpr int kSlots = 64;
  static struct {
    int dev;
    const void *fn;
    size_t bytes;
  } done[kSlots];
  static int n = 0;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (done[i].dev == dev && done[i].fn == fn && done[i].bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  int slot = -1;
  for (int i = 0; i < n; ++i)
    if (done[i].dev == dev && done[i].fn == fn) slot = i;
  if (slot < 0 && n < kSlots) slot = n++;
  if (slot >= 0) done[slot] = {dev, fn, bytes};
  return hipSuccess;
}
}  // namespace ssd

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
  p.s_st = a->channels;
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

int ssd_chunk_scan_fwd_noalloc(const ssd_scan_args *a, void *stream) {
  ssd::ScanParams p;
  const int rc = check_scan(a, p);
  if (rc != SSD_OK) return rc;
  // the same plan (and so the same kernels and results) as ssd_chunk_scan_fwd
  const ssd::ScanPlan plan = ssd::make_scan_plan(p, a->seg_chunks);
  if (plan.ws_bytes > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
    return fail(SSD_ERR_WORKSPACE_TOO_SMALL,
                "ssd_chunk_scan_fwd_noalloc: this call needs %zu bytes of workspace, more than the library's "
                "%zu-byte array (use ssd_chunk_scan_fwd with a caller workspace)",
                plan.ws_bytes, (size_t)SSD_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (plan.ws_bytes > 0) {
    const int src = scratch_address(&ws);
    if (src != SSD_OK) return src;
  }
  const int drc = debug_check_seq_idx("ssd_chunk_scan_fwd_noalloc", a->seq_idx, a->seqlen, a->num_seqs, stream);
  if (drc != SSD_OK) return drc;
  const hipError_t e = ssd::launch_chunk_scan(p, plan, ws, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_chunk_scan_fwd_noalloc: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// conv + scan in one call
// ---------------------------------------------------------------------------
namespace {
struct ConvScanPlan {
  ssd::ScanParams sp;
  ssd::ScanPlan plan;
  ssd::ConvParams conv;  // the conv launch (B|C channels for bf16, all for fp32)
  size_t conv_bytes, scan_off, total;
};

constexpr size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int plan_conv_scan(const ssd_conv_scan_args *a, ConvScanPlan &cp) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_conv_scan_fwd: args is NULL");
  if (a->struct_size != sizeof(ssd_conv_scan_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_conv_scan_fwd: struct_size %u != %zu", a->struct_size,
                sizeof(ssd_conv_scan_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_conv_scan_fwd: dtype %d not supported", a->dtype);
  if (a->conv_width != ssd::kConvWidth)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_conv_scan_fwd: built for conv width 4 (got %d)", a->conv_width);
  if (!a->conv_weight) return fail(SSD_ERR_INVALID_ARG, "ssd_conv_scan_fwd: conv_weight is NULL");
  if (a->seqlen > 0 && !a->xBC) return fail(SSD_ERR_INVALID_ARG, "ssd_conv_scan_fwd: xBC is required");
  if (!aligned16(a->conv_weight) || (a->conv_state_in && !aligned16(a->conv_state_in)) ||
      (a->conv_state_out && !aligned16(a->conv_state_out)))
    return fail(SSD_ERR_MISALIGNED, "ssd_conv_scan_fwd: conv_weight and conv states must be 16-byte aligned");
  // the scan's own checks, on the views it will read: x at column 0 of xBC,
  // B and C at the conv output's layout (any 256-aligned base stands in for
  // the workspace here)
  const bool bf16 = a->dtype == SSD_DTYPE_BF16;
  const int es = dtype_size(a->dtype);
  if (a->nheads < 1 || a->ngroups < 1 || a->headdim < 1 || a->dstate < 1 || a->batch < 1 || a->seqlen < 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_conv_scan_fwd: non-positive dims");
  const int64_t HP = (int64_t)a->nheads * a->headdim, GN = (int64_t)a->ngroups * a->dstate;
  const int64_t conv_dim = HP + 2 * GN;
  if (a->seqlen > 0) {
    if (!vec_ok(a->xBC, a->xBC_stride_batch, a->xBC_stride_token, es))
      return fail(SSD_ERR_MISALIGNED,
                  "ssd_conv_scan_fwd: xBC needs a 16-byte aligned base and strides multiples of %d elements", 16 / es);
    if (a->xBC_stride_token < conv_dim)
      return fail(SSD_ERR_INVALID_ARG, "ssd_conv_scan_fwd: xBC token stride %lld below conv_dim %lld",
                  (long long)a->xBC_stride_token, (long long)conv_dim);
  }
  const int64_t out_ch = bf16 ? 2 * GN : conv_dim;  // channels of the conv output in the workspace
  const int64_t L = a->seqlen;
  static const char kDummy[16] __attribute__((aligned(256))) = {};
  ssd_scan_args s{};
  s.struct_size = sizeof(ssd_scan_args);
  s.dtype = a->dtype;
  s.batch = a->batch; s.seqlen = a->seqlen; s.nheads = a->nheads; s.headdim = a->headdim;
  s.dstate = a->dstate; s.ngroups = a->ngroups; s.chunk_size = a->chunk_size; s.seg_chunks = a->seg_chunks;
  if (bf16) {
    s.x = a->xBC; s.x_stride_batch = a->xBC_stride_batch; s.x_stride_token = a->xBC_stride_token;
  } else {
    s.x = kDummy; s.x_stride_batch = L * out_ch; s.x_stride_token = out_ch;
  }
  s.B = kDummy; s.B_stride_batch = L * out_ch; s.B_stride_token = out_ch;
  s.C = kDummy; s.C_stride_batch = L * out_ch; s.C_stride_token = out_ch;
  s.dt = a->dt; s.dt_stride_batch = a->dt_stride_batch; s.dt_stride_token = a->dt_stride_token;
  s.dt_bias = a->dt_bias; s.A = a->A; s.D = a->D;
  s.seq_idx = a->seq_idx; s.num_seqs = a->num_seqs;
  s.initial_state = a->initial_state; s.final_state = a->final_state;
  s.y = a->y; s.y_stride_batch = a->y_stride_batch; s.y_stride_token = a->y_stride_token;
  if (a->seqlen == 0) { s.x = s.B = s.C = nullptr; }
  int rc = check_scan(&s, cp.sp);
  if (rc != SSD_OK) return rc;  // (its messages name ssd_chunk_scan_fwd: the scan half of this call)
  cp.plan = ssd::make_scan_plan(cp.sp, a->seg_chunks);
  cp.conv_bytes = align256((size_t)a->batch * (size_t)L * (size_t)out_ch * (size_t)es);
  cp.scan_off = cp.conv_bytes;
  cp.total = cp.conv_bytes + cp.plan.ws_bytes;

  ssd::ConvParams &c = cp.conv;
  c = ssd::ConvParams{};
  c.bf16 = bf16;
  c.batch = a->batch; c.L = a->seqlen; c.CH = (int)out_ch;
  const int64_t ch0 = bf16 ? HP : 0;  // first channel the conv launch covers
  c.x = a->xBC ? static_cast<const char *>(a->xBC) + ch0 * es : nullptr;
  c.x_sb = a->xBC_stride_batch; c.x_st = a->xBC_stride_token;
  c.o_sb = L * out_ch; c.o_st = out_ch;
  c.w = a->conv_weight + ch0 * ssd::kConvWidth;
  c.bias = a->conv_bias ? a->conv_bias + ch0 : nullptr;
  c.seq_idx = a->seq_idx; c.num_seqs = a->num_seqs;
  c.state_in = a->conv_state_in ? static_cast<const char *>(a->conv_state_in) + ch0 * es : nullptr;
  c.state_out = nullptr;
  c.s_st = conv_dim;
  if (bf16) {
    cp.sp.xconv = 1;
    cp.sp.conv_w = a->conv_weight;
    cp.sp.conv_b = a->conv_bias;
    cp.sp.conv_state = a->conv_state_in;
    cp.sp.conv_ch = conv_dim;
  }
  return SSD_OK;
}
}  // namespace

extern "C" {

size_t ssd_conv_scan_workspace_size(const ssd_conv_scan_args *a) {
  ConvScanPlan cp;
  if (plan_conv_scan(a, cp) != SSD_OK) return (size_t)-1;
  return cp.total;
}

int ssd_conv_scan_fwd(const ssd_conv_scan_args *a, void *workspace, size_t ws_bytes, void *stream) {
  ConvScanPlan cp;
  const int rc = plan_conv_scan(a, cp);
  if (rc != SSD_OK) return rc;
  if (ws_bytes < cp.total || (cp.total > 0 && !workspace))
    return fail(SSD_ERR_WORKSPACE_TOO_SMALL, "ssd_conv_scan_fwd: workspace needs %zu bytes, got %zu", cp.total,
                ws_bytes);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(SSD_ERR_MISALIGNED, "ssd_conv_scan_fwd: workspace must be 256-byte aligned");
  const int drc = debug_check_seq_idx("ssd_conv_scan_fwd", a->seq_idx, a->seqlen, a->num_seqs, stream);
  if (drc != SSD_OK) return drc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const int es = dtype_size(a->dtype);
  const int64_t HP = (int64_t)a->nheads * a->headdim, GN = (int64_t)a->ngroups * a->dstate;
  ssd::ConvParams c = cp.conv;
  ssd::ScanParams sp = cp.sp;
  if (a->seqlen > 0) {
    c.out = ws;
    hipError_t e = ssd::launch_conv1d_silu(c, st);
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_conv_scan_fwd (conv): %s", hipGetErrorString(e));
    if (sp.xconv) {
      sp.B = ws;                 // conv output: B | C channels
      sp.C = ws + GN * es;
    } else {
      sp.x = ws;                 // conv output: x | B | C channels
      sp.B = ws + HP * es;
      sp.C = ws + (HP + GN) * es;
    }
  }
  hipError_t e = ssd::launch_chunk_scan(sp, cp.plan, ws + cp.scan_off, st);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_conv_scan_fwd (scan): %s", hipGetErrorString(e));
  if (a->conv_state_out) {
    // after every read of conv_state_in (the two may be one buffer)
    ssd::ConvParams x = ssd::ConvParams{};
    x.bf16 = c.bf16;
    x.batch = a->batch; x.L = a->seqlen; x.CH = (int)(HP + 2 * GN);
    x.x = a->xBC; x.x_sb = a->xBC_stride_batch; x.x_st = a->xBC_stride_token;
    x.seq_idx = a->seq_idx; x.num_seqs = a->num_seqs;
    x.state_in = a->conv_state_in; x.state_out = a->conv_state_out;
    x.s_st = HP + 2 * GN;
    e = ssd::launch_conv_state_out(x, st);
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_conv_scan_fwd (conv state): %s", hipGetErrorString(e));
  }
  return ok();
}

static int check_bwd(const ssd_scan_bwd_args *a) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_bwd: args is NULL");
  if (a->struct_size != sizeof(ssd_scan_bwd_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_bwd: struct_size %u != %zu", a->struct_size,
                sizeof(ssd_scan_bwd_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_chunk_scan_bwd: dtype %d not supported", a->dtype);
  if (a->batch < 1 || a->seqlen < 0 || a->nheads < 1 || a->ngroups < 1)
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_bwd: non-positive dims");
  if (a->nheads % a->ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_bwd: nheads %d not a multiple of ngroups %d", a->nheads,
                a->ngroups);
  if (a->headdim != ssd::kHeadDim || a->dstate != ssd::kDState)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_chunk_scan_bwd: built for headdim 64, dstate 128 (got %d, %d)", a->headdim,
                a->dstate);
  if (!a->A || !a->dA) return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_bwd: A and dA are required");
  if (a->seqlen > 0 && (!a->x || !a->dt || !a->B || !a->C || !a->dy || !a->dx || !a->ddt || !a->dB || !a->dC))
    return fail(SSD_ERR_INVALID_ARG, "ssd_chunk_scan_bwd: x, dt, B, C, dy, dx, ddt, dB and dC are required");
  const void *al[] = {a->x, a->B, a->C, a->dy, a->dx, a->dB, a->dC, a->initial_state, a->d_final_state,
                      a->d_initial_state};
  for (const void *q : al)
    if (q && !aligned16(q)) return fail(SSD_ERR_MISALIGNED, "ssd_chunk_scan_bwd: tensors must be 16-byte aligned");
  return SSD_OK;
}

size_t ssd_chunk_scan_bwd_workspace_size(const ssd_scan_bwd_args *a) {
  if (check_bwd(a) != SSD_OK) return (size_t)-1;
  return ssd::bwd_layout(a->batch, a->seqlen, a->nheads, a->ngroups).bytes;
}

int ssd_chunk_scan_bwd(const ssd_scan_bwd_args *a, void *workspace, size_t ws_bytes, void *stream) {
  const int rc = check_bwd(a);
  if (rc != SSD_OK) return rc;
  const ssd::BwdLayout w = ssd::bwd_layout(a->batch, a->seqlen, a->nheads, a->ngroups);
  if (ws_bytes < w.bytes || !workspace)
    return fail(SSD_ERR_WORKSPACE_TOO_SMALL, "ssd_chunk_scan_bwd: workspace needs %zu bytes, got %zu", w.bytes,
                ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(SSD_ERR_MISALIGNED, "ssd_chunk_scan_bwd: workspace must be 256-byte aligned");
  char *ws = reinterpret_cast<char *>(workspace);
  ssd::BwdParams p{};
  p.bf16 = a->dtype == SSD_DTYPE_BF16;
  p.batch = a->batch; p.L = a->seqlen; p.H = a->nheads; p.G = a->ngroups; p.nchunks = w.nchunks;
  p.x = a->x; p.dt = a->dt; p.B = a->B; p.C = a->C; p.dy = a->dy;
  p.dt_bias = a->dt_bias; p.A = a->A; p.D = a->D; p.init = a->initial_state; p.dfinal = a->d_final_state;
  p.dx = a->dx; p.ddt = a->ddt; p.dB = a->dB; p.dC = a->dC;
  p.ddt_bias = a->d_dt_bias; p.dA = a->dA; p.dD = a->dD; p.dinit = a->d_initial_state;
  p.ws_states = reinterpret_cast<float *>(ws + w.states_off);
  p.ws_dB = reinterpret_cast<float *>(ws + w.dB_off);
  p.ws_dC = reinterpret_cast<float *>(ws + w.dC_off);
  p.ws_scalars = reinterpret_cast<float *>(ws + w.scalars_off);
  const hipError_t e = ssd::launch_chunk_scan_bwd(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_chunk_scan_bwd: %s", hipGetErrorString(e));
  return ok();
}

int ssd_linear(const ssd_linear_args *a, void *stream) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_linear: args is NULL");
  if (a->struct_size != sizeof(ssd_linear_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_linear: struct_size %u != %zu", a->struct_size, sizeof(ssd_linear_args));
  if (a->dtype != SSD_DTYPE_BF16) return fail(SSD_ERR_UNSUPPORTED, "ssd_linear: dtype %d not supported (bf16)", a->dtype);
  if (a->M < 0 || a->N < 0 || a->K < 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_linear: negative dims (M %d N %d K %d)", a->M, a->N, a->K);
  if (a->K % 64 != 0) return fail(SSD_ERR_UNSUPPORTED, "ssd_linear: K %d not a multiple of 64", a->K);
  if (a->N % 8 != 0) return fail(SSD_ERR_UNSUPPORTED, "ssd_linear: N %d not a multiple of 8", a->N);
  if (a->M == 0 || a->N == 0) return ok();
  if (!a->x || !a->w || !a->y) return fail(SSD_ERR_INVALID_ARG, "ssd_linear: x, w and y are required");
  if (a->x_stride < a->K || a->w_stride < a->K || a->y_stride < a->N)
    return fail(SSD_ERR_INVALID_ARG, "ssd_linear: row strides below the row widths");
  const int64_t kMaxSt = int64_t(1) << 22;
  if (a->x_stride >= kMaxSt || a->w_stride >= kMaxSt || a->y_stride >= kMaxSt)
    return fail(SSD_ERR_INVALID_ARG, "ssd_linear: row strides must be below 2^22 elements");
  if (!vec_ok(a->x, 0, a->x_stride, 2) || !vec_ok(a->w, 0, a->w_stride, 2) || !vec_ok(a->y, 0, a->y_stride, 2))
    return fail(SSD_ERR_MISALIGNED, "ssd_linear: 16-byte aligned bases and row strides multiples of 8 elements");
  ssd::LinearParams p{};
  p.M = a->M; p.N = a->N; p.K = a->K;
  p.x = a->x; p.x_st = a->x_stride;
  p.w = a->w; p.w_st = a->w_stride;
  p.y = a->y; p.y_st = a->y_stride;
  if (a->K == 0) return fail(SSD_ERR_UNSUPPORTED, "ssd_linear: K must be positive");
  const hipError_t e = ssd::launch_linear_bf16(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_linear: %s", hipGetErrorString(e));
  return ok();
}

int ssd_gated_rmsnorm(const ssd_norm_args *a, void *stream) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: args is NULL");
  if (a->struct_size != sizeof(ssd_norm_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: struct_size %u != %zu", a->struct_size,
                sizeof(ssd_norm_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_gated_rmsnorm: dtype %d not supported", a->dtype);
  if (a->batch < 1 || a->seqlen < 0 || a->channels < 1 || a->group_size < 1)
    return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: non-positive dims (batch %d seqlen %d channels %d group %d)",
                a->batch, a->seqlen, a->channels, a->group_size);
  if (a->channels % a->group_size != 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: channels %d not a multiple of group_size %d", a->channels,
                a->group_size);
  const int es = dtype_size(a->dtype);
  const int gmax = es == 2 ? 8192 : 4096;  // 16 vectors of 16 bytes per lane
  if (a->group_size % (16 / es) != 0 || a->group_size > gmax)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_gated_rmsnorm: group_size %d must be a multiple of %d and at most %d",
                a->group_size, 16 / es, gmax);
  if (!(a->eps >= 0.f) || a->eps > 3.0e38f)
    return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: eps must be finite and >= 0");
  if (!a->weight) return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: weight is NULL");
  if (a->seqlen > 0 && (!a->y || !a->out))
    return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: y and out are required");
  if (a->seqlen > 0) {
    if (!vec_ok(a->y, a->y_stride_batch, a->y_stride_token, es) ||
        !vec_ok(a->out, a->out_stride_batch, a->out_stride_token, es) ||
        (a->z && !vec_ok(a->z, a->z_stride_batch, a->z_stride_token, es)) || !aligned16(a->weight))
      return fail(SSD_ERR_MISALIGNED,
                  "ssd_gated_rmsnorm: y, z, out, weight need 16-byte aligned bases and strides multiple of %d",
                  16 / es);
    if (a->y_stride_token < a->channels || a->out_stride_token < a->channels ||
        (a->z && a->z_stride_token < a->channels))
      return fail(SSD_ERR_INVALID_ARG, "ssd_gated_rmsnorm: token strides smaller than channels");
  }
  ssd::NormParams p{};
  p.bf16 = a->dtype == SSD_DTYPE_BF16;
  p.batch = a->batch; p.L = a->seqlen; p.CH = a->channels; p.gs = a->group_size;
  p.before = a->norm_before_gate != 0; p.eps = a->eps;
  p.y = a->y; p.y_sb = a->y_stride_batch; p.y_st = a->y_stride_token;
  p.z = a->z; p.z_sb = a->z_stride_batch; p.z_st = a->z_stride_token;
  p.w = a->weight;
  p.out = a->out; p.o_sb = a->out_stride_batch; p.o_st = a->out_stride_token;
  const hipError_t e = ssd::launch_gated_rmsnorm(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_gated_rmsnorm: %s", hipGetErrorString(e));
  return ok();
}

int ssd_decode_step_mimo(const ssd_mimo_decode_args *a, void *stream) {
  if (!a) return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: args is NULL");
  if (a->struct_size != sizeof(ssd_mimo_decode_args))
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: struct_size %u != %zu", a->struct_size,
                sizeof(ssd_mimo_decode_args));
  if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step_mimo: dtype %d not supported", a->dtype);
  if (a->batch < 1 || a->nheads < 1 || a->ngroups < 1)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: non-positive dims");
  if (a->nheads % a->ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: nheads %d not a multiple of ngroups %d", a->nheads,
                a->ngroups);
  if (a->headdim != ssd::kHeadDim || a->dstate != ssd::kDState)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step_mimo: built for headdim 64, dstate 128 (got %d, %d)",
                a->headdim, a->dstate);
  if (a->rank != 1 && a->rank != 2 && a->rank != 4 && a->rank != 8)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step_mimo: rank %d not in {1, 2, 4, 8}", a->rank);
  if (!a->x || !a->B || !a->C || !a->dt || !a->A || !a->ssm_state || !a->y)
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: x, B, C, dt, A, ssm_state and y are required");
  if (a->trapezoid && (!a->prev_x || !a->prev_B))
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: the trapezoidal form needs prev_x and prev_B");
  const int hpg = a->nheads / a->ngroups;
  if (ssd::mimo_lds_bytes(hpg, a->rank, a->trapezoid != 0) > 160 * 1024)
    return fail(SSD_ERR_UNSUPPORTED, "ssd_decode_step_mimo: nheads / ngroups = %d at rank %d exceeds the LDS of one "
                "workgroup", hpg, a->rank);
  if (!aligned16(a->ssm_state)) return fail(SSD_ERR_MISALIGNED, "ssd_decode_step_mimo: ssm_state must be 16-byte aligned");
  const int64_t R = a->rank;
  if (a->x_stride_batch < (int64_t)a->nheads * a->headdim * R || a->y_stride_batch < (int64_t)a->nheads * a->headdim * R ||
      a->B_stride_batch < (int64_t)a->ngroups * a->dstate * R || a->C_stride_batch < (int64_t)a->ngroups * a->dstate * R ||
      a->dt_stride_batch < a->nheads || (a->lam && a->lam_stride_batch < a->nheads))
    return fail(SSD_ERR_INVALID_ARG, "ssd_decode_step_mimo: batch strides smaller than the row width");
  ssd::MimoParams p{};
  p.bf16 = a->dtype == SSD_DTYPE_BF16;
  p.batch = a->batch; p.H = a->nheads; p.G = a->ngroups; p.R = a->rank; p.trapezoid = a->trapezoid != 0;
  p.x = a->x; p.x_sb = a->x_stride_batch;
  p.B = a->B; p.B_sb = a->B_stride_batch;
  p.C = a->C; p.C_sb = a->C_stride_batch;
  p.dt = a->dt; p.dt_sb = a->dt_stride_batch;
  p.lam = a->lam; p.lam_sb = a->lam_stride_batch;
  p.dt_bias = a->dt_bias; p.A = a->A; p.D = a->D;
  p.ssm_state = a->ssm_state; p.prev_x = a->prev_x; p.prev_B = a->prev_B;
  p.y = a->y; p.y_sb = a->y_stride_batch;
  const hipError_t e = ssd::launch_decode_mimo(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_decode_step_mimo: %s", hipGetErrorString(e));
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
