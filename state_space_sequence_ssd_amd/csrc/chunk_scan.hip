// Chunked SSD prefill of the Mamba-2 selective scan on gfx950: the work
// plan, the fp32 path and the launch sequence (the bf16 MFMA kernel is in
// chunk_scan_bf16.hip).
//
// The layer's per-head recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t B_t^T,
// y_t = S_t C_t + D x_t has a scalar-times-identity transition ("Mamba-3: an
// inference-first state space model", on Mamba-2's simplified transition),
// which makes the map over a block of tokens a masked matrix product -- the
// state space duality with (linear) attention ("AI Engineering EP6",
// sec. 8 and sec. 10).  Blocks are chunk_size = 128 tokens ("Nemotron-H style
// Hybrid Mamba-Transformer 3B feasibility study", sec. 1.4).  For a block
// with inclusive in-block cumulative log-decay cs_i = sum_{k<=i} dt_k A:
//
//   CB    = C B^T                                           (K = N)
//   M_ij  = CB_ij exp(cs_i - cs_j) dt_j  for j <= i, else 0  (+ D on j == i)
//   y     = exp(cs_i) C_i H_prev^T  +  sum_j M_ij x_j
//   H     = exp(cs_last) H_prev + sum_j exp(cs_last - cs_j) dt_j x_j B_j^T
//
// Every exponent is a difference cs_i - cs_j with j <= i, so it is <= 0:
// no exp(+large) ever forms.  The result does not depend on the block
// length, which the fp32 path uses (64-token sub-blocks).
//
// Work: one workgroup = one segment of one sequence x one head; it walks
// the segment's chunks in order and keeps the state on chip, so chunk
// states never go to HBM.
//   * packed sequences: a chunk grid is anchored at each sequence start, so
//     no chunk spans two sequences; plan_kernel builds the sequence table
//     and work list from seq_idx on the device.
//   * long sequences with too few (sequence, head) pairs to fill the chip
//     are cut into segments: a state-only pre-pass gives each segment's
//     local end state and total log-decay, combine_kernel chains them into
//     entry states (affine maps h -> a h + S), and the full pass then runs
//     all segments in parallel -- the split of the scan over chunks that the
//     "Nemotron-Mamba3 architecture" article, sec. 2.2, mentions, one level
//     deep.
//   * workgroup -> work mapping is XCD-aware: consecutive work (the heads of
//     one group on one segment, which read the same B and C) goes to the
//     same XCD, so B/C come from HBM once and from that XCD's L2 after.
#include "common.h"
#include "kernels.h"
#include "scan_items.h"

namespace ssd {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// fp32 path: register-tiled FMA kernel (all-fp32 arithmetic, for fp32 inputs)
// ---------------------------------------------------------------------------
// The chunk form is exact for any block length, so this path walks each
// 128-token chunk of the work list as two sub-chunks of kSub = 64 tokens: x,
// B and C of a sub-chunk, its decay-masked matrix M and a copy of the state
// then all fit in LDS, and every product is a 4x4 (state: 4x8) register tile
// per thread over LDS operands.  The fp32 state itself stays in registers.
constexpr int kSub = 64;
constexpr int kPadX = kHeadDim + 4;  // LDS row strides (floats): rows stay 16-byte aligned
constexpr int kPadN = kDState + 4;
constexpr int kPadM = kSub + 4;

// dt = softplus(dt_raw + bias), inclusive in-sub-chunk cumulative log-decay
// cs, w = exp(cs_last - cs) dt, and exp(cs_last), cs_last; one token per lane
// of one wave.  Tokens past the end get dt = 0: cs stays flat and they drop
// out of every product.
__device__ __forceinline__ void subchunk_dt(float raw, bool valid, float bias, float A, float *s_cs,
                                            float *s_dt, float *s_w, float *s_misc) {
  const int lane = threadIdx.x & 63;
  const float d = valid ? softplus_f32(raw + bias) : 0.f;
  float incl = d * A;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  const float total = __shfl(incl, 63, 64);
  s_cs[lane] = incl;
  s_dt[lane] = d;
  s_w[lane] = expf(total - incl) * d;
  if (lane == 0) {
    s_misc[0] = expf(total);
    s_misc[1] = total;
  }
}

__device__ __forceinline__ float4 lds4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// acc[r][c] += a[r] . b[c] over 4 consecutive K values
__device__ __forceinline__ void fma4x4(float (&acc)[4][4], const float4 (&a)[4], const float4 (&b)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[r][c] = fmaf(a[r].w, b[c].w, fmaf(a[r].z, b[c].z, fmaf(a[r].y, b[c].y, fmaf(a[r].x, b[c].x, acc[r][c]))));
}

template <bool kFull>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_f32_kernel(ScanParams p, ScanPlan plan,
                                                                     char *ws) {
  __shared__ __attribute__((aligned(16))) float sX[kSub * kPadX];      // x[j][p]
  __shared__ __attribute__((aligned(16))) float sB[kSub * kPadN];      // B[j][n]
  __shared__ __attribute__((aligned(16))) float sC[kSub * kPadN];      // C[i][n]
  __shared__ __attribute__((aligned(16))) float sH[kHeadDim * kPadN];  // H[p][n] entering the sub-chunk
  __shared__ __attribute__((aligned(16))) float sM[kSub * kPadM];      // M[i][j]
  __shared__ __attribute__((aligned(16))) float s_cs[kSub];
  __shared__ __attribute__((aligned(16))) float s_dt[kSub];
  __shared__ __attribute__((aligned(16))) float s_w[kSub];
  __shared__ float s_misc[2];

  int item, h, g;
  if (!map_workgroup(p, plan, ws, item, h, g)) return;
  Item it;
  if (!get_item(p, plan, ws, item, it)) return;
  if (!kFull && it.last) return;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const float *xg = reinterpret_cast<const float *>(p.x) + it.boff * p.x_sb + h * kHeadDim;
  const float *Bg = reinterpret_cast<const float *>(p.B) + it.boff * p.B_sb + g * kDState;
  const float *Cg = reinterpret_cast<const float *>(p.C) + it.boff * p.C_sb + g * kDState;
  const float *dtg = reinterpret_cast<const float *>(p.dt) + it.boff * p.dt_sb + h;
  float *yg = reinterpret_cast<float *>(p.y) + it.boff * p.y_sb + h * kHeadDim;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;

  // output tiles: rows i in [4 ti, +4), columns (j of M, or p of y) in [4 tj, +4)
  const int ti = tid >> 4, tj = tid & 15;
  // state tile: p in [4 ti, +4), n in [8 tj, +8), in registers
  float hs[4][8];
  {
    const float *entry = nullptr;
    if (kFull) {
      if (it.first) entry = p.init ? p.init + ((int64_t)it.row * p.H + h) * kPN : nullptr;
      else entry = ws_f32(plan, ws, plan.ws_entry_off) + ((int64_t)item * p.H + h) * kPN;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) hs[r][c] = entry ? entry[(4 * ti + r) * kDState + 8 * tj + c] : 0.f;
    if (kFull) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<float4 *>(sH + (4 * ti + r) * kPadN + 8 * tj) = make_float4(hs[r][0], hs[r][1], hs[r][2], hs[r][3]);
        *reinterpret_cast<float4 *>(sH + (4 * ti + r) * kPadN + 8 * tj + 4) = make_float4(hs[r][4], hs[r][5], hs[r][6], hs[r][7]);
      }
    }
  }

  float logdecay = 0.f;
  for (int c0 = it.tok0; c0 < it.tok1; c0 += kSub) {
    const int nv = min(kSub, it.tok1 - c0);
    // stage x, B (and C) of this sub-chunk, rows past the end zero
#pragma unroll
    for (int k = 0; k < kSub * kHeadDim / 4 / kThreads; ++k) {
      const int f = tid + k * kThreads, j = f >> 4, c4 = f & 15;
      *reinterpret_cast<float4 *>(sX + j * kPadX + 4 * c4) =
          j < nv ? *reinterpret_cast<const float4 *>(xg + (int64_t)(c0 + j) * p.x_st + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kSub * kDState / 4 / kThreads; ++k) {
      const int f = tid + k * kThreads, j = f >> 5, c4 = f & 31;
      *reinterpret_cast<float4 *>(sB + j * kPadN + 4 * c4) =
          j < nv ? *reinterpret_cast<const float4 *>(Bg + (int64_t)(c0 + j) * p.B_st + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (kFull)
        *reinterpret_cast<float4 *>(sC + j * kPadN + 4 * c4) =
            j < nv ? *reinterpret_cast<const float4 *>(Cg + (int64_t)(c0 + j) * p.C_st + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wv == 0) {
      const float raw = lane < nv ? dtg[(int64_t)(c0 + lane) * p.dt_st] : 0.f;
      subchunk_dt(raw, lane < nv, bias, Ah, s_cs, s_dt, s_w, s_misc);
    }
    __syncthreads();

    float yo[4][4];
    if (kFull) {
      // M[i][j] = (C_i . B_j) exp(cs_i - cs_j) dt_j for j < i, (C_i . B_i) dt_i + D on
      // the diagonal, 0 above it; tiles entirely above the diagonal are never read
      if (tj <= ti) {
        float cb[4][4] = {};
        for (int n = 0; n < kDState; n += 4) {
          float4 a[4], b[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = lds4(sC + (4 * ti + r) * kPadN + n);
#pragma unroll
          for (int c = 0; c < 4; ++c) b[c] = lds4(sB + (4 * tj + c) * kPadN + n);
          fma4x4(cb, a, b);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * ti + r;
          const float cs_i = s_cs[i];
          float m[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = 4 * tj + c;
            m[c] = j < i ? cb[r][c] * expf(cs_i - s_cs[j]) * s_dt[j] : j == i ? fmaf(cb[r][c], s_dt[j], Dh) : 0.f;
          }
          *reinterpret_cast<float4 *>(sM + i * kPadM + 4 * tj) = make_float4(m[0], m[1], m[2], m[3]);
        }
      }
      // state -> output: yo[i][p] = C_i . H_prev[p]
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) yo[r][c] = 0.f;
      for (int n = 0; n < kDState; n += 4) {
        float4 a[4], b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = lds4(sC + (4 * ti + r) * kPadN + n);
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = lds4(sH + (4 * tj + c) * kPadN + n);
        fma4x4(yo, a, b);
      }
    }
    __syncthreads();  // M complete; every read of the entering state done

    if (kFull) {
      // y[i][p] = exp(cs_i) yo[i][p] + sum_{j <= i} M[i][j] x[j][p]
      float yd[4][4] = {};
      for (int j0 = 0; j0 <= 4 * ti; j0 += 4) {
        float4 m[4], xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = lds4(sM + (4 * ti + r) * kPadM + j0);
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = lds4(sX + (j0 + q) * kPadX + 4 * tj);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float mr[4] = {m[r].x, m[r].y, m[r].z, m[r].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            yd[r][0] = fmaf(mr[q], xv[q].x, yd[r][0]);
            yd[r][1] = fmaf(mr[q], xv[q].y, yd[r][1]);
            yd[r][2] = fmaf(mr[q], xv[q].z, yd[r][2]);
            yd[r][3] = fmaf(mr[q], xv[q].w, yd[r][3]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * ti + r;
        if (i < nv) {
          const float ecs = expf(s_cs[i]);
          *reinterpret_cast<float4 *>(yg + (int64_t)(c0 + i) * p.y_st + 4 * tj) =
              make_float4(fmaf(ecs, yo[r][0], yd[r][0]), fmaf(ecs, yo[r][1], yd[r][1]),
                          fmaf(ecs, yo[r][2], yd[r][2]), fmaf(ecs, yo[r][3], yd[r][3]));
        }
      }
    }
    // state: H = exp(cs_last) H + sum_j w_j x_j B_j^T on this thread's tile
    {
      float acc[4][8] = {};
      for (int j = 0; j < nv; ++j) {
        const float wj = s_w[j];
        const float4 xv = lds4(sX + j * kPadX + 4 * ti);
        const float4 b0 = lds4(sB + j * kPadN + 8 * tj), b1 = lds4(sB + j * kPadN + 8 * tj + 4);
        const float xw[4] = {xv.x * wj, xv.y * wj, xv.z * wj, xv.w * wj};
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(xw[r], bb[c], acc[r][c]);
      }
      const float dec = s_misc[0];
      logdecay += s_misc[1];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) hs[r][c] = fmaf(dec, hs[r][c], acc[r][c]);
    }
    __syncthreads();  // every read of this sub-chunk's LDS operands done
    if (kFull) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<float4 *>(sH + (4 * ti + r) * kPadN + 8 * tj) = make_float4(hs[r][0], hs[r][1], hs[r][2], hs[r][3]);
        *reinterpret_cast<float4 *>(sH + (4 * ti + r) * kPadN + 8 * tj + 4) = make_float4(hs[r][4], hs[r][5], hs[r][6], hs[r][7]);
      }
    }
  }

  float *dst = nullptr;
  if (kFull) {
    if (it.last && p.final_state) dst = p.final_state + ((int64_t)it.row * p.H + h) * kPN;
  } else {
    dst = ws_f32(plan, ws, plan.ws_local_off) + ((int64_t)item * p.H + h) * kPN;
    if (tid == 0) ws_f32(plan, ws, plan.ws_decay_off)[(int64_t)item * p.H + h] = logdecay;
  }
  if (dst) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4 *>(dst + (4 * ti + r) * kDState + 8 * tj) = make_float4(hs[r][0], hs[r][1], hs[r][2], hs[r][3]);
      *reinterpret_cast<float4 *>(dst + (4 * ti + r) * kDState + 8 * tj + 4) = make_float4(hs[r][4], hs[r][5], hs[r][6], hs[r][7]);
    }
  }
}

// ---------------------------------------------------------------------------
// packed-sequence planner: sequence bounds from seq_idx and the work list
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanSortMax = 4096;  // longer work lists are not reordered

// First index in [0, L] with seq_idx[i] >= s, found by a group of gs lanes
// (gs a power of two up to 64, the group aligned inside its wave, lane k of
// it): every round the group probes gs points of [lo, hi) at once and keeps
// the gap between the last probe below s and the first one not below, so a
// search takes log_{gs+1} L rounds of one load each.  gs = 1 is a binary
// search.  The result stays in [0, L] whatever seq_idx holds.
__device__ __forceinline__ int lower_bound_group(const int32_t *seq_idx, int L, int s, int gs, int k) {
  const int gbase = (threadIdx.x & 63) & ~(gs - 1);
  const uint64_t gmask = (gs == 64 ? ~0ull : (1ull << gs) - 1) << gbase;
  int lo = 0, hi = L;
  while (hi - lo > gs) {
    const int n = hi - lo;
    const int pk = lo + (int)((int64_t)(k + 1) * n / (gs + 1));
    const int c = __popcll(__ballot(seq_idx[pk] < s) & gmask);
    const int nlo = c > 0 ? lo + (int)((int64_t)c * n / (gs + 1)) + 1 : lo;
    const int nhi = c < gs ? lo + (int)((int64_t)(c + 1) * n / (gs + 1)) : hi;
    lo = nlo;
    hi = nhi;
  }
  const bool below = lo + k < hi && seq_idx[lo + k] < s;
  return lo + __popcll(__ballot(below) & gmask);
}

// Where every sequence id starts: one search per id in [0, rows], all of them
// in parallel, with as many lanes per search as the workgroup has to spare;
// the end of id s is the start of id s + 1.
__device__ __forceinline__ void sequence_bounds(const int32_t *seq_idx, int L, int rows, int *seq_start,
                                                int *seq_end) {
  int gs = 64;
  while (gs > 1 && gs * (rows + 1) > kPlanThreads) gs >>= 1;
  const int per_pass = kPlanThreads / gs;
  for (int b0 = 0; b0 <= rows; b0 += per_pass) {
    const int b = b0 + (int)threadIdx.x / gs;  // the same for the whole group
    if (b <= rows) {
      const int k = (int)threadIdx.x & (gs - 1);
      const int st = lower_bound_group(seq_idx, L, b, gs, k);
      if (k == 0) {
        if (b < rows) seq_start[b] = st;
        if (b >= 1) seq_end[b - 1] = st;
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t *seq_idx, int L,
                                                            ScanPlan plan, char *ws) {
  int *b = reinterpret_cast<int *>(ws + plan.ws_plan_off);
  int *seq_start = b, *seq_end = b + plan.rows, *seq_nseg = b + 2 * plan.rows;
  int *seq_off = b + 3 * plan.rows;
  int *item_seq = b + 4 * plan.rows;
  int *item_k = item_seq + plan.items;
  int *n_items = item_k + plan.items;
  __shared__ int scan[kPlanThreads];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  sequence_bounds(seq_idx, L, plan.rows, seq_start, seq_end);
  for (int base = 0; base < plan.rows; base += kPlanThreads) {
    const int s = base + threadIdx.x;
    int nseg = 0, st = 0, en = 0;
    if (s < plan.rows) {
      st = seq_start[s];
      en = max(st, seq_end[s]);
      nseg = max(1, (en - st + plan.seg_len - 1) / plan.seg_len);
    }
    scan[threadIdx.x] = nseg;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int t = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += t;
      __syncthreads();
    }
    const int off0 = carry + scan[threadIdx.x] - nseg;  // exclusive offset
    if (s < plan.rows) {
      seq_start[s] = st;
      seq_end[s] = en;
      seq_nseg[s] = nseg;
      seq_off[s] = off0;
      for (int k = 0; k < nseg; ++k) {
        if (off0 + k < plan.items) {
          item_seq[off0 + k] = s;
          item_k[off0 + k] = k;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == kPlanThreads - 1) carry += scan[kPlanThreads - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_items = min(carry, plan.items);
  __syncthreads();
  // Items ranked longest first (ties in list order), the order in which the
  // scan kernels start them.  The rank count is quadratic, so very long work
  // lists keep their list order.
  int *item_order = n_items + 1;
  const int n = min(carry, plan.items);
  __shared__ int nchunks[kPlanSortMax];
  const bool sort = n <= kPlanSortMax;
  if (sort) {
    for (int i = threadIdx.x; i < n; i += kPlanThreads) {
      const int s = item_seq[i], t0 = seq_start[s] + item_k[i] * plan.seg_len;
      nchunks[i] = (min(seq_end[s], t0 + plan.seg_len) - t0 + kChunk - 1) / kChunk;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kPlanThreads) {
    int rank = i;
    if (sort) {
      const int ci = nchunks[i];
      rank = 0;
      for (int j = 0; j < n; ++j) {
        const int cj = nchunks[j];
        rank += cj > ci || (cj == ci && j < i);
      }
    }
    item_order[rank] = i;
  }
}

// ---------------------------------------------------------------------------
// segment combine: entry state of segment k = decay_{k-1} entry_{k-1} + local_{k-1}
// ---------------------------------------------------------------------------
// The map is elementwise over the state, so each (row, head) is split over
// kCombSplit workgroups with one float4 of the state per thread, and the local
// states of kCombBatch segments are all in flight before their chain runs:
// the kernel then costs a few memory round trips instead of one per segment.
constexpr int kCombSplit = 8;
constexpr int kCombBatch = 8;
static_assert(kPN / 4 == kCombSplit * kThreads, "one float4 of the state per thread");

__global__ __launch_bounds__(kThreads) void combine_kernel(ScanParams p, ScanPlan plan, char *ws) {
  const int part = blockIdx.x % kCombSplit;
  const int row = blockIdx.x / kCombSplit / p.H;
  const int h = blockIdx.x / kCombSplit % p.H;
  int nseg, off;
  if (plan.packed) {
    const PlanView v = plan_view(plan, ws);
    nseg = v.seq_nseg[row];
    off = v.seq_off[row];
  } else {
    nseg = plan.nseg;
    off = row * plan.nseg;
  }
  if (nseg <= 1) return;
  const float *__restrict__ local = ws_f32(plan, ws, plan.ws_local_off);
  const float *__restrict__ ldec = ws_f32(plan, ws, plan.ws_decay_off);
  float *__restrict__ entry = ws_f32(plan, ws, plan.ws_entry_off);
  const int idx = part * kThreads + threadIdx.x;  // float4 of the head's state
  float4 e = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.init) e = reinterpret_cast<const float4 *>(p.init + ((int64_t)row * p.H + h) * kPN)[idx];
  const int last = min(nseg, plan.items - off);  // entries 1 .. last-1 are written
  for (int k0 = 1; k0 < last; k0 += kCombBatch) {
    float4 l[kCombBatch];
    float d[kCombBatch];
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      const int prev = off + k0 + j - 1;
      if (k0 + j < last) {
        d[j] = __expf(ldec[(int64_t)prev * p.H + h]);
        l[j] = reinterpret_cast<const float4 *>(local + ((int64_t)prev * p.H + h) * kPN)[idx];
      }
    }
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      if (k0 + j < last) {
        e.x = fmaf(d[j], e.x, l[j].x);
        e.y = fmaf(d[j], e.y, l[j].y);
        e.z = fmaf(d[j], e.z, l[j].z);
        e.w = fmaf(d[j], e.w, l[j].w);
        reinterpret_cast<float4 *>(entry + ((int64_t)(off + k0 + j) * p.H + h) * kPN)[idx] = e;
      }
    }
  }
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

ScanPlan make_scan_plan(const ScanParams &p, int seg_chunks) {
  ScanPlan plan{};
  plan.packed = p.seq_idx != nullptr;
  plan.rows = plan.packed ? p.num_seqs : p.batch;
  if (!p.bf16 && !plan.packed && p.L <= kQuadMaxL) {
    // short fp32 batch rows: one quadratic-form launch (the model's chunk and
    // seg_chunks do not change its result), no workspace
    plan.quad = 1;
    plan.seg_len = std::max(p.L, 1);
    plan.nseg = 1;
    plan.items = p.batch;
    return plan;
  }
  const int chunks_max = std::max(1, (p.L + kChunk - 1) / kChunk);
  // Automatic segments are whole tiles of the kernel that runs them: 128
  // tokens for bf16, the fp32 kernel's 64-token sub-chunks for fp32 (its
  // result does not depend on where segments start, so short inputs with few
  // (sequence, head) pairs get twice the workgroups).
  const int unit = p.bf16 ? kChunk : kSub;
  int seg_units;
  if (seg_chunks <= 0) {
    const int units_max = std::max(1, (p.L + unit - 1) / unit);
    // workgroup slots of one wave of launches: the bf16 kernel fits two per CU
    const long long slots = p.bf16 ? 2LL * kNumCU : (long long)kNumCU;
    const long long base = (long long)plan.rows * p.H;
    if (base >= slots) {
      seg_units = units_max;
    } else {
      const int factor = (int)((slots + base - 1) / base);
      seg_units = std::max(1, (units_max + factor - 1) / factor);
    }
    seg_units = std::min(seg_units, units_max);
  } else {
    seg_units = std::min(seg_chunks, chunks_max) * (kChunk / unit);
  }
  plan.seg_len = seg_units * unit;
  plan.segmented = plan.seg_len < p.L;
  if (!plan.packed) {
    plan.nseg = std::max(1, (p.L + plan.seg_len - 1) / plan.seg_len);
    plan.items = p.batch * plan.nseg;
  } else {
    plan.nseg = 0;
    plan.items = plan.rows + (p.L + plan.seg_len - 1) / plan.seg_len;
  }
  size_t off = 0;
  plan.ws_plan_off = off;
  if (plan.packed) off = align256(off + sizeof(int) * (4 * (size_t)plan.rows + 3 * (size_t)plan.items + 1));
  plan.ws_local_off = plan.ws_entry_off = plan.ws_decay_off = off;
  if (plan.segmented) {
    const size_t st = sizeof(float) * (size_t)plan.items * p.H * kPN;
    plan.ws_local_off = off;
    off = align256(off + st);
    plan.ws_entry_off = off;
    off = align256(off + st);
    plan.ws_decay_off = off;
    off = align256(off + sizeof(float) * (size_t)plan.items * p.H);
  }
  plan.ws_bytes = off;
  return plan;
}

hipError_t launch_chunk_scan(const ScanParams &p, const ScanPlan &plan, void *workspace,
                             hipStream_t stream) {
  if (plan.quad) return launch_quad_scan_f32(p, stream);
  char *ws = reinterpret_cast<char *>(workspace);
  if (plan.packed) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p.seq_idx, p.L, plan, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned nblk = scan_grid_size(p, plan);
  if (nblk == 0) return hipSuccess;
  if (plan.segmented) {
    hipError_t e;
    if (p.bf16) {
      e = launch_chunk_scan_bf16(p, plan, ws, nblk, false, stream);
    } else {
      hipLaunchKernelGGL(chunk_scan_f32_kernel<false>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(plan.rows * p.H * kCombSplit), dim3(kThreads), 0, stream, p, plan, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.bf16) return launch_chunk_scan_bf16(p, plan, ws, nblk, true, stream);
  hipLaunchKernelGGL(chunk_scan_f32_kernel<true>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
  return hipGetLastError();
}

}  // namespace ssd
