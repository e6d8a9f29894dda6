// Chunked SSD prefill of the Mamba-2 selective scan on gfx950.
//
// The layer's per-head recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t B_t^T,
// y_t = S_t C_t + D x_t has a scalar-times-identity transition ("Mamba-3: an
// inference-first state space model", on Mamba-2's simplified transition),
// which makes the map over a block of tokens a masked matrix product -- the
// state space duality with (linear) attention ("AI Engineering EP6",
// sec. 8 and sec. 10).  Blocks are chunk_size = 128 tokens ("Nemotron-H style
// Hybrid Mamba-Transformer 3B feasibility study", sec. 1.4).  For a chunk
// with inclusive in-chunk cumulative log-decay cs_i = sum_{k<=i} dt_k A:
//
//   CB    = C B^T                                           (Q x Q, K = N)
//   M_ji  = CB_ij exp(cs_i - cs_j) dt_j  for j <= i, else 0  (+ D on j == i)
//   y     = exp(cs_i) C_i H_prev^T  +  sum_j M_ji x_j       (K = N, K = Q)
//   H     = exp(cs_last) H_prev + sum_j exp(cs_last - cs_j) dt_j x_j B_j^T
//
// Every exponent is a difference cs_i - cs_j with j <= i, so it is <= 0:
// no exp(+large) ever forms.
//
// Design (one workgroup = one segment of one sequence x one head, 4 waves):
//   * the running state H (64 x 128 fp32) never leaves the chip: it lives in
//     MFMA accumulator registers (wave w owns state rows n in [32w, 32w+32))
//     and, rounded to bf16, in LDS as the operand of the state->output
//     product.  Chunk states are never written to HBM, so the kernel moves
//     each input byte once and each output byte once.
//   * all four products run on v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32
//     accumulation).  Wave w owns output rows i in [32w, 32w+32) of the
//     chunk; it computes the causal CB tiles j-block <= w, turns them into
//     the decay-masked M in registers, and feeds them straight back as the
//     MFMA operand of the intra-chunk product (the accumulator layout holds
//     4+4 rows per lane, used as a permuted K order that the other operand,
//     read from LDS, follows).
//   * B is staged twice in LDS (token-major for C B^T, transposed for the
//     chunk-state product), x once (transposed); C goes global -> registers,
//     each wave loading only its own 32 rows.  The next chunk's loads are
//     issued before the current chunk's math.
//   * packed sequences: a chunk grid is anchored at each sequence start, so
//     no chunk ever spans two sequences; the sequence table comes from
//     seq_idx on the device.
//   * long sequences with too few (sequence, head) pairs to fill 256 CUs are
//     cut into segments; a state-only pre-pass gives each segment's local
//     end state and total decay, a small combine kernel chains them into
//     entry states, and the full pass then runs all segments in parallel
//     (segments are the Blelloch-style split of the scan over chunks that
//     the "Nemotron-Mamba3 architecture" article, sec. 2.2, mentions, one
//     level deep).
//   * workgroup -> work mapping is XCD-aware: consecutive work (the heads of
//     one group on one segment, which read the same B and C) is sent to the
//     same XCD, so B/C come from HBM once and from that XCD's L2 after.
#include "common.h"
#include "kernels.h"
#include "scan_items.h"

namespace ssd {

namespace {

constexpr int kThreads = 256;

// dt, in-chunk cumulative log-decay cs, and the chunk-state weights
// w_j = exp(cs_last - cs_j) dt_j for one chunk; run by one wave (2 tokens per
// lane).  Tokens past the end of the sequence get dt = 0, which leaves cs
// flat and removes them from every product.  Also v_j = exp(cs_r - cs_j) dt_j
// with r the last token of j's 32-token block (the row factor of the
// off-diagonal decay tiles).
__device__ __forceinline__ void chunk_dt(float raw0, float raw1, int j0, int n_valid, float bias,
                                         float A, float *s_cs, float *s_dt, float *s_w,
                                         float *s_misc, float *s_v = nullptr) {
  const int lane = threadIdx.x & 63;
  const float d0 = j0 < n_valid ? softplus_f32(raw0 + bias) : 0.f;
  const float d1 = j0 + 1 < n_valid ? softplus_f32(raw1 + bias) : 0.f;
  const float a0 = d0 * A, a1 = d1 * A;
  float incl = a0 + a1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  const float total = __shfl(incl, 63, 64);
  const float cs1 = incl, cs0 = incl - a1;
  *reinterpret_cast<float2 *>(s_cs + j0) = make_float2(cs0, cs1);
  *reinterpret_cast<float2 *>(s_dt + j0) = make_float2(d0, d1);
  *reinterpret_cast<float2 *>(s_w + j0) =
      make_float2(__expf(total - cs0) * d0, __expf(total - cs1) * d1);
  if (s_v) {
    const float cr = __shfl(incl, lane | 15, 64);  // cs at the end of this 32-token block
    *reinterpret_cast<float2 *>(s_v + j0) = make_float2(__expf(cr - cs0) * d0, __expf(cr - cs1) * d1);
  }
  if (lane == 0) {
    s_misc[0] = __expf(total);
    s_misc[1] = total;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: plain FMA chunk kernel (all-fp32 arithmetic, for fp32 inputs)
// ---------------------------------------------------------------------------
template <bool kFull>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_f32_kernel(ScanParams p, ScanPlan plan,
                                                                     char *ws) {
  __shared__ __attribute__((aligned(16))) float sX[kChunk * kHeadDim];  // [j][p]
  __shared__ __attribute__((aligned(16))) float sB[kChunk * kDState];   // [j][n]
  __shared__ __attribute__((aligned(16))) float sH[kHeadDim * kDState]; // [p][n], the running state
  __shared__ __attribute__((aligned(16))) float s_cs[kChunk];
  __shared__ __attribute__((aligned(16))) float s_dt[kChunk];
  __shared__ __attribute__((aligned(16))) float s_w[kChunk];
  __shared__ float s_misc[2];

  int item, h, g;
  if (!map_workgroup(p, plan, item, h, g)) return;
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
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;

  // state entries updated by this thread: p = tid / 4, n in [32 (tid % 4), +32)
  const int sp = tid >> 2, sn0 = 32 * (tid & 3);
  {
    const float *entry = nullptr;
    if (kFull) {
      if (it.first) entry = p.init ? p.init + ((int64_t)it.row * p.H + h) * kPN : nullptr;
      else entry = ws_f32(plan, ws, plan.ws_entry_off) + ((int64_t)item * p.H + h) * kPN;
    }
    for (int k = 0; k < 32; ++k) sH[sp * kDState + sn0 + k] = entry ? entry[sp * kDState + sn0 + k] : 0.f;
  }

  float logdecay = 0.f;
  for (int c0 = it.tok0; c0 < it.tok1; c0 += kChunk) {
    const int nv = min(kChunk, it.tok1 - c0);
    // stage x, B and dt of this chunk
    for (int f = tid; f < kChunk * kHeadDim / 4; f += kThreads) {
      const int j = f / (kHeadDim / 4), c4 = f % (kHeadDim / 4);
      reinterpret_cast<float4 *>(sX)[f] =
          j < nv ? *reinterpret_cast<const float4 *>(xg + (int64_t)(c0 + j) * p.x_st + 4 * c4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int f = tid; f < kChunk * kDState / 4; f += kThreads) {
      const int j = f / (kDState / 4), c4 = f % (kDState / 4);
      reinterpret_cast<float4 *>(sB)[f] =
          j < nv ? *reinterpret_cast<const float4 *>(Bg + (int64_t)(c0 + j) * p.B_st + 4 * c4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wv == 0) {
      const int j = 2 * lane;
      const float r0 = j < nv ? dtg[(int64_t)(c0 + j) * p.dt_st] : 0.f;
      const float r1 = j + 1 < nv ? dtg[(int64_t)(c0 + j + 1) * p.dt_st] : 0.f;
      chunk_dt(r0, r1, j, nv, bias, Ah, s_cs, s_dt, s_w, s_misc);
    }
    __syncthreads();

    if (kFull) {
      // outputs: thread -> row i = tid / 2, p in [32 (tid % 2), +32)
      const int i = tid >> 1, p0 = 32 * (tid & 1);
      if (i < nv) {
        const float *cr = Cg + (int64_t)(c0 + i) * p.C_st;
        const float cs_i = s_cs[i];
        // state -> output: yo[k] = sum_n C[i][n] H[p0 + k][n]
        float yo[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) yo[k] = 0.f;
        for (int n4 = 0; n4 < kDState / 4; ++n4) {
          const float4 cv = reinterpret_cast<const float4 *>(cr)[n4];
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            const float4 hv = *reinterpret_cast<const float4 *>(sH + (p0 + k) * kDState + 4 * n4);
            yo[k] = fmaf(cv.x, hv.x, fmaf(cv.y, hv.y, fmaf(cv.z, hv.z, fmaf(cv.w, hv.w, yo[k]))));
          }
        }
        // intra-chunk: yd[k] = sum_{j<=i} (C_i . B_j) exp(cs_i - cs_j) dt_j x[j][p0 + k]
        float crow[kDState];
#pragma unroll
        for (int n4 = 0; n4 < kDState / 4; ++n4) {
          const float4 v = reinterpret_cast<const float4 *>(cr)[n4];
          crow[4 * n4] = v.x; crow[4 * n4 + 1] = v.y; crow[4 * n4 + 2] = v.z; crow[4 * n4 + 3] = v.w;
        }
        float yd[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) yd[k] = 0.f;
        for (int j = 0; j <= i; ++j) {
          const float4 *br = reinterpret_cast<const float4 *>(sB + j * kDState);
          float cb = 0.f;
#pragma unroll
          for (int n4 = 0; n4 < kDState / 4; ++n4) {
            const float4 bv = br[n4];
            cb = fmaf(crow[4 * n4], bv.x, cb);
            cb = fmaf(crow[4 * n4 + 1], bv.y, cb);
            cb = fmaf(crow[4 * n4 + 2], bv.z, cb);
            cb = fmaf(crow[4 * n4 + 3], bv.w, cb);
          }
          const float m = cb * expf(cs_i - s_cs[j]) * s_dt[j];
          const float4 *xr = reinterpret_cast<const float4 *>(sX + j * kHeadDim + p0);
#pragma unroll
          for (int k4 = 0; k4 < 8; ++k4) {
            const float4 xv = xr[k4];
            yd[4 * k4] = fmaf(m, xv.x, yd[4 * k4]);
            yd[4 * k4 + 1] = fmaf(m, xv.y, yd[4 * k4 + 1]);
            yd[4 * k4 + 2] = fmaf(m, xv.z, yd[4 * k4 + 2]);
            yd[4 * k4 + 3] = fmaf(m, xv.w, yd[4 * k4 + 3]);
          }
        }
        const float ecs = expf(cs_i);
        float *yrow = reinterpret_cast<float *>(p.y) + it.boff * p.y_sb + (int64_t)(c0 + i) * p.y_st +
                      h * kHeadDim + p0;
        const float *xi = sX + i * kHeadDim + p0;
#pragma unroll
        for (int k4 = 0; k4 < 8; ++k4) {
          float4 o;
          o.x = fmaf(ecs, yo[4 * k4 + 0], yd[4 * k4 + 0]) + Dh * xi[4 * k4 + 0];
          o.y = fmaf(ecs, yo[4 * k4 + 1], yd[4 * k4 + 1]) + Dh * xi[4 * k4 + 1];
          o.z = fmaf(ecs, yo[4 * k4 + 2], yd[4 * k4 + 2]) + Dh * xi[4 * k4 + 2];
          o.w = fmaf(ecs, yo[4 * k4 + 3], yd[4 * k4 + 3]) + Dh * xi[4 * k4 + 3];
          reinterpret_cast<float4 *>(yrow)[k4] = o;
        }
      }
      __syncthreads();  // the state is read above and rewritten below
    }
    // state update of this thread's 32 entries: H = exp(cs_last) H + sum_j w_j x_j B_j^T
    {
      const float dec = s_misc[0];
      logdecay += s_misc[1];
      float acc[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) acc[k] = 0.f;
      for (int j = 0; j < nv; ++j) {
        const float xw = sX[j * kHeadDim + sp] * s_w[j];
        const float4 *br = reinterpret_cast<const float4 *>(sB + j * kDState + sn0);
#pragma unroll
        for (int k4 = 0; k4 < 8; ++k4) {
          const float4 bv = br[k4];
          acc[4 * k4] = fmaf(xw, bv.x, acc[4 * k4]);
          acc[4 * k4 + 1] = fmaf(xw, bv.y, acc[4 * k4 + 1]);
          acc[4 * k4 + 2] = fmaf(xw, bv.z, acc[4 * k4 + 2]);
          acc[4 * k4 + 3] = fmaf(xw, bv.w, acc[4 * k4 + 3]);
        }
      }
      float *hrow = sH + sp * kDState + sn0;
#pragma unroll
      for (int k = 0; k < 32; ++k) hrow[k] = fmaf(dec, hrow[k], acc[k]);
    }
    __syncthreads();
  }

  float *dst = nullptr;
  if (kFull) {
    if (it.last && p.final_state) dst = p.final_state + ((int64_t)it.row * p.H + h) * kPN;
  } else {
    dst = ws_f32(plan, ws, plan.ws_local_off) + ((int64_t)item * p.H + h) * kPN;
    if (tid == 0) ws_f32(plan, ws, plan.ws_decay_off)[(int64_t)item * p.H + h] = logdecay;
  }
  if (dst) {
    __syncthreads();
    for (int k = 0; k < 32; ++k) dst[sp * kDState + sn0 + k] = sH[sp * kDState + sn0 + k];
  }
}

// ---------------------------------------------------------------------------
// packed-sequence planner: sequence bounds from seq_idx and the work list
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lower_bound_seq(const int32_t *seq_idx, int L, int s) {
  int lo = 0, hi = L;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (seq_idx[mid] < s) lo = mid + 1; else hi = mid;
  }
  return lo;
}

constexpr int kPlanThreads = 1024;

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
  __syncthreads();
  for (int base = 0; base < plan.rows; base += kPlanThreads) {
    const int s = base + threadIdx.x;
    int nseg = 0, st = 0, en = 0;
    if (s < plan.rows) {
      st = lower_bound_seq(seq_idx, L, s);
      en = max(st, lower_bound_seq(seq_idx, L, s + 1));
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
}

// ---------------------------------------------------------------------------
// segment combine: entry state of segment k = decay_{k-1} entry_{k-1} + local_{k-1}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void combine_kernel(ScanParams p, ScanPlan plan, char *ws) {
  const int row = blockIdx.x / p.H;
  const int h = blockIdx.x % p.H;
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
  const float *local = ws_f32(plan, ws, plan.ws_local_off);
  const float *ldec = ws_f32(plan, ws, plan.ws_decay_off);
  float *entry = ws_f32(plan, ws, plan.ws_entry_off);
  constexpr int kPer = kPN / 4 / kThreads;  // float4 per thread (8)
  float4 e[kPer];
  const float4 *init = p.init ? reinterpret_cast<const float4 *>(p.init + ((int64_t)row * p.H + h) * kPN)
                              : nullptr;
#pragma unroll
  for (int i = 0; i < kPer; ++i) e[i] = init ? init[i * kThreads + threadIdx.x] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 1; k < nseg; ++k) {
    const int prev = off + k - 1;
    if (off + k >= plan.items) break;
    const float d = __expf(ldec[(int64_t)prev * p.H + h]);
    const float4 *lp = reinterpret_cast<const float4 *>(local + ((int64_t)prev * p.H + h) * kPN);
    float4 *ep = reinterpret_cast<float4 *>(entry + ((int64_t)(off + k) * p.H + h) * kPN);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float4 l = lp[i * kThreads + threadIdx.x];
      e[i].x = fmaf(d, e[i].x, l.x);
      e[i].y = fmaf(d, e[i].y, l.y);
      e[i].z = fmaf(d, e[i].z, l.z);
      e[i].w = fmaf(d, e[i].w, l.w);
      ep[i * kThreads + threadIdx.x] = e[i];
    }
  }
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

ScanPlan make_scan_plan(const ScanParams &p, int seg_chunks) {
  ScanPlan plan{};
  plan.packed = p.seq_idx != nullptr;
  plan.rows = plan.packed ? p.num_seqs : p.batch;
  const int chunks_max = std::max(1, (p.L + kChunk - 1) / kChunk);
  if (seg_chunks <= 0) {
    // workgroup slots of one wave of launches: the bf16 kernel fits two per CU
    const long long slots = p.bf16 ? 2LL * kNumCU : (long long)kNumCU;
    const long long base = (long long)plan.rows * p.H;
    if (base >= slots) {
      seg_chunks = chunks_max;
    } else {
      const int factor = (int)((slots + base - 1) / base);
      seg_chunks = std::max(1, (chunks_max + factor - 1) / factor);
    }
  }
  seg_chunks = std::min(seg_chunks, chunks_max);
  plan.seg_len = seg_chunks * kChunk;
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
  if (plan.packed) off = align256(off + sizeof(int) * (4 * (size_t)plan.rows + 2 * (size_t)plan.items + 1));
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
  char *ws = reinterpret_cast<char *>(workspace);
  if (plan.packed) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p.seq_idx, p.L, plan, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long total = (long long)plan.items * p.H;
  const unsigned nblk = (unsigned)((total + kNumXCD - 1) / kNumXCD * kNumXCD);
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
    hipLaunchKernelGGL(combine_kernel, dim3(plan.rows * p.H), dim3(kThreads), 0, stream, p, plan, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.bf16) return launch_chunk_scan_bf16(p, plan, ws, nblk, true, stream);
  hipLaunchKernelGGL(chunk_scan_f32_kernel<true>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
  return hipGetLastError();
}

}  // namespace ssd
