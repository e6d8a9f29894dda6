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

namespace ssd {

namespace {

constexpr int kThreads = 256;
constexpr int kPN = kHeadDim * kDState;

// ---------------------------------------------------------------------------
// Work items
// ---------------------------------------------------------------------------
struct Item {
  int row, k, tok0, tok1, first, last, item;
  int64_t boff;  // batch row used for strides (0 in packed mode)
};

struct PlanView {
  const int *seq_start, *seq_end, *seq_nseg, *seq_off, *item_seq, *item_k, *n_items;
};

__device__ __forceinline__ PlanView plan_view(const ScanPlan &plan, const char *ws) {
  const int *b = reinterpret_cast<const int *>(ws + plan.ws_plan_off);
  PlanView v;
  v.seq_start = b;
  v.seq_end = b + plan.rows;
  v.seq_nseg = b + 2 * plan.rows;
  v.seq_off = b + 3 * plan.rows;
  v.item_seq = b + 4 * plan.rows;
  v.item_k = v.item_seq + plan.items;
  v.n_items = v.item_k + plan.items;
  return v;
}

__device__ __forceinline__ bool get_item(const ScanParams &p, const ScanPlan &plan,
                                         const char *ws, int item, Item &it) {
  it.item = item;
  if (!plan.packed) {
    it.row = item / plan.nseg;
    it.k = item % plan.nseg;
    it.tok0 = it.k * plan.seg_len;
    it.tok1 = min(p.L, it.tok0 + plan.seg_len);
    it.first = it.k == 0;
    it.last = it.k == plan.nseg - 1;
    it.boff = it.row;
    return true;
  }
  const PlanView v = plan_view(plan, ws);
  if (item >= *v.n_items) return false;
  it.row = v.item_seq[item];
  it.k = v.item_k[item];
  const int start = v.seq_start[it.row], end = v.seq_end[it.row];
  it.tok0 = start + it.k * plan.seg_len;
  it.tok1 = min(end, it.tok0 + plan.seg_len);
  it.first = it.k == 0;
  it.last = it.k == v.seq_nseg[it.row] - 1;
  it.boff = 0;
  return true;
}

// blockIdx -> (item, head): XCD x gets a contiguous range of the work list,
// ordered item-major, then group, then head.
__device__ __forceinline__ bool map_workgroup(const ScanParams &p, const ScanPlan &plan, int &item,
                                              int &h, int &g) {
  const int total = plan.items * p.H;
  const int per_xcd = gridDim.x / kNumXCD;
  const int w = (blockIdx.x % kNumXCD) * per_xcd + blockIdx.x / kNumXCD;
  if (w >= total) return false;
  const int hpg = p.H / p.G;
  const int hl = w % hpg;
  const int t = w / hpg;
  g = t % p.G;
  item = t / p.G;
  h = g * hpg + hl;
  return true;
}

__device__ __forceinline__ float *ws_f32(const ScanPlan &plan, char *ws, size_t off) {
  return reinterpret_cast<float *>(ws + off);
}

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
// bf16 path: fused MFMA chunk kernel
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// (lo16(a), lo16(b)) or (hi16(a), hi16(b)) packed into one dword: one v_perm_b32.
__device__ __forceinline__ uint32_t pair16(uint32_t a, uint32_t b, int hi) {
  return __builtin_amdgcn_perm(b, a, hi ? 0x07060302u : 0x05040100u);
}

// LDS tiles: rows of 128 bf16 padded to 136 (272 B = 17 x 16 B), so MFMA
// operand reads -- consecutive lanes on consecutive rows -- are conflict-free.
// The transposed tiles (feature-major) are written by lanes 8 rows apart;
// rotating the row order inside each group of 8 (prow) makes those writes
// conflict-free too, while keeping every column offset a compile-time
// immediate for the reads.
constexpr int kRS = 136;
__device__ __forceinline__ int prow(int r) { return (r & ~7) | ((r + (r >> 3)) & 7); }

struct SmemBF16 {
  bf16_t B[kChunk * kRS];       // B[j][n]                 (operand of C B^T)
  bf16_t Bt[kDState * kRS];     // B^T[n][j], row prow(n)   (operand of the chunk state)
  bf16_t Xt[kHeadDim * kRS];    // x^T[p][j], row prow(p)   (operand of the intra-chunk product)
  bf16_t Xw[kHeadDim * kRS];    // (w_j x_j)^T[p][j], row prow(p)
  bf16_t H[kHeadDim * kRS];     // running state H[p][n] rounded to bf16
  float cs[2][kChunk];          // per-chunk vectors, double-buffered one chunk ahead
  float dt[2][kChunk];
  float w[2][kChunk];
  float v[2][kChunk];
  float misc[2][2];             // exp(cs_last), cs_last
};

// Chunk-state tiles (rows n-block nb, cols p-block pb of H^T) owned by each
// wave.  In the full pass wave w also owns output rows [32w, 32w+32) and
// its w+1 causal C B^T tiles, so the state tiles are dealt 4/3/1/0 to even
// out the MFMA count per wave (60/64/60/64 of 248 per chunk).  The
// state-only pre-pass deals them 2/2/2/2.
constexpr int kNSFull[4] = {4, 3, 1, 0};
constexpr int kNbFull[4][4] = {{0, 0, 1, 1}, {2, 2, 3, 0}, {3, 0, 0, 0}, {0, 0, 0, 0}};
constexpr int kPbFull[4][4] = {{0, 1, 0, 1}, {0, 1, 0, 0}, {1, 0, 0, 0}, {0, 0, 0, 0}};

template <bool kFull, int W> struct Tiles {
  static constexpr int NS = kFull ? kNSFull[W] : 2;
  static constexpr int NCB = kFull ? W + 1 : 0;
  __device__ static constexpr int nb(int t) { return kFull ? kNbFull[W][t] : W; }
  __device__ static constexpr int pb(int t) { return kFull ? kPbFull[W][t] : t; }
  __device__ static constexpr bool uses_pb(int q) {
    for (int t = 0; t < NS; ++t)
      if (pb(t) == q) return true;
    return false;
  }
};

template <bool kFull, int W>
__device__ __forceinline__ void chunk_scan_wave(const ScanParams &p, const ScanPlan &plan, char *ws,
                                                const Item &it, int item, int h, int g, SmemBF16 &sm) {
  using T = Tiles<kFull, W>;
  constexpr int NS = T::NS;
  constexpr int NCB = T::NCB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const bf16_t *xg = reinterpret_cast<const bf16_t *>(p.x) + it.boff * p.x_sb + h * kHeadDim;
  const bf16_t *Bg = reinterpret_cast<const bf16_t *>(p.B) + it.boff * p.B_sb + g * kDState;
  const bf16_t *Cg = reinterpret_cast<const bf16_t *>(p.C) + it.boff * p.C_sb + g * kDState;
  const bf16_t *dtg = reinterpret_cast<const bf16_t *>(p.dt) + it.boff * p.dt_sb + h;
  bf16_t *yg = reinterpret_cast<bf16_t *>(p.y) + it.boff * p.y_sb + h * kHeadDim;
  const uint32_t xst = (uint32_t)p.x_st, bst = (uint32_t)p.B_st, cst = (uint32_t)p.C_st;
  const uint32_t dst_ = (uint32_t)p.dt_st, yst = (uint32_t)p.y_st;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;

  // global -> LDS staging: x as 4 tokens x 8 features, B as 8 tokens x 8 features per thread
  const int xa = tid & 7, xj0 = 4 * (tid >> 3);
  const int ba = tid & 15, bj0 = 8 * (tid >> 4);
  const int ci = 32 * W + l32;  // this lane's chunk row i (full pass)

  u32x4 xr[4], br[8], cf[8];
  uint32_t draw = 0;  // wave 0: raw bf16 dt of tokens 2 lane, 2 lane + 1

  // Loads never branch: rows past the segment end are clamped to its last
  // row.  Their values are finite and every use is cancelled exactly
  // (dt = 0 past the end, and output rows past the end are not stored).
  auto load_c = [&](int c0, int nv) {
    if (kFull) {
      const bf16_t *crow = Cg + (int64_t)c0 * p.C_st + (uint32_t)min(ci, nv - 1) * cst + 8 * hh;
#pragma unroll
      for (int s = 0; s < 8; ++s) cf[s] = *reinterpret_cast<const u32x4 *>(crow + 16 * s);
    }
  };
  auto load_chunk = [&](int c0, int nv) {
    const int last = nv - 1;
    const bf16_t *xc = xg + (int64_t)c0 * p.x_st;
    const bf16_t *bc = Bg + (int64_t)c0 * p.B_st;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      xr[r] = *reinterpret_cast<const u32x4 *>(xc + (uint32_t)min(xj0 + r, last) * xst + 8 * xa);
#pragma unroll
    for (int r = 0; r < 8; ++r)
      br[r] = *reinterpret_cast<const u32x4 *>(bc + (uint32_t)min(bj0 + r, last) * bst + 8 * ba);
    if (W == 0) {
      const bf16_t *dc = dtg + (int64_t)c0 * p.dt_st;
      const uint32_t lo = dc[(uint32_t)min(2 * lane, last) * dst_];
      const uint32_t hi = dc[(uint32_t)min(2 * lane + 1, last) * dst_];
      draw = lo | (hi << 16);
    }
  };

  // registers -> LDS for one chunk whose per-token vectors sit in buffer `buf`
  auto store_chunk = [&](int buf) {
    const float4 w4 = *reinterpret_cast<const float4 *>(&sm.w[buf][xj0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = prow(8 * xa + e);
      if (kFull) {
        u32x2 v;
        v[0] = pair16(xr[0][e >> 1], xr[1][e >> 1], e & 1);
        v[1] = pair16(xr[2][e >> 1], xr[3][e >> 1], e & 1);
        *reinterpret_cast<u32x2 *>(&sm.Xt[r * kRS + xj0]) = v;
      }
      const int sh = (e & 1) ? 0 : 16;
      const float x0 = __uint_as_float((xr[0][e >> 1] << sh) & 0xFFFF0000u);
      const float x1 = __uint_as_float((xr[1][e >> 1] << sh) & 0xFFFF0000u);
      const float x2 = __uint_as_float((xr[2][e >> 1] << sh) & 0xFFFF0000u);
      const float x3 = __uint_as_float((xr[3][e >> 1] << sh) & 0xFFFF0000u);
      u32x2 vw;
      vw[0] = pack2_bf16(x0 * w4.x, x1 * w4.y);
      vw[1] = pack2_bf16(x2 * w4.z, x3 * w4.w);
      *reinterpret_cast<u32x2 *>(&sm.Xw[r * kRS + xj0]) = vw;
    }
    if (kFull) {
#pragma unroll
      for (int r = 0; r < 8; ++r) *reinterpret_cast<u32x4 *>(&sm.B[(bj0 + r) * kRS + 8 * ba]) = br[r];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pair16(br[2 * q][e >> 1], br[2 * q + 1][e >> 1], e & 1);
      *reinterpret_cast<u32x4 *>(&sm.Bt[prow(8 * ba + e) * kRS + bj0]) = v;
    }
  };

  auto run_dt = [&](int nv, int buf) {
    if (W == 0)
      chunk_dt(lo_bf16(draw), hi_bf16(draw), 2 * lane, nv, bias, Ah, sm.cs[buf], sm.dt[buf], sm.w[buf],
               sm.misc[buf], kFull ? sm.v[buf] : nullptr);
  };

  // entry state -> this wave's H^T tiles (rows n = 32 nb + 8q + 4hh + 0..3, col p = 32 pb + l32)
  f32x16 hs[NS > 0 ? NS : 1];
  const float *entry = nullptr;
  if (kFull) {
    if (it.first) entry = p.init ? p.init + ((int64_t)it.row * p.H + h) * kPN : nullptr;
    else entry = ws_f32(plan, ws, plan.ws_entry_off) + ((int64_t)item * p.H + h) * kPN;
  }
#pragma unroll
  for (int t = 0; t < NS; ++t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (entry)
        v = *reinterpret_cast<const float4 *>(entry + (32 * T::pb(t) + l32) * kDState + 32 * T::nb(t) + 8 * q + 4 * hh);
      hs[t][4 * q + 0] = v.x; hs[t][4 * q + 1] = v.y;
      hs[t][4 * q + 2] = v.z; hs[t][4 * q + 3] = v.w;
    }
  }
  auto write_state_lds = [&]() {
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 v;
        v[0] = pack2_bf16(hs[t][4 * q], hs[t][4 * q + 1]);
        v[1] = pack2_bf16(hs[t][4 * q + 2], hs[t][4 * q + 3]);
        *reinterpret_cast<u32x2 *>(&sm.H[(32 * T::pb(t) + l32) * kRS + 32 * T::nb(t) + 8 * q + 4 * hh]) = v;
      }
  };

  float logdecay = 0.f;
  const int ntok = it.tok1 - it.tok0;
  if (ntok > 0) {
    load_chunk(it.tok0, min(kChunk, ntok));
    load_c(it.tok0, min(kChunk, ntok));
    if (kFull) write_state_lds();
    run_dt(min(kChunk, ntok), 0);
    __syncthreads();
    store_chunk(0);
    __syncthreads();
  }

  // physical row of logical row 32 k + l32 of a transposed tile: 32 k + pr[k & 1]
  const int pr0 = prow(l32), pr1 = prow(32 + l32) - 32;
#define PROW(k) (32 * (k) + (((k) & 1) ? pr1 : pr0))
  int buf = 0;
  for (int c0 = it.tok0; c0 < it.tok1; c0 += kChunk, buf ^= 1) {
    const int nv = min(kChunk, it.tok1 - c0);
    const int c1 = c0 + kChunk;
    const bool has_next = c1 < it.tok1;
    // Prefetch the next chunk into registers.  The load is unconditional (the
    // last chunk re-reads itself): a conditional load would make the
    // compiler join the registers at the branch and wait for them there.
    const int cn = has_next ? c1 : c0;
    const int nvn = has_next ? min(kChunk, it.tok1 - c1) : nv;
    load_chunk(cn, nvn);

    const float dec = sm.misc[buf][0];
    logdecay += sm.misc[buf][1];
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) hs[t][r] *= dec;

    f32x16 G[NCB > 0 ? NCB : 1];
    f32x16 yo[2], yd[2];
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) G[jb] = f32x16{};
    if (kFull) {
      yo[0] = f32x16{}; yo[1] = f32x16{};
      yd[0] = f32x16{}; yd[1] = f32x16{};
    }

    // One pass over the 8 k-steps feeds every independent accumulator chain
    // of this wave: the chunk-state tiles (K = tokens), the causal C B^T
    // tiles and the state->output tiles (K = d_state).  Operand fragments
    // are double-buffered: the LDS reads of step s+1 are issued before the
    // MFMAs of step s, so each MFMA finds its operands already in registers.
    constexpr int NX = (T::uses_pb(0) ? 1 : 0) + (T::uses_pb(1) ? 1 : 0);
    constexpr int NF = NX + NS + (kFull ? NCB + 2 : 0);  // fragments per k-step
    bf16x8 fr[2][NF > 0 ? NF : 1];
    auto load_frags = [&](int s, bf16x8 *f) {
      const int col = 16 * s + 8 * hh;
      int k = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (T::uses_pb(q)) f[k++] = *reinterpret_cast<const bf16x8 *>(&sm.Xw[PROW(q) * kRS + col]);
#pragma unroll
      for (int t = 0; t < NS; ++t)
        f[k++] = *reinterpret_cast<const bf16x8 *>(&sm.Bt[PROW(T::nb(t)) * kRS + col]);
      if (kFull) {
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
          f[k++] = *reinterpret_cast<const bf16x8 *>(&sm.B[(32 * jb + l32) * kRS + col]);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          f[k++] = *reinterpret_cast<const bf16x8 *>(&sm.H[(32 * q + l32) * kRS + col]);
      }
    };
    auto mfma_step = [&](int s, const bf16x8 *f) {
      int k = 0;
      bf16x8 xw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (T::uses_pb(q)) xw[q] = f[k++];
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        hs[t] = mfma32(f[k++], xw[T::pb(t)], hs[t]);
      }
      if (kFull) {
        const bf16x8 cb = as_bf16x8(cf[s]);
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb) G[jb] = mfma32(f[k++], cb, G[jb]);
#pragma unroll
        for (int q = 0; q < 2; ++q) yo[q] = mfma32(f[k++], cb, yo[q]);
      }
    };
    load_frags(0, fr[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < 7) load_frags(s + 1, fr[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(s, fr[s & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the C fragments of this chunk are dead: fetch the next chunk's now
    load_c(cn, nvn);

    if (kFull) {
      // y^T[p][i] = exp(cs_i) (H_prev C_i)[p]  +  sum_j x[j][p] M[j][i]
      const float cs_i = sm.cs[buf][ci];
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb) {
        // decay mask and dt (D on the diagonal) -> bf16 operand (rows j, col i)
        bf16x8 Mb[2];
        if (jb < W) {
          // all j < i: exp(cs_i - cs_j) = exp(cs_i - cs_r) exp(cs_r - cs_j), r the
          // block's last row; both exponents are <= 0
          const float u = __expf(cs_i - sm.cs[buf][32 * jb + 31]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v4 = *reinterpret_cast<const float4 *>(&sm.v[buf][32 * jb + 8 * q + 4 * hh]);
            const float vj[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int r = 4 * q + t;
              Mb[r >> 3][r & 7] = (__bf16)(G[jb][r] * (u * vj[t]));
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int jq = 32 * jb + 8 * q + 4 * hh;
            const float4 csj = *reinterpret_cast<const float4 *>(&sm.cs[buf][jq]);
            const float4 dtj = *reinterpret_cast<const float4 *>(&sm.dt[buf][jq]);
            const float cj[4] = {csj.x, csj.y, csj.z, csj.w};
            const float dj[4] = {dtj.x, dtj.y, dtj.z, dtj.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int r = 4 * q + t;
              const int j = jq + t;
              const float gv = G[jb][r];
              float m = gv * __expf(fminf(cs_i - cj[t], 0.f)) * dj[t];
              m = j < ci ? m : (j == ci ? fmaf(gv, dj[t], Dh) : 0.f);
              Mb[r >> 3][r & 7] = (__bf16)m;
            }
          }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const bf16_t *row = &sm.Xt[PROW(q) * kRS + 32 * jb + 16 * s + 4 * hh];
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(row);
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + 8);
            const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
            yd[q] = mfma32(as_bf16x8(av), Mb[s], yd[q]);
          }
        }
      }
      // y rows i < nv: this lane holds p = 32q + 8r4 + 4hh + 0..3 of token c0 + ci
      if (ci < nv) {
        const float ecs = __expf(cs_i);
        bf16_t *yrow = yg + (int64_t)c0 * p.y_st + (uint32_t)ci * yst;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            u32x2 v;
            v[0] = pack2_bf16(fmaf(ecs, yo[q][4 * r4], yd[q][4 * r4]), fmaf(ecs, yo[q][4 * r4 + 1], yd[q][4 * r4 + 1]));
            v[1] = pack2_bf16(fmaf(ecs, yo[q][4 * r4 + 2], yd[q][4 * r4 + 2]), fmaf(ecs, yo[q][4 * r4 + 3], yd[q][4 * r4 + 3]));
            *reinterpret_cast<u32x2 *>(yrow + 32 * q + 8 * r4 + 4 * hh) = v;
          }
      }
    }
    if (has_next) run_dt(nvn, buf ^ 1);  // next chunk's dt / cumsum into the other buffer

    __syncthreads();  // every wave is done reading this chunk's LDS
    if (kFull) write_state_lds();
    if (has_next) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // outputs of the segment
  float *dst = nullptr;
  if (kFull) {
    if (it.last && p.final_state) dst = p.final_state + ((int64_t)it.row * p.H + h) * kPN;
  } else {
    dst = ws_f32(plan, ws, plan.ws_local_off) + ((int64_t)item * p.H + h) * kPN;
    if (tid == 0) ws_f32(plan, ws, plan.ws_decay_off)[(int64_t)item * p.H + h] = logdecay;
  }
  if (dst) {
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(dst + (32 * T::pb(t) + l32) * kDState + 32 * T::nb(t) + 8 * q + 4 * hh) =
            make_float4(hs[t][4 * q], hs[t][4 * q + 1], hs[t][4 * q + 2], hs[t][4 * q + 3]);
  }
}

#undef PROW

template <bool kFull>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_bf16_kernel(ScanParams p, ScanPlan plan,
                                                                      char *ws) {
  __shared__ __attribute__((aligned(16))) SmemBF16 sm;
  int item, h, g;
  if (!map_workgroup(p, plan, item, h, g)) return;
  Item it;
  if (!get_item(p, plan, ws, item, it)) return;
  if (!kFull && it.last) return;  // the pre-pass only needs segments that have a successor
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: chunk_scan_wave<kFull, 0>(p, plan, ws, it, item, h, g, sm); break;
    case 1: chunk_scan_wave<kFull, 1>(p, plan, ws, it, item, h, g, sm); break;
    case 2: chunk_scan_wave<kFull, 2>(p, plan, ws, it, item, h, g, sm); break;
    default: chunk_scan_wave<kFull, 3>(p, plan, ws, it, item, h, g, sm); break;
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
    const long long base = (long long)plan.rows * p.H;
    if (base >= kNumCU) {
      seg_chunks = chunks_max;
    } else {
      const int factor = (int)((kNumCU + base - 1) / base);
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
    if (p.bf16) hipLaunchKernelGGL(chunk_scan_bf16_kernel<false>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
    else hipLaunchKernelGGL(chunk_scan_f32_kernel<false>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(plan.rows * p.H), dim3(kThreads), 0, stream, p, plan, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.bf16) hipLaunchKernelGGL(chunk_scan_bf16_kernel<true>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
  else hipLaunchKernelGGL(chunk_scan_f32_kernel<true>, dim3(nblk), dim3(kThreads), 0, stream, p, plan, ws);
  return hipGetLastError();
}

}  // namespace ssd
