// Short fp32 sequences: the scan as one masked quadratic form, one launch.
//
// For a sequence short enough (L <= kQuadMaxL) the whole causal map is cheap
// as a masked matrix -- the state space duality with (linear) attention
// ("AI Engineering EP6", sec. 8 and 10):
//   y_i = sum_{j<=i} (C_i . B_j) e^{cs_i - cs_j} dt_j x_j + e^{cs_i} C_i h0^T + D x_i
//   S_L = e^{cs_last} h0 + sum_j e^{cs_last - cs_j} dt_j x_j B_j^T
// with cs_i = sum_{k<=i} dt_k A the cumulative log-decay from the sequence
// start.  cs is summed in fp64 and every difference cs_i - cs_j is taken in
// fp64 before the fp32 exponential, so the decays keep full fp32 accuracy
// however long the sequence is.
//
// Both products are dense contractions, so they run on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: fp32 products, fp32 sums -- no reduced
// precision anywhere).  The 16 x 16 accumulator of (B_j . C_i) holds, per
// lane, one column i and four rows j; that is exactly the operand layout
// the next product (masked tile times x) takes, so the masked tile never
// leaves the registers.
//
// One launch, 16-wave workgroups of two kinds per (row, head):
//  * y blocks of 16 rows: the block's C rows sit in LDS; its tiles j <= i
//    (16 tokens each) and the initial-state term (one task per 16 columns
//    of y) are dealt to the waves, every wave's tasks summed in its
//    registers, the waves' partial sums added in a fixed order through LDS;
//  * state blocks of 32 columns of S: x and the block's B columns are staged
//    through LDS in 64-token pieces (one coalesced 16-byte load per thread,
//    a piece ahead); each wave owns a 16 x 16 tile and one half of every
//    piece; the halves are added in a fixed order.
// Every workgroup recomputes the row's dt and cs (one softplus per thread
// and one fp64 block scan).  Batch rows only (no seq_idx).
#include "common.h"
#include "kernels.h"
#include "scan_items.h"

namespace ssd {

namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / 64;
constexpr int kR = 16;              // y rows / tokens / state rows per tile
constexpr int kPT = kHeadDim / kR;  // 16-column tiles of a y row
constexpr int kSN = 32;             // state columns per state block
constexpr int kSB = kDState / kSN;  // state blocks per (row, head)
constexpr int kCP = kDState + 4;    // padded C rows: 16-byte aligned, rows on distinct banks
constexpr int kYP = kHeadDim + 4;   // padded rows of a partial y tile
constexpr int kPc = 64;             // tokens per piece of a state block
constexpr int kXP = kHeadDim + 16;  // padded x rows of a piece (rows 16 banks apart)
constexpr int kBP = kSN + 16;       // padded B rows of a piece
static_assert(kQuadMaxL <= kT, "one token per thread in the cumsum");
static_assert(kPc * kHeadDim / 4 == kT && kPc * kSN / 4 <= kT, "one 16-byte load per thread and piece");

struct YSmem {
  float C[kR * kCP];                   // the block's C rows
  float red[(kWaves / 2) * kR * kYP];  // half of the waves' partial sums
};
struct StateSmem {
  float X[2][kPc * kXP];  // weighted x rows of a piece (double-buffered)
  float B[2][kPc * kBP];  // the block's B columns of a piece
  float red[(kWaves / 2) * kR * kR];
};
struct QuadSmem {
  double cs[kQuadMaxL];
  float dt[kQuadMaxL];  // y blocks: dt_j; state blocks: e^{cs_last - cs_j} dt_j
  union {
    YSmem y;
    StateSmem st;
  } u;
};

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// this thread's raw dt (token tid, clamped into the sequence: the cumsum
// ignores it past the end); loaded before anything else, so that the cumsum
// waits only for it and not for the loads issued after it.  Needs L >= 1.
__device__ __forceinline__ float load_dt(const ScanParams &p, int row, int h) {
  const float *dtg = reinterpret_cast<const float *>(p.dt) + (int64_t)row * p.dt_sb + h;
  return dtg[(int64_t)min((int)threadIdx.x, p.L - 1) * p.dt_st];
}

// A DPP move of a double (both 32-bit halves with the same control): lanes
// outside the pattern's rows, or reading outside their row with kBound, get 0.
template <int kCtrl, int kRowMask, bool kBound> __device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, kCtrl, kRowMask, 0xF, kBound);
  const unsigned hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), kCtrl, kRowMask, 0xF, kBound);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// Inclusive prefix sum over the 64 lanes of a wave: row shifts within each
// 16-lane row, then the row totals carried by row broadcasts (no LDS traffic).
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
  x += dpp_f64<0x111, 0xF, true>(x);   // row_shr:1
  x += dpp_f64<0x112, 0xF, true>(x);   // row_shr:2
  x += dpp_f64<0x114, 0xF, true>(x);   // row_shr:4
  x += dpp_f64<0x118, 0xF, true>(x);   // row_shr:8
  x += dpp_f64<0x142, 0xA, false>(x);  // row_bcast:15 -> rows 1, 3
  x += dpp_f64<0x143, 0xC, false>(x);  // row_bcast:31 -> rows 2, 3
  return x;
}

// dt and the fp64 inclusive cumsum of dt A over the whole sequence (one token per thread)
__device__ void row_cumsum(const ScanParams &p, int h, float raw_dt, QuadSmem &s) {
  const int tid = threadIdx.x;
  float d = 0.f;
  if (tid < p.L) d = softplus_f32(raw_dt + (p.dt_bias ? p.dt_bias[h] : 0.f));
  if (tid < kQuadMaxL) s.dt[tid] = d;
  const double v = (double)(d * p.A[h]);
  const int lane = tid & 63, w = tid >> 6;
  const double incl = wave_incl_scan_f64(v);
  __shared__ double wsum[kWaves];
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  double before = 0.0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {  // independent reads, summed in wave order
    const double ws = wsum[k];
    before += k < w ? ws : 0.0;
  }
  if (tid < kQuadMaxL) s.cs[tid] = before + incl;
  __syncthreads();
}

__global__ __launch_bounds__(kT) void quad_scan_f32_kernel(ScanParams p, int nib, int nsb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  QuadSmem &s = *reinterpret_cast<QuadSmem *>(smem_raw);
  // part-major order, state blocks first, then y blocks from the longest
  // (most tiles) to the shortest: the tail of the launch is the light work
  const int units = p.batch * p.H;
  const int part = blockIdx.x / units, unit = blockIdx.x % units;
  const int row = unit / p.H, h = unit % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int L = p.L;
  const float *xg = reinterpret_cast<const float *>(p.x) + (int64_t)row * p.x_sb + h * kHeadDim;
  const float *Bg = reinterpret_cast<const float *>(p.B) + (int64_t)row * p.B_sb + g * kDState;
  const float *Cg = reinterpret_cast<const float *>(p.C) + (int64_t)row * p.C_sb + g * kDState;
  const float *h0 = p.init ? p.init + ((int64_t)row * p.H + h) * kPN : nullptr;
  if (L == 0) {
    // no tokens (only state blocks exist): the final state is the initial
    // state, or zero
    const int n0 = part * kSN;
    for (int e = tid; e < kHeadDim * kSN; e += kT) {
      const int pp = e / kSN, n = n0 + e % kSN;
      p.final_state[((int64_t)row * p.H + h) * kPN + pp * kDState + n] = h0 ? h0[pp * kDState + n] : 0.f;
    }
    return;
  }
  const float raw_dt = load_dt(p, row, h);

  if (part >= nsb) {
    // ---------------- y rows i0 .. i0 + 15 ----------------
    const int ib = nib - 1 - (part - nsb);
    const int i0 = ib * kR;
    const int ntile = ib + 1;
    const int ntask = ntile + (h0 ? kPT : 0);
    // tiles in a rotated order, so that the workgroups of one launch do not
    // all start on the same rows of B and x
    const int rot = (unit * 7 + ib * 5) % ntile;
    auto tile_of = [&](int task) { return task + rot < ntile ? task + rot : task + rot - ntile; };
    // lane roles in a 16 x 16 x 4 product: operand row l16 and k slot kq;
    // accumulator rows 4 kq .. 4 kq + 3, column l16.  The state columns of
    // a row are split as n = 16 c + 4 kq + q (c < 8, q < 4): each load
    // instruction reads 64 contiguous bytes of a row per four lanes.
    //
    // A task is a tile (B rows and x rows of 16 tokens) or an initial-state
    // term (16 rows of h0); its operands are loaded one task ahead.
    f32x4 bq[8];
    float xo[kPT][4];  // x_{j0 + 4 kq + u}[16 pt + l16]: the second product's k slot kq, step u
    // (a wave with no task left loads nothing: a block's waves outnumber its
    // tasks up to the middle of the sequence, and every load costs the CU's
    // memory pipeline, which bounds this kernel)
    auto load_rows = [&](int task) {
      if (task < ntile) {
        const int jr = tile_of(task) * kR + l16;
#pragma unroll
        for (int c = 0; c < 8; ++c) bq[c] = jr < L ? ld4(Bg + (int64_t)jr * p.B_st + 16 * c + 4 * kq) : f32x4{};
      } else if (task < ntask) {
        const float *hrow = h0 + (16 * (task - ntile) + l16) * kDState + 4 * kq;
#pragma unroll
        for (int c = 0; c < 8; ++c) bq[c] = ld4(hrow + 16 * c);
      }
    };
    auto load_x = [&](int task) {
      if (task < ntile) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = tile_of(task) * kR + 4 * kq + u;
#pragma unroll
          for (int pt = 0; pt < kPT; ++pt) xo[pt][u] = j < L ? xg[(int64_t)j * p.x_st + 16 * pt + l16] : 0.f;
        }
      }
    };
    // loads in the order they are needed (they complete in order): dt, the
    // C rows (before the cumsum's barrier), then the first task's operands
    // and the epilogue's x value, whose latencies overlap the cumsum
    static_assert(kR * kDState / 4 <= kT, "one 16-byte piece of C per thread");
    const bool c_ld = tid < kR * kDState / 4;
    const int c_i = tid / (kDState / 4), c_n = 4 * (tid % (kDState / 4));
    const f32x4 c_val = (c_ld && i0 + c_i < L) ? ld4(Cg + (int64_t)(i0 + c_i) * p.C_st + c_n) : f32x4{};
    load_rows(wave);
    load_x(wave);
    const int ti = tid >> 6, tp = tid & 63;  // this thread's output: row ti, column tp
    const float x_self = i0 + ti < L ? xg[(int64_t)(i0 + ti) * p.x_st + tp] : 0.f;
    const float Dh = p.D ? p.D[h] : 0.f;
    if (c_ld) *reinterpret_cast<f32x4 *>(&s.u.y.C[c_i * kCP + c_n]) = c_val;
    row_cumsum(p, h, raw_dt, s);  // its barriers also publish the C rows

    const float *crow = &s.u.y.C[l16 * kCP + 4 * kq];  // C_{i0 + l16}, this lane's columns at 16 c
    f32x4 yacc[kPT];  // y[i0 + 4 kq + r][16 pt + l16]
#pragma unroll
    for (int pt = 0; pt < kPT; ++pt) yacc[pt] = f32x4{};
    for (int task = wave; task < ntask; task += kWaves) {
      const int next = task + kWaves;
      if (task < ntile) {
        const int j0 = tile_of(task) * kR;
        // G[j][i] = B_j . C_i (A operand: B row j0 + l16; B operand: C row i0 + l16)
        f32x4 gacc = f32x4{};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const f32x4 cv = ld4(crow + 16 * c);
#pragma unroll
          for (int q = 0; q < 4; ++q) gacc = mfma16(bq[c][q], cv[q], gacc);
        }
        load_rows(next);
        // this lane holds G[j0 + 4 kq + r][i0 + l16]: mask, decay, dt
        const int i = i0 + l16;
        const double csi = s.cs[min(i, kQuadMaxL - 1)];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 4 * kq + r;
          gacc[r] = (j <= i && i < L) ? gacc[r] * __expf((float)(csi - s.cs[j])) * s.dt[j] : 0.f;
        }
        // y[i][p] += sum_j M[i][j] x_j[p]: step u takes tokens j0 + 4 k + u (k slot k),
        // whose M values this lane holds as gacc[u] (row i0 + l16, k slot kq)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int pt = 0; pt < kPT; ++pt) yacc[pt] = mfma16(gacc[u], xo[pt][u], yacc[pt]);
        load_x(next);
      } else {
        // initial-state term for columns 16 pt .. 16 pt + 15: e^{cs_i} C_i . h0[p]
        // (A operand: C row i0 + l16; B operand: h0 row 16 pt + l16)
        const int pt = task - ntile;
        f32x4 t = f32x4{};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const f32x4 cv = ld4(crow + 16 * c);
#pragma unroll
          for (int q = 0; q < 4; ++q) t = mfma16(cv[q], bq[c][q], t);
        }
        load_rows(next);
        load_x(next);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + 4 * kq + r;
          t[r] *= i < L ? __expf((float)s.cs[i]) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < kPT; ++q)
          if (q == pt) yacc[q] += t;
      }
    }
    // the waves' partial sums, added in a fixed order: waves 8..15 into 0..7,
    // then the eight sums of waves 0..7 per output
    auto put = [&](int slot) {
#pragma unroll
      for (int pt = 0; pt < kPT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s.u.y.red[(slot * kR + 4 * kq + r) * kYP + 16 * pt + l16] = yacc[pt][r];
    };
    if (wave >= kWaves / 2) put(wave - kWaves / 2);
    __syncthreads();
    if (wave < kWaves / 2) {
#pragma unroll
      for (int pt = 0; pt < kPT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[pt][r] += s.u.y.red[(wave * kR + 4 * kq + r) * kYP + 16 * pt + l16];
    }
    __syncthreads();
    if (wave < kWaves / 2) put(wave);
    __syncthreads();
    const int i = i0 + ti;
    if (i < L) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves / 2; ++w) v += s.u.y.red[(w * kR + ti) * kYP + tp];
      v = fmaf(Dh, x_self, v);
      reinterpret_cast<float *>(p.y)[(int64_t)row * p.y_sb + (int64_t)i * p.y_st + h * kHeadDim + tp] = v;
    }
  } else {
    // ---------------- final-state columns n0 .. n0 + 31 ----------------
    // S[p][n] = e^{cs_last} h0[p][n] + sum_j w_j x_j[p] B_j[n], w_j = e^{cs_last - cs_j} dt_j.
    // The workgroup walks the tokens in 64-token pieces: each thread loads one
    // 16-byte piece of x (and of the block's B columns) a piece ahead, stores
    // it (x weighted by w_j) into a double-buffered LDS tile, and the waves
    // multiply from LDS.  Wave roles: rows 16 pt .., columns n0 + 16 nt ..,
    // tokens 32 half .. 32 half + 31 of every piece (step u: tokens 4 u ..
    // 4 u + 3, k slot kq takes token 4 u + kq).
    StateSmem &st = s.u.st;
    const int n0 = part * kSN;
    const int pt = wave & 3, nt = (wave >> 2) & 1, half = wave >> 3;
    const int xt = tid >> 4, xc = 4 * (tid & 15);  // this thread's x load: token, columns
    const int bt = tid >> 3, bc = 4 * (tid & 7);   // its B load (threads below kPc * kSN / 4)
    const bool stores_b = tid < kPc * kSN / 4;
    f32x4 xv, bv;
    auto load_piece = [&](int t0) {
      const int jx = t0 + xt, jb = t0 + bt;
      xv = jx < L ? ld4(xg + (int64_t)jx * p.x_st + xc) : f32x4{};
      bv = (stores_b && jb < L) ? ld4(Bg + (int64_t)jb * p.B_st + n0 + bc) : f32x4{};
    };
    load_piece(0);
    float h0v[4] = {0.f, 0.f, 0.f, 0.f};
    if (h0 && half == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) h0v[r] = h0[(16 * pt + 4 * kq + r) * kDState + n0 + 16 * nt + l16];
    }
    row_cumsum(p, h, raw_dt, s);
    const double last = L > 0 ? s.cs[L - 1] : 0.0;
    if (tid < L) s.dt[tid] = __expf((float)(last - s.cs[tid])) * s.dt[tid];
    __syncthreads();
    f32x4 acc = f32x4{};
    for (int t0 = 0, buf = 0; t0 < L; t0 += kPc, buf ^= 1) {
      // this piece's tiles (the buffer was last read two pieces ago, before
      // the previous piece's barrier)
      const float w = s.dt[min(t0 + xt, kQuadMaxL - 1)];  // 0 past the end: xv is 0 there too
      *reinterpret_cast<f32x4 *>(&st.X[buf][xt * kXP + xc]) = xv * w;
      if (stores_b) *reinterpret_cast<f32x4 *>(&st.B[buf][bt * kBP + bc]) = bv;
      __syncthreads();
      if (t0 + kPc < L) load_piece(t0 + kPc);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jl = 32 * half + 4 * u + kq;
        acc = mfma16(st.X[buf][jl * kXP + 16 * pt + l16], st.B[buf][jl * kBP + 16 * nt + l16], acc);
      }
    }
    // this lane holds S[16 pt + 4 kq + r][n0 + 16 nt + l16] over one half of every piece
    const int slot = wave & 7;
    if (half == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st.red[(slot * kR + 4 * kq + r) * kR + l16] = acc[r];
    }
    __syncthreads();
    if (half == 0) {
      const float dec = __expf((float)last);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pp = 16 * pt + 4 * kq + r, n = n0 + 16 * nt + l16;
        const float v = acc[r] + st.red[(slot * kR + 4 * kq + r) * kR + l16];
        p.final_state[((int64_t)row * p.H + h) * kPN + pp * kDState + n] = fmaf(dec, h0v[r], v);
      }
    }
  }
}

}  // namespace

hipError_t launch_quad_scan_f32(const ScanParams &p, hipStream_t stream) {
  const int nib = (p.L + kR - 1) / kR;
  const int nsb = p.final_state ? kSB : 0;
  const long long nblk = (long long)p.batch * p.H * (nib + nsb);
  if (nblk == 0) return hipSuccess;
  const size_t lds = sizeof(QuadSmem);
  hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void *>(quad_scan_f32_kernel), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quad_scan_f32_kernel, dim3((unsigned)nblk), dim3(kT), lds, stream, p, nib, nsb);
  return hipGetLastError();
}

}  // namespace ssd
