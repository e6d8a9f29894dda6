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
// One launch, two kinds of workgroup per (row, head): kIB-row blocks of y
// (the kJB-token blocks j <= its rows are dealt to its four waves, each
// with its own tiles and its next block's loads in flight while it
// multiplies the current one) and kSP-row blocks of the final state.  Every workgroup recomputes the row's dt and cs
// (L softplus and one fp64 block scan).  Batch rows only (no seq_idx).
#include <cstddef>

#include "common.h"
#include "kernels.h"
#include "scan_items.h"

namespace ssd {

namespace {

constexpr int kT = 256;
constexpr int kIB = 16;   // y rows per workgroup
constexpr int kJB = 16;   // tokens per j block (one wave's step)
constexpr int kSP = 8;    // state rows per state workgroup
// B / C / h0 rows padded to 132 floats: 16-byte aligned, and lanes reading
// float4s of 16 different rows at one column fall in different bank groups
constexpr int kNP = kDState + 4;

struct WaveTiles {
  float B[kJB * kNP];        // B rows of the wave's current j block
  float X[kJB * kHeadDim];   // x rows of that block
  float M[kIB * kJB];        // masked C B^T tile
};
struct QuadSmem {
  double cs[kQuadMaxL];
  float dt[kQuadMaxL];
  float Cr[kIB * kNP];       // C rows of the y block
  WaveTiles w[kT / 64];      // one set per wave; after the j loop, the waves' partial y
  float H0[kHeadDim * kNP];  // initial state (y blocks)
};
static_assert(sizeof(WaveTiles) * (kT / 64) >= (kT / 64) * kIB * kHeadDim * sizeof(float), "partial y overlay");

// dt and the fp64 inclusive cumsum of dt A over the whole sequence
__device__ void row_cumsum(const ScanParams &p, int row, int h, QuadSmem &s) {
  const int tid = threadIdx.x;
  const float *dtg = reinterpret_cast<const float *>(p.dt) + (int64_t)row * p.dt_sb + h;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Ah = p.A[h];
  constexpr int per = kQuadMaxL / kT;  // tokens per thread
  double loc[per];
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int t = tid * per + k;
    float d = 0.f;
    if (t < p.L) d = softplus_f32(dtg[(int64_t)t * p.dt_st] + bias);
    if (t < kQuadMaxL) s.dt[t] = d;
    run += (double)(d * Ah);
    loc[k] = run;
  }
  // exclusive scan of the per-thread totals: waves by shuffles, then across waves
  double tot = run;
  const int lane = tid & 63, w = tid >> 6;
  double incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  __shared__ double wsum[kT / 64];
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  double before = incl - tot;
  for (int k = 0; k < w; ++k) before += wsum[k];
#pragma unroll
  for (int k = 0; k < per; ++k) s.cs[tid * per + k] = before + loc[k];
  __syncthreads();
}

__global__ __launch_bounds__(kT) void quad_scan_f32_kernel(ScanParams p, int nib, int nsb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  QuadSmem &s = *reinterpret_cast<QuadSmem *>(smem_raw);
  const int per_unit = nib + nsb;
  const int unit = blockIdx.x / per_unit, part = blockIdx.x % per_unit;
  const int row = unit / p.H, h = unit % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x;
  const int L = p.L;
  row_cumsum(p, row, h, s);
  const float *xg = reinterpret_cast<const float *>(p.x) + (int64_t)row * p.x_sb + h * kHeadDim;
  const float *Bg = reinterpret_cast<const float *>(p.B) + (int64_t)row * p.B_sb + g * kDState;
  const float *Cg = reinterpret_cast<const float *>(p.C) + (int64_t)row * p.C_sb + g * kDState;
  const float *h0 = p.init ? p.init + ((int64_t)row * p.H + h) * kPN : nullptr;

  if (part < nib) {
    // ---- y rows i0 .. i0 + kIB - 1 ----
    // Wave w takes the j blocks w, w + 4, ... on its own tiles (no workgroup
    // barrier in the loop: four independent chains of loads and products),
    // and the four partial sums are added at the end.
    const int i0 = part * kIB;
    for (int e = tid; e < kIB * kDState; e += kT) {
      const int i = e / kDState, n = e % kDState;
      s.Cr[i * kNP + n] = i0 + i < L ? Cg[(int64_t)(i0 + i) * p.C_st + n] : 0.f;
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    WaveTiles &T = s.w[wave];
    const int njb = min((i0 + kIB - 1) / kJB, (L - 1) / kJB) + 1;  // j blocks with j <= the last row
    // lane roles: CB rows ci = lane / 4, columns cj = 4 (lane % 4) .. + 3;
    //             y row yi = lane / 4, columns 16 (lane % 4) .. + 15
    const int ci = lane >> 2, cj = 4 * (lane & 3);
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.f;
    f32x4 rb[8], rx[4];
    auto fetch = [&](int jb) {
      const int j0 = jb * kJB;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = (lane + 64 * k) * 4, j = e / kDState, n = e % kDState;
        rb[k] = j0 + j < L ? *reinterpret_cast<const f32x4 *>(Bg + (int64_t)(j0 + j) * p.B_st + n) : f32x4{};
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = (lane + 64 * k) * 4, j = e / kHeadDim, q = e % kHeadDim;
        rx[k] = j0 + j < L ? *reinterpret_cast<const f32x4 *>(xg + (int64_t)(j0 + j) * p.x_st + q) : f32x4{};
      }
    };
    if (wave < njb) fetch(wave);
    for (int jb = wave; jb < njb; jb += kT / 64) {
      const int j0 = jb * kJB;
      // the block's B and x into this wave's tiles (the previous step's reads are done:
      // one wave's LDS accesses complete in order)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = (lane + 64 * k) * 4, j = e / kDState, n = e % kDState;
        *reinterpret_cast<f32x4 *>(&T.B[j * kNP + n]) = rb[k];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) *reinterpret_cast<f32x4 *>(&T.X[(lane + 64 * k) * 4]) = rx[k];
      if (jb + kT / 64 < njb) fetch(jb + kT / 64);  // the wave's next block, in flight during the products
      __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's tile writes are done
      __builtin_amdgcn_wave_barrier();
      // CB for rows ci, columns cj .. cj + 3
      float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int n = 0; n < kDState; n += 4) {
        const f32x4 cv = *reinterpret_cast<const f32x4 *>(&s.Cr[ci * kNP + n]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 bv = *reinterpret_cast<const f32x4 *>(&T.B[(cj + k) * kNP + n]);
          c4[k] = fmaf(cv[0], bv[0], fmaf(cv[1], bv[1], fmaf(cv[2], bv[2], fmaf(cv[3], bv[3], c4[k]))));
        }
      }
      const int i = i0 + ci;
      const double csi = i < L ? s.cs[i] : 0.0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = j0 + cj + k;
        T.M[ci * kJB + cj + k] = (j <= i && i < L) ? c4[k] * __expf((float)(csi - s.cs[j])) * s.dt[j] : 0.f;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
      // y[yi][16 (lane % 4) ..] += sum_j M[yi][j] x_j[..]
#pragma unroll 2
      for (int j = 0; j < kJB; ++j) {
        const float m = T.M[ci * kJB + j];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 xv = *reinterpret_cast<const f32x4 *>(&T.X[j * kHeadDim + cj * 4 + 4 * k]);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[4 * k + c] = fmaf(m, xv[c], acc[4 * k + c]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();  // every wave is done with its tiles: they now hold the partial y
    float *py = reinterpret_cast<float *>(&s.w[0]);  // [wave][kIB][kHeadDim]
#pragma unroll
    for (int k = 0; k < 16; ++k) py[(wave * kIB + ci) * kHeadDim + cj * 4 + k] = acc[k];
    if (h0)
      for (int e = tid; e < kPN; e += kT) s.H0[(e / kDState) * kNP + (e % kDState)] = h0[e];
    __syncthreads();
    // this thread's outputs: row ti, columns 4 tj .. 4 tj + 3
    const int ti = tid >> 4, tj = tid & 15;
    const int i = i0 + ti;
    if (i < L) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kT / 64; ++w) v += py[(w * kIB + ti) * kHeadDim + 4 * tj + c];
        o[c] = v;
      }
      if (h0) {
        float hsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int n = 0; n < kDState; n += 4) {
          const f32x4 cv = *reinterpret_cast<const f32x4 *>(&s.Cr[ti * kNP + n]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 hv = *reinterpret_cast<const f32x4 *>(&s.H0[(4 * tj + c) * kNP + n]);
            hsum[c] = fmaf(cv[0], hv[0], fmaf(cv[1], hv[1], fmaf(cv[2], hv[2], fmaf(cv[3], hv[3], hsum[c]))));
          }
        }
        const float ei = __expf((float)s.cs[i]);
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = fmaf(ei, hsum[c], o[c]);
      }
      const float Dh = p.D ? p.D[h] : 0.f;
      const f32x4 xi = *reinterpret_cast<const f32x4 *>(xg + (int64_t)i * p.x_st + 4 * tj);
      f32x4 out;
#pragma unroll
      for (int c = 0; c < 4; ++c) out[c] = fmaf(Dh, xi[c], o[c]);
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.y) + (int64_t)row * p.y_sb + (int64_t)i * p.y_st +
                                 h * kHeadDim + 4 * tj) = out;
    }
  } else {
    // ---- final-state rows p0 .. p0 + kSP - 1: S[q][n] = e^{cs_last} h0 + sum_j w_j x_j[q] B_j[n] ----
    // 128-token blocks of B and of x's kSP columns go to LDS in one round trip
    // each (every thread's loads independent), then 128 tokens of FMAs.
    // the y blocks' tiles are not used here: 128 x 128 B rows (unpadded) and
    // 128 x kSP weighted x values overlay them from Cr on
    float *sB = s.Cr;
    float *sw = s.Cr + 128 * kDState;
    static_assert(sizeof(QuadSmem) - offsetof(QuadSmem, Cr) >= (128 * kDState + 128 * kSP) * sizeof(float),
                  "state block tiles");
    const int p0 = (part - nib) * kSP;
    const int q = tid >> 5, n0 = 4 * (tid & 31);
    const double last = L > 0 ? s.cs[L - 1] : 0.0;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < L; t0 += 128) {
      f32x4 rb[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = (tid + k * kT) * 4, j = e / kDState, n = e % kDState;
        rb[k] = t0 + j < L ? *reinterpret_cast<const f32x4 *>(Bg + (int64_t)(t0 + j) * p.B_st + n) : f32x4{};
      }
      // token tid / 2, columns p0 + 4 (tid % 2) .. + 3 of x, weighted
      const int jw = tid >> 1, cw = 4 * (tid & 1);
      f32x4 xv = t0 + jw < L ? *reinterpret_cast<const f32x4 *>(xg + (int64_t)(t0 + jw) * p.x_st + p0 + cw) : f32x4{};
      __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
      for (int k = 0; k < 16; ++k) *reinterpret_cast<f32x4 *>(sB + (tid + k * kT) * 4) = rb[k];
      const float wj = t0 + jw < L ? __expf((float)(last - s.cs[t0 + jw])) * s.dt[t0 + jw] : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) sw[jw * kSP + cw + c] = wj * xv[c];
      __syncthreads();
      const int nj = min(128, L - t0);
#pragma unroll 4
      for (int j = 0; j < nj; ++j) {
        const float wq = sw[j * kSP + q];
        const f32x4 bv = *reinterpret_cast<const f32x4 *>(sB + j * kDState + n0);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(wq, bv[c], acc[c]);
      }
    }
    const int qq = p0 + q;
    f32x4 out;
    const float dec = __expf((float)last);
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = h0 ? fmaf(dec, h0[qq * kDState + n0 + c], acc[c]) : acc[c];
    *reinterpret_cast<f32x4 *>(p.final_state + ((int64_t)row * p.H + h) * kPN + qq * kDState + n0) = out;
  }
}

}  // namespace

size_t quad_lds_bytes() { return sizeof(QuadSmem); }

hipError_t launch_quad_scan_f32(const ScanParams &p, hipStream_t stream) {
  const int nib = (p.L + kIB - 1) / kIB;
  const int nsb = p.final_state ? kHeadDim / kSP : 0;
  const long long nblk = (long long)p.batch * p.H * (nib + nsb);
  if (nblk == 0) return hipSuccess;
  const size_t lds = sizeof(QuadSmem);
  hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void *>(quad_scan_f32_kernel), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quad_scan_f32_kernel, dim3((unsigned)nblk), dim3(kT), lds, stream, p, nib, nsb);
  return hipGetLastError();
}

}  // namespace ssd
