// MIMO decode step (Mamba-3's multi-input multi-output SSM, optionally with
// the exponential-trapezoidal input term) on gfx950.
//
// "Mamba-3: an inference-first state space model": MIMO widens B and C to
// rank R per head, adding parallel work to each update at almost no extra
// decode cost, and an exponential-trapezoidal discretization gives a more
// general recurrence.  Per head, with a = exp(dt A), state S (P x N):
//   Euler:        S <- a S + dt X B^T
//   trapezoidal:  S <- a S + (1 - lam) dt a Xp B_p^T + lam dt X B^T
//   Y = S C + D X                                   (X, Y: P x R; B, C: N x R)
// where Xp, B_p are the previous token's X and B, kept as decode state.
//
// Like the single-input step this is a stream over the fp32 state (read and
// written once, 16-byte non-temporal accesses); R only multiplies the
// arithmetic per state value (2R or 4R fused multiply-adds and R row
// reductions), which stays far below what the HBM stream leaves room for.
// One workgroup owns one (batch row, group): X, B, C (and the previous
// inputs) of the group go to LDS once; each lane keeps its four state
// columns' rows of B, C (and B_p) in registers for every head of the group;
// each wave streams one head's 32 KiB of state at a time, two rows per load.
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

// 16 waves for ranks 1 and 2; 8 waves (two heads each, 256 registers per
// lane) for ranks 4 and 8, whose rows of B, C and B_p take 12 R registers.
template <int R> constexpr int threads_for() { return R <= 2 ? 1024 : 512; }

template <typename T, int R, bool kTrap>
__global__ __launch_bounds__(threads_for<R>()) void decode_mimo_kernel(MimoParams p) {
  constexpr int kThreads = threads_for<R>();
  extern __shared__ float smem[];
  const int b = blockIdx.x / p.G;
  const int g = blockIdx.x % p.G;
  const int hpg = p.H / p.G;
  const int nxr = hpg * kHeadDim * R;  // the group's X values
  float *sx = smem;                     // [hpg][P][R]
  float *spx = sx + nxr;                // [hpg][P][R] previous X (trapezoid)
  float *sy = spx + (kTrap ? nxr : 0);  // [hpg][P][R]
  float *sB = sy + nxr;                 // [N][R]
  float *sC = sB + kDState * R;
  float *spB = sC + kDState * R;        // [N][R] previous B (trapezoid)
  float *scoef = spB + (kTrap ? kDState * R : 0);  // [hpg][3]: a, lam dt, (1 - lam) dt a

  const T *xg = reinterpret_cast<const T *>(p.x) + (int64_t)b * p.x_sb + (int64_t)g * nxr;
  const T *Bg = reinterpret_cast<const T *>(p.B) + (int64_t)b * p.B_sb + (int64_t)g * kDState * R;
  const T *Cg = reinterpret_cast<const T *>(p.C) + (int64_t)b * p.C_sb + (int64_t)g * kDState * R;
  T *pxg = kTrap ? reinterpret_cast<T *>(p.prev_x) + ((int64_t)b * p.H + (int64_t)g * hpg) * kHeadDim * R : nullptr;
  T *pBg = kTrap ? reinterpret_cast<T *>(p.prev_B) + ((int64_t)b * p.G + g) * kDState * R : nullptr;
  for (int e = threadIdx.x; e < nxr; e += kThreads) {
    sx[e] = to_f32<T>(xg[e]);
    if (kTrap) spx[e] = to_f32<T>(pxg[e]);
  }
  for (int e = threadIdx.x; e < kDState * R; e += kThreads) {
    sB[e] = to_f32<T>(Bg[e]);
    sC[e] = to_f32<T>(Cg[e]);
    if (kTrap) spB[e] = to_f32<T>(pBg[e]);
  }
  const T *dtp = reinterpret_cast<const T *>(p.dt) + (int64_t)b * p.dt_sb;
  const T *lp = (kTrap && p.lam) ? reinterpret_cast<const T *>(p.lam) + (int64_t)b * p.lam_sb : nullptr;
  for (int hl = threadIdx.x; hl < hpg; hl += kThreads) {
    const int h = g * hpg + hl;
    const float dt = softplus_f32(to_f32<T>(dtp[h]) + (p.dt_bias ? p.dt_bias[h] : 0.f));
    const float a = __expf(dt * p.A[h]);
    const float lam = kTrap ? (lp ? to_f32<T>(lp[h]) : 0.5f) : 1.f;
    scoef[3 * hl] = a;
    scoef[3 * hl + 1] = lam * dt;
    scoef[3 * hl + 2] = (1.f - lam) * dt * a;
  }
  __syncthreads();

  // this lane's four state columns n = 4 lane32 + k: their rows of B, C, B_p
  const int lane32 = threadIdx.x & 31;
  float Bv[4][R], Cv[4][R], Pv[kTrap ? 4 : 1][R];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      Bv[k][r] = sB[(4 * lane32 + k) * R + r];
      Cv[k][r] = sC[(4 * lane32 + k) * R + r];
      if (kTrap) Pv[k][r] = spB[(4 * lane32 + k) * R + r];
    }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int hl = wave; hl < hpg; hl += kThreads / 64) {
    const int h = g * hpg + hl;
    f32x4 *S = reinterpret_cast<f32x4 *>(p.ssm_state + ((int64_t)b * p.H + h) * kHeadDim * kDState);
    const float a = scoef[3 * hl], cE = scoef[3 * hl + 1], cP = scoef[3 * hl + 2];
    const float dskip = p.D ? p.D[h] : 0.f;
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      f32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(S + (c * 8 + i) * 64 + lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int prow = (c * 8 + i) * 2 + (lane >> 5);
        const float *xr = sx + (hl * kHeadDim + prow) * R;
        const float *pr = spx + (hl * kHeadDim + prow) * R;
        float xs[R], ps[kTrap ? R : 1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          xs[r] = xr[r];
          if (kTrap) ps[r] = pr[r];
        }
        f32x4 n;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float cur = 0.f, prev = 0.f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            cur = fmaf(xs[r], Bv[k][r], cur);
            if (kTrap) prev = fmaf(ps[r], Pv[k][r], prev);
          }
          float u = fmaf(a, v[i][k], cE * cur);
          if (kTrap) u = fmaf(cP, prev, u);
          n[k] = u;
        }
        __builtin_nontemporal_store(n, S + (c * 8 + i) * 64 + lane);
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          part[r] = n[0] * Cv[0][r] + n[1] * Cv[1][r] + n[2] * Cv[2][r] + n[3] * Cv[3][r];
        // the row's R sums over the 32 lanes as a reduce-scatter: each halving
        // step sends the half of the values this lane does not keep, so R = 8
        // takes 4 + 2 + 1 + 1 + 1 lane exchanges instead of 5 R; afterwards
        // every lane holds the sum of output column rsel
        int rsel = 0;
        RowScatter<R, 3>::run(part, lane32, rsel);
        if ((lane32 & kRowWriterMask<R>) == 0)
          sy[(hl * kHeadDim + prow) * R + rsel] = fmaf(dskip, xr[rsel], part[0]);
      }
    }
  }
  __syncthreads();
  // the group's heads are contiguous in y (and in prev_x): coalesced writes
  T *yg = reinterpret_cast<T *>(p.y) + (int64_t)b * p.y_sb + (int64_t)g * nxr;
  for (int e = threadIdx.x; e < nxr; e += kThreads) {
    yg[e] = from_f32<T>(sy[e]);
    if (kTrap) pxg[e] = xg[e];  // the new token's X becomes the previous one
  }
  if (kTrap)
    for (int e = threadIdx.x; e < kDState * R; e += kThreads) pBg[e] = Bg[e];
}

// bf16 inputs, ranks 2..8: the same stream over the state, with the rank
// sums x . B_n and x_prev . B_prev,n taken by v_dot2_f32_bf16 on the inputs'
// own bf16 pairs (exact products, fp32 sums).  That halves both the
// instructions of those sums and the registers that hold the lane's rows of
// B and B_prev, and X, X_prev and B, B_prev stay bf16 in LDS; y goes straight
// from the reducing lanes to HBM.  Per lane about half the registers and per
// workgroup about a third of the LDS of the kernel above, so two workgroups
// (16 waves) share a CU.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}


constexpr int kMimoThreads16 = 256;
template <int R, bool kTrap>
__global__ __launch_bounds__(kMimoThreads16) void decode_mimo_bf16_kernel(MimoParams p) {
  constexpr int R2 = R / 2;  // bf16 pairs per row of X, B
  extern __shared__ __attribute__((aligned(16))) float smem16[];
  const int b = blockIdx.x / p.G;
  const int g = blockIdx.x % p.G;
  const int hpg = p.H / p.G;
  const int nxw = hpg * kHeadDim * R2;                            // the group's X words (bf16 pairs)
  uint32_t *sx = reinterpret_cast<uint32_t *>(smem16);            // [hpg][P][R2]
  uint32_t *spx = sx + nxw;                                       // [hpg][P][R2] previous X (trapezoid)
  uint32_t *sB = spx + (kTrap ? nxw : 0);                         // [N][R2]
  uint32_t *spB = sB + kDState * R2;                              // [N][R2] previous B (trapezoid)
  float *sC = reinterpret_cast<float *>(spB + (kTrap ? kDState * R2 : 0));  // [N][R] fp32
  float *scoef = sC + kDState * R;                                // [hpg][3]: a, lam dt, (1 - lam) dt a

  const uint32_t *xg = reinterpret_cast<const uint32_t *>(reinterpret_cast<const bf16_t *>(p.x) + (int64_t)b * p.x_sb) +
                       (int64_t)g * nxw;
  const uint32_t *Bg =
      reinterpret_cast<const uint32_t *>(reinterpret_cast<const bf16_t *>(p.B) + (int64_t)b * p.B_sb) +
      (int64_t)g * kDState * R2;
  const bf16_t *Cg = reinterpret_cast<const bf16_t *>(p.C) + (int64_t)b * p.C_sb + (int64_t)g * kDState * R;
  uint32_t *pxg = kTrap ? reinterpret_cast<uint32_t *>(p.prev_x) + ((int64_t)b * p.H + (int64_t)g * hpg) * kHeadDim * R2
                        : nullptr;
  uint32_t *pBg = kTrap ? reinterpret_cast<uint32_t *>(p.prev_B) + ((int64_t)b * p.G + g) * kDState * R2 : nullptr;
  for (int e = threadIdx.x; e < nxw; e += kMimoThreads16) {
    sx[e] = xg[e];
    if (kTrap) spx[e] = pxg[e];
  }
  for (int e = threadIdx.x; e < kDState * R2; e += kMimoThreads16) {
    sB[e] = Bg[e];
    if (kTrap) spB[e] = pBg[e];
  }
  for (int e = threadIdx.x; e < kDState * R; e += kMimoThreads16) sC[e] = bf16_to_f32(Cg[e]);
  const bf16_t *dtp = reinterpret_cast<const bf16_t *>(p.dt) + (int64_t)b * p.dt_sb;
  const bf16_t *lp = (kTrap && p.lam) ? reinterpret_cast<const bf16_t *>(p.lam) + (int64_t)b * p.lam_sb : nullptr;
  for (int hl = threadIdx.x; hl < hpg; hl += kMimoThreads16) {
    const int h = g * hpg + hl;
    const float dt = softplus_f32(bf16_to_f32(dtp[h]) + (p.dt_bias ? p.dt_bias[h] : 0.f));
    const float a = __expf(dt * p.A[h]);
    const float lam = kTrap ? (lp ? bf16_to_f32(lp[h]) : 0.5f) : 1.f;
    scoef[3 * hl] = a;
    scoef[3 * hl + 1] = lam * dt;
    scoef[3 * hl + 2] = (1.f - lam) * dt * a;
  }
  __syncthreads();

  // this lane's four state columns n = 4 lane32 + k: their rows of B, B_prev (bf16 pairs) and C
  const int lane32 = threadIdx.x & 31;
  uint32_t Bw[4][R2], Pw[kTrap ? 4 : 1][R2];
  float Cv[4][R];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int m = 0; m < R2; ++m) {
      Bw[k][m] = sB[(4 * lane32 + k) * R2 + m];
      if (kTrap) Pw[k][m] = spB[(4 * lane32 + k) * R2 + m];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) Cv[k][r] = sC[(4 * lane32 + k) * R + r];
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  bf16_t *yb = reinterpret_cast<bf16_t *>(p.y) + (int64_t)b * p.y_sb + (int64_t)g * hpg * kHeadDim * R;
  for (int hl = wave; hl < hpg; hl += kMimoThreads16 / 64) {
    const int h = g * hpg + hl;
    f32x4 *S = reinterpret_cast<f32x4 *>(p.ssm_state + ((int64_t)b * p.H + h) * kHeadDim * kDState);
    const float a = scoef[3 * hl], cE = scoef[3 * hl + 1], cP = scoef[3 * hl + 2];
    const float dskip = p.D ? p.D[h] : 0.f;
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      f32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(S + (c * 8 + i) * 64 + lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int prow = (c * 8 + i) * 2 + (lane >> 5);
        const uint32_t *xr = sx + (hl * kHeadDim + prow) * R2;
        const uint32_t *pr = spx + (hl * kHeadDim + prow) * R2;
        uint32_t xs[R2], ps[kTrap ? R2 : 1];
#pragma unroll
        for (int m = 0; m < R2; ++m) {
          xs[m] = xr[m];
          if (kTrap) ps[m] = pr[m];
        }
        f32x4 n;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float cur = 0.f, prev = 0.f;
#pragma unroll
          for (int m = 0; m < R2; ++m) {
            cur = dot2(xs[m], Bw[k][m], cur);
            if (kTrap) prev = dot2(ps[m], Pw[k][m], prev);
          }
          float u = fmaf(a, v[i][k], cE * cur);
          if (kTrap) u = fmaf(cP, prev, u);
          n[k] = u;
        }
        __builtin_nontemporal_store(n, S + (c * 8 + i) * 64 + lane);
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          part[r] = n[0] * Cv[0][r] + n[1] * Cv[1][r] + n[2] * Cv[2][r] + n[3] * Cv[3][r];
        // the row's R sums over the 32 lanes as a reduce-scatter; afterwards
        // every lane holds the sum of column rsel
        int rsel = 0;
        RowScatter<R, 3>::run(part, lane32, rsel);
        if ((lane32 & kRowWriterMask<R>) == 0) {
          const uint32_t xw = xr[rsel >> 1];
          const float xv = (rsel & 1) ? hi_bf16(xw) : lo_bf16(xw);
          yb[(hl * kHeadDim + prow) * R + rsel] = f32_to_bf16(fmaf(dskip, xv, part[0]));
        }
      }
    }
  }
  if (kTrap) {
    __syncthreads();  // every read of the previous-input caches is done
    // the new token's X and B become the previous ones
    for (int e = threadIdx.x; e < nxw; e += kMimoThreads16) pxg[e] = sx[e];
    for (int e = threadIdx.x; e < kDState * R2; e += kMimoThreads16) pBg[e] = sB[e];
  }
}

size_t mimo_bf16_lds_bytes(int hpg, int R, bool trapezoid) {
  const size_t nxw = (size_t)hpg * kHeadDim * (R / 2);
  return 4 * ((trapezoid ? 2 : 1) * nxw + (trapezoid ? 2 : 1) * (size_t)kDState * (R / 2) + (size_t)kDState * R +
              3 * (size_t)hpg);
}

template <int R>
hipError_t launch_bf16(const MimoParams &p, hipStream_t s) {
  const size_t lds = mimo_bf16_lds_bytes(p.H / p.G, R, p.trapezoid != 0);
  dim3 grid(p.batch * p.G), block(kMimoThreads16);
  if (p.trapezoid) {
    auto fn = decode_mimo_bf16_kernel<R, true>;
    if (lds > 65536) {
      const hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, block, lds, s, p);
  } else {
    auto fn = decode_mimo_bf16_kernel<R, false>;
    if (lds > 65536) {
      const hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, block, lds, s, p);
  }
  return hipGetLastError();
}

template <typename T, int R>
hipError_t launch_r(const MimoParams &p, hipStream_t s) {
  const int hpg = p.H / p.G;
  // the bf16 kernel reads X and B as 4-byte pairs: even batch strides and 4-byte aligned bases
  const bool pairs = ((reinterpret_cast<uintptr_t>(p.x) | reinterpret_cast<uintptr_t>(p.B) |
                       reinterpret_cast<uintptr_t>(p.prev_x) | reinterpret_cast<uintptr_t>(p.prev_B)) & 3) == 0 &&
                     (p.x_sb % 2) == 0 && (p.B_sb % 2) == 0;
  if constexpr (R >= 2 && std::is_same<T, bf16_t>::value) {
    if (pairs) return launch_bf16<R>(p, s);
  }
  const size_t lds = mimo_lds_bytes(hpg, R, p.trapezoid != 0);
  dim3 grid(p.batch * p.G), block(threads_for<R>());
  if (p.trapezoid) {
    auto fn = decode_mimo_kernel<T, R, true>;
    if (lds > 65536) {
      const hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, block, lds, s, p);
  } else {
    auto fn = decode_mimo_kernel<T, R, false>;
    if (lds > 65536) {
      const hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, block, lds, s, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const MimoParams &p, hipStream_t s) {
  switch (p.R) {
    case 1: return launch_r<T, 1>(p, s);
    case 2: return launch_r<T, 2>(p, s);
    case 4: return launch_r<T, 4>(p, s);
    default: return launch_r<T, 8>(p, s);
  }
}

}  // namespace

size_t mimo_lds_bytes(int hpg, int R, bool trapezoid) {
  const size_t nxr = (size_t)hpg * kHeadDim * R;
  return sizeof(float) * ((trapezoid ? 3 : 2) * nxr + (trapezoid ? 3 : 2) * (size_t)kDState * R + 3 * (size_t)hpg);
}

hipError_t launch_decode_mimo(const MimoParams &p, hipStream_t stream) {
  return p.bf16 ? launch_t<bf16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace ssd
