// Single-token decode step of the Mamba-2 SSD layer on gfx950.
//
// Per token and head the recurrence is S <- exp(dt A) S + dt x (outer) B,
// y = S . C + D x ("Mamba-3: an inference-first state space model": Mamba-2's
// scalar-times-identity transition leaves each decode token with very little
// compute per byte of state, so the step is bound by memory traffic; the
// "Bamba-9B" summary's inference-efficiency section makes the same point).
// The kernel therefore streams the fp32 state exactly once: one 16-byte
// non-temporal load and one store per four state values, nothing else of
// size.
//
// One workgroup of 16 waves owns one (batch row, group): it runs the conv
// window of the group's channels (its heads' x channels plus the group's B
// and C channels) and shifts that part of the conv state -- every channel
// belongs to exactly one workgroup, so the in-place update has no race.
// Then each wave takes one head and streams its 32 KiB of state in four
// pieces of 8 KiB; every load instruction covers two whole state rows, so
// the workgroup walks all of its heads' states at once.  A state row (128
// floats) is 32 lanes x float4, so y[p] is a 32-lane sum (DPP moves within
// each 16-lane row, a permlane swap across the two); y is staged in LDS and
// written once per group.
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kThreads = 1024;  // 16 waves: one head each (group of 16 heads)

template <typename T>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeParams p) {
  extern __shared__ float smem[];  // [hpg*P x | N B | N C] post-conv values, dt, a, then y
  const int b = blockIdx.x / p.G;
  const int g = blockIdx.x % p.G;
  const int hpg = p.H / p.G;
  const int nx = hpg * kHeadDim;
  const int nloc = nx + 2 * kDState;
  const int HP = p.H * kHeadDim;
  const int CH = HP + 2 * p.G * kDState;
  float *sv = smem;
  float *s_dt = smem + nloc;
  float *s_a = s_dt + hpg;
  float *s_y = s_a + hpg;

  auto state_of = [&](int hl) {
    return reinterpret_cast<f32x4 *>(p.ssm_state + ((int64_t)b * p.H + g * hpg + hl) * kHeadDim * kDState);
  };

  const T *xbc = reinterpret_cast<const T *>(p.xBC) + (int64_t)b * p.xBC_sb;
  T *cst = p.conv_state ? reinterpret_cast<T *>(p.conv_state) + (int64_t)b * (kConvWidth - 1) * CH
                        : nullptr;

  // conv window + SiLU on this workgroup's channels, and the conv-state shift
  for (int lc = threadIdx.x; lc < nloc; lc += kThreads) {
    int c;
    if (lc < nx) c = g * nx + lc;
    else if (lc < nx + kDState) c = HP + g * kDState + (lc - nx);
    else c = HP + p.G * kDState + g * kDState + (lc - nx - kDState);
    const float tok = to_f32<T>(xbc[c]);
    float v;
    if (cst) {
      const float4 w = *reinterpret_cast<const float4 *>(p.conv_w + (int64_t)c * kConvWidth);
      const T r0 = cst[c], r1 = cst[CH + c], r2 = cst[2 * CH + c];
      float u = p.conv_b ? p.conv_b[c] : 0.f;
      u += w.x * to_f32<T>(r0);
      u += w.y * to_f32<T>(r1);
      u += w.z * to_f32<T>(r2);
      u += w.w * tok;
      v = silu_f32(u);
      cst[c] = r1;
      cst[CH + c] = r2;
      cst[2 * CH + c] = xbc[c];
    } else {
      v = tok;
    }
    sv[lc] = v;
  }
  const T *dtp = reinterpret_cast<const T *>(p.dt) + (int64_t)b * p.dt_sb;
  for (int hl = threadIdx.x; hl < hpg; hl += kThreads) {
    const int h = g * hpg + hl;
    const float dt = softplus_f32(to_f32<T>(dtp[h]) + (p.dt_bias ? p.dt_bias[h] : 0.f));
    s_dt[hl] = dt;
    s_a[hl] = __expf(dt * p.A[h]);
  }
  __syncthreads();

  const float *sB = sv + nx;
  const float *sC = sv + nx + kDState;
  const int lane32 = threadIdx.x & 31;
  // this thread's four state columns are the same for every row and head
  const float4 Bv = *reinterpret_cast<const float4 *>(sB + 4 * lane32);
  const float4 Cv = *reinterpret_cast<const float4 *>(sC + 4 * lane32);
  T *yb = reinterpret_cast<T *>(p.y) + (int64_t)b * p.y_sb;

  // one wave per head: it streams the head's 32 KiB of state in four pieces
  // of 8 KiB (each load instruction covers two whole state rows)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int hl = wave; hl < hpg; hl += kThreads / 64) {
    const int h = g * hpg + hl;
    f32x4 *S = state_of(hl);
    const float dt = s_dt[hl], a = s_a[hl];
    const float dskip = p.D ? p.D[h] : 0.f;
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      f32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(S + (c * 8 + i) * 64 + lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int prow = (c * 8 + i) * 2 + (lane >> 5);
        const float xp = sv[hl * kHeadDim + prow];
        const float dx = dt * xp;
        f32x4 n;
        n[0] = fmaf(a, v[i][0], dx * Bv.x);
        n[1] = fmaf(a, v[i][1], dx * Bv.y);
        n[2] = fmaf(a, v[i][2], dx * Bv.z);
        n[3] = fmaf(a, v[i][3], dx * Bv.w);
        __builtin_nontemporal_store(n, S + (c * 8 + i) * 64 + lane);
        const float part = half_wave_sum(n[0] * Cv.x + n[1] * Cv.y + n[2] * Cv.z + n[3] * Cv.w);
        if (lane32 == 0) s_y[hl * kHeadDim + prow] = part + dskip * xp;
      }
    }
  }
  // the group's heads are contiguous in y: one coalesced write of hpg * P values
  __syncthreads();
  T *yg = yb + (int64_t)g * hpg * kHeadDim;
  for (int e = threadIdx.x; e < hpg * kHeadDim; e += kThreads) yg[e] = from_f32<T>(s_y[e]);
}

}  // namespace

hipError_t launch_decode_step(const DecodeParams &p, hipStream_t stream) {
  const int hpg = p.H / p.G;
  const size_t lds = sizeof(float) * (2 * hpg * kHeadDim + 2 * kDState + 2 * hpg);
  dim3 grid(p.batch * p.G), block(kThreads);
  const void *fn = p.bf16 ? reinterpret_cast<const void *>(decode_step_kernel<bf16_t>)
                         : reinterpret_cast<const void *>(decode_step_kernel<float>);
  if (lds > 65536) {
    const hipError_t e = set_max_dynamic_lds(fn, lds);
    if (e != hipSuccess) return e;
  }
  if (p.bf16) hipLaunchKernelGGL(decode_step_kernel<bf16_t>, grid, block, lds, stream, p);
  else hipLaunchKernelGGL(decode_step_kernel<float>, grid, block, lds, stream, p);
  return hipGetLastError();
}

}  // namespace ssd
