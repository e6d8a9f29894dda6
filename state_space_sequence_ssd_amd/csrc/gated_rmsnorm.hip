// Gated RMSNorm of the mixer output on gfx950 (HBM-bound streaming kernel).
//
// Mamba-2 keeps an RMSNorm together with the output gate z; the norm may sit
// before or after the gate, per group of channels or over the whole width
// ("Mamba-3: an inference-first state space model": the normalization
// paragraph, and the later remark on the norm's placement and its grouped or
// plain type).  Per token row and group of group_size channels, with
// rms(v) = sqrt(mean(v^2) + eps):
//   after the gate:   g = y SiLU(z),  out = g / rms(g) w
//   before the gate:  out = y / rms(y) w SiLU(z)
//
// One wave per (token, group).  Each lane holds NI 16-byte vectors of the
// group (8 bf16 or 4 fp32 channels each), 64 lanes x VEC channels apart, so
// every load and store instruction moves 1 KiB of consecutive bytes; y and z
// are read once and out written once (non-temporal: nothing is reused), the
// weights come from L2.  The mean square is a wave reduction in fp32; the
// group's raw vectors stay in registers between the two passes, so HBM sees
// each byte exactly once.
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kNormThreads = 256;  // four (token, group) units per workgroup

template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  typedef u32x4 raw;
  __device__ static void unpack(raw r, float *f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = lo_bf16(r[k]);
      f[2 * k + 1] = hi_bf16(r[k]);
    }
  }
  __device__ static raw pack(const float *f) {
    raw r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = pack2_bf16(f[2 * k], f[2 * k + 1]);
    return r;
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef f32x4 raw;
  __device__ static void unpack(raw r, float *f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = r[k];
  }
  __device__ static raw pack(const float *f) { return raw{f[0], f[1], f[2], f[3]}; }
};

template <typename T, int NI, bool kGate, bool kBefore>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(NormParams p) {
  using V = Vec<T>;
  using raw = typename V::raw;
  constexpr int VEC = V::N;
  const int lane = threadIdx.x & 63;
  const long long unit = (long long)blockIdx.x * (kNormThreads / 64) + (threadIdx.x >> 6);
  const int ngroups = p.CH / p.gs;
  if (unit >= (long long)p.batch * p.L * ngroups) return;
  const int gi = (int)(unit % ngroups);
  const long long tok = unit / ngroups;
  const long long b = tok / p.L, t = tok % p.L;
  const int c0 = gi * p.gs;
  const T *yr = reinterpret_cast<const T *>(p.y) + b * p.y_sb + t * p.y_st + c0;
  const T *zr = kGate ? reinterpret_cast<const T *>(p.z) + b * p.z_sb + t * p.z_st + c0 : nullptr;
  T *outr = reinterpret_cast<T *>(p.out) + b * p.o_sb + t * p.o_st + c0;

  // the group's raw vectors stay in registers between the two passes; the
  // gated values are recomputed from them in the second pass
  raw ry[NI], rz[kGate ? NI : 1];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int c = (k * 64 + lane) * VEC;
    ry[k] = raw{};
    if (kGate) rz[k] = raw{};
    if (c < p.gs) {
      ry[k] = __builtin_nontemporal_load(reinterpret_cast<const raw *>(yr + c));
      if (kGate) rz[k] = __builtin_nontemporal_load(reinterpret_cast<const raw *>(zr + c));
    }
  }
  // out-of-range lanes hold zeros: they add nothing to the sum of squares
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    float v[VEC], zg[VEC];
    V::unpack(ry[k], v);
    if (kGate && !kBefore) {
      V::unpack(rz[k], zg);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] *= silu_f32(zg[e]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss = fmaf(v[e], v[e], ss);
  }
  ss = wave_sum(ss);
  const float inv = __builtin_amdgcn_rsqf(ss / (float)p.gs + p.eps);
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int c = (k * 64 + lane) * VEC;
    if (c >= p.gs) continue;
    float v[VEC], zg[VEC], w[VEC], o[VEC];
    V::unpack(ry[k], v);
    if (kGate) {
      V::unpack(rz[k], zg);
#pragma unroll
      for (int e = 0; e < VEC; ++e) zg[e] = silu_f32(zg[e]);
    }
    const f32x4 *wp = reinterpret_cast<const f32x4 *>(p.w + c0 + c);
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const f32x4 wq = wp[q];
      w[4 * q] = wq[0]; w[4 * q + 1] = wq[1]; w[4 * q + 2] = wq[2]; w[4 * q + 3] = wq[3];
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float g = (kGate && !kBefore) ? v[e] * zg[e] : v[e];
      o[e] = g * inv * w[e];
      if (kGate && kBefore) o[e] *= zg[e];
    }
    __builtin_nontemporal_store(V::pack(o), reinterpret_cast<raw *>(outr + c));
  }
}

template <typename T, int NI>
hipError_t launch_ni(const NormParams &p, unsigned nblk, hipStream_t s) {
  if (!p.z)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, NI, false, false>), dim3(nblk), dim3(kNormThreads), 0, s, p);
  else if (p.before)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, NI, true, true>), dim3(nblk), dim3(kNormThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, NI, true, false>), dim3(nblk), dim3(kNormThreads), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const NormParams &p, unsigned nblk, hipStream_t s) {
  const int per = 64 * Vec<T>::N;  // channels one pass of the wave covers
  const int ni = (p.gs + per - 1) / per;
  if (ni <= 1) return launch_ni<T, 1>(p, nblk, s);
  if (ni <= 2) return launch_ni<T, 2>(p, nblk, s);
  if (ni <= 4) return launch_ni<T, 4>(p, nblk, s);
  if (ni <= 8) return launch_ni<T, 8>(p, nblk, s);
  return launch_ni<T, 16>(p, nblk, s);
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormParams &p, hipStream_t stream) {
  const long long units = (long long)p.batch * p.L * (p.CH / p.gs);
  if (units == 0) return hipSuccess;
  const unsigned nblk = (unsigned)((units + kNormThreads / 64 - 1) / (kNormThreads / 64));
  return p.bf16 ? launch_t<bf16_t>(p, nblk, stream) : launch_t<float>(p, nblk, stream);
}

}  // namespace ssd
