// Depthwise causal conv1d (width 4) + SiLU on gfx950.
//
// The Mamba-2 mixer runs a width-4 depthwise causal conv with SiLU over the
// x|B|C channels before the selective scan ("Nemotron-H style Hybrid
// Mamba-Transformer 3B feasibility study", sec. 1.4 "Mamba-2
// configuration"; "Nemotron-Mamba3 architecture" article, sec. 2.2).
//
// Layout choice: the channel dimension is contiguous in HBM, so lanes run
// along channels (8 per lane = one 16-byte bf16 vector; a wave reads 1 KiB
// of one token row per instruction) and each thread walks a tile of kTile
// consecutive tokens.  The 3-token halo then lives in registers: the window
// slides by one register copy per token, and only the first 3 rows of a
// tile are read twice (by this tile and, as its last rows, by the previous
// one).  Packed sequences reset the window to that sequence's conv state
// (or zeros) when seq_idx changes.  The conv-state export is a separate
// tiny kernel that binary-searches each sequence's end in seq_idx.
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;    // channels per thread
constexpr int kTile = 32;  // tokens per thread (the 3-row halo re-read is 3/32 of the input)
constexpr int kAhead = 8;  // token rows loaded ahead of their use

template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  __device__ static void load(const bf16_t *p, float (&v)[kVec]) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = lo_bf16(w[i]); v[2 * i + 1] = hi_bf16(w[i]); }
  }
  __device__ static void store(bf16_t *p, const float (&v)[kVec]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(v[2 * i], v[2 * i + 1]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));  // streamed out, not re-read here
  }
};
template <> struct Vec8<float> {
  __device__ static void load(const float *p, float (&v)[kVec]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static void store(float *p, const float (&v)[kVec]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <typename T>
__device__ __forceinline__ void zero8(float (&v)[kVec]) {
#pragma unroll
  for (int i = 0; i < kVec; ++i) v[i] = 0.f;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void conv1d_silu_kernel(ConvParams p) {
  const int nvec = p.CH / kVec;
  const int ntile = (p.L + kTile - 1) / kTile;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)p.batch * ntile * nvec;
  if (gid >= total) return;
  const int vec = (int)(gid % nvec);
  const int64_t rest = gid / nvec;
  const int tile = (int)(rest % ntile);
  const int b = (int)(rest / ntile);
  const int c0 = vec * kVec;
  const int t0 = tile * kTile;
  const int t1 = min(p.L, t0 + kTile);

  const T *__restrict__ x = reinterpret_cast<const T *>(p.x) + (int64_t)b * p.x_sb + c0;
  T *__restrict__ out = reinterpret_cast<T *>(p.out) + (int64_t)b * p.o_sb + c0;
  const T *sin = reinterpret_cast<const T *>(p.state_in);

  float w[kVec][kConvWidth];
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const float4 wv = *reinterpret_cast<const float4 *>(p.w + (int64_t)(c0 + i) * kConvWidth);
    w[i][0] = wv.x; w[i][1] = wv.y; w[i][2] = wv.z; w[i][3] = wv.w;
  }
  float bias[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) bias[i] = p.bias ? p.bias[c0 + i] : 0.f;

  // window rows v(t-3), v(t-2), v(t-1) for the first token of the tile
  float win[3][kVec];
  // state row of the current sequence (clamped: a bad seq_idx gives wrong
  // values, never an out-of-bounds read)
  const int rows = p.seq_idx ? p.num_seqs : p.batch;
  int cur = p.seq_idx ? min(max(p.seq_idx[t0], 0), rows - 1) : b;
  {
    // d = number of tokens of the current sequence just before t0 (at most 3)
    int d = 0;
    while (d < 3 && t0 - d - 1 >= 0 &&
           (!p.seq_idx || min(max(p.seq_idx[t0 - d - 1], 0), rows - 1) == cur))
      ++d;
#pragma unroll
    for (int k = 1; k <= 3; ++k) {
      float(&v)[kVec] = win[3 - k];
      if (k <= d) {
        Vec8<T>::load(x + (int64_t)(t0 - k) * p.x_st, v);
      } else if (sin) {
        // v(t0 - k) = state row (t0 - k) - start + 3 with start = t0 - d
        Vec8<T>::load(sin + ((int64_t)cur * (kConvWidth - 1) + (3 - k + d)) * p.s_st + c0, v);
      } else {
        zero8<T>(v);
      }
    }
  }

  auto step = [&](int t, const float(&v)[kVec]) {
    if (p.seq_idx) {
      const int sq = min(max(p.seq_idx[t], 0), rows - 1);
      if (sq != cur) {  // first token of a new sequence: its window is its conv state
        cur = sq;
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          if (sin) Vec8<T>::load(sin + ((int64_t)cur * (kConvWidth - 1) + r) * p.s_st + c0, win[r]);
          else zero8<T>(win[r]);
        }
      }
    }
    float o[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      float u = bias[i];
      u = fmaf(w[i][0], win[0][i], u);
      u = fmaf(w[i][1], win[1][i], u);
      u = fmaf(w[i][2], win[2][i], u);
      u = fmaf(w[i][3], v[i], u);
      o[i] = silu_f32(u);
    }
    Vec8<T>::store(out + (int64_t)t * p.o_st, o);
#pragma unroll
    for (int i = 0; i < kVec; ++i) { win[0][i] = win[1][i]; win[1][i] = win[2][i]; win[2][i] = v[i]; }
  };
  // kAhead rows in flight per thread; the tail of a tile one row at a time
  int t = t0;
  for (; t + kAhead <= t1; t += kAhead) {
    float v[kAhead][kVec];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) Vec8<T>::load(x + (int64_t)(t + k) * p.x_st, v[k]);
#pragma unroll
    for (int k = 0; k < kAhead; ++k) step(t + k, v[k]);
  }
  for (; t < t1; ++t) {
    float v[kVec];
    Vec8<T>::load(x + (int64_t)t * p.x_st, v);
    step(t, v);
  }
}

// First indices in [0, L] with seq_idx[i] >= s and >= s + 1 (seq_idx
// non-decreasing): both binary searches advance in the same loop, so their
// dependent loads overlap.
__device__ __forceinline__ void sequence_span(const int32_t *seq_idx, int L, int s, int &start, int &end) {
  int lo0 = 0, hi0 = L, lo1 = 0, hi1 = L;
  while (lo0 < hi0 || lo1 < hi1) {
    const int m0 = (lo0 + hi0) >> 1, m1 = (lo1 + hi1) >> 1;
    const int v0 = lo0 < hi0 ? seq_idx[m0] : 0;
    const int v1 = lo1 < hi1 ? seq_idx[m1] : 0;
    if (lo0 < hi0) { if (v0 < s) lo0 = m0 + 1; else hi0 = m0; }
    if (lo1 < hi1) { if (v1 < s + 1) lo1 = m1 + 1; else hi1 = m1; }
  }
  start = lo0;
  end = max(lo0, lo1);
}

// conv_state_out[row][r] = v(end - 3 + r) of each sequence.
template <typename T>
__global__ __launch_bounds__(kThreads) void conv_state_out_kernel(ConvParams p, int rows) {
  const int nvec = p.CH / kVec;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (int64_t)rows * nvec) return;
  const int vec = (int)(gid % nvec);
  const int s = (int)(gid / nvec);
  const int c0 = vec * kVec;
  int start = 0, end = p.L;
  const T *x = reinterpret_cast<const T *>(p.x) + c0;
  if (p.seq_idx) {
    sequence_span(p.seq_idx, p.L, s, start, end);
  } else {
    x += (int64_t)s * p.x_sb;
  }
  const T *sin = reinterpret_cast<const T *>(p.state_in);
  T *so = reinterpret_cast<T *>(p.state_out) + (int64_t)s * (kConvWidth - 1) * p.s_st + c0;
  for (int r = 0; r < kConvWidth - 1; ++r) {
    const int tau = end - (kConvWidth - 1) + r;
    float v[kVec];
    if (tau >= start) Vec8<T>::load(x + (int64_t)tau * p.x_st, v);
    else if (sin) Vec8<T>::load(sin + ((int64_t)s * (kConvWidth - 1) + (tau - start + kConvWidth - 1)) * p.s_st + c0, v);
    else zero8<T>(v);
    Vec8<T>::store(so + (int64_t)r * p.s_st, v);
  }
}

}  // namespace

hipError_t launch_conv1d_silu(const ConvParams &p, hipStream_t stream) {
  const int nvec = p.CH / kVec;
  const int ntile = (p.L + kTile - 1) / kTile;
  const int64_t total = (int64_t)p.batch * ntile * nvec;
  if (total > 0) {
    dim3 grid((unsigned)((total + kThreads - 1) / kThreads)), block(kThreads);
    if (p.bf16) hipLaunchKernelGGL(conv1d_silu_kernel<bf16_t>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(conv1d_silu_kernel<float>, grid, block, 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return p.state_out ? launch_conv_state_out(p, stream) : hipSuccess;
}

hipError_t launch_conv_state_out(const ConvParams &p, hipStream_t stream) {
  const int nvec = p.CH / kVec;
  const int rows = p.seq_idx ? p.num_seqs : p.batch;
  const int64_t n = (int64_t)rows * nvec;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + kThreads - 1) / kThreads)), block(kThreads);
  if (p.bf16) hipLaunchKernelGGL(conv_state_out_kernel<bf16_t>, grid, block, 0, stream, p, rows);
  else hipLaunchKernelGGL(conv_state_out_kernel<float>, grid, block, 0, stream, p, rows);
  return hipGetLastError();
}

}  // namespace ssd
