// Backward pass of the chunked SSD scan on gfx950 (batch rows, fp32
// arithmetic).  The training workload of the layer needs the gradient of
// every input ("Nemotron-H style Hybrid Mamba-Transformer 3B feasibility
// study", sec. 3.1, forward/backward verification; sec. 7, Phase 2).
//
// Forward per (row, head), in chunks of Q tokens with the inclusive in-chunk
// cumulative log-decay cs_i = sum_{k<=i} dt_k A (every exponent below is a
// difference cs_i - cs_j with j <= i, or cs_i itself, so it is <= 0):
//   y_i   = e^{cs_i} S0 C_i + sum_{j<=i} e^{cs_i - cs_j} (C_i . B_j) dt_j x_j + D x_i
//   S_end = e^{cs_Q} S0 + sum_j e^{cs_Q - cs_j} dt_j x_j B_j^T
// (S0 the state entering the chunk, cs_Q the chunk's last cs).  Given dy and
// G1 = dL/dS_end, with L_ij = e^{cs_i - cs_j} (j <= i), e_i = e^{cs_i},
// f_j = e^{cs_Q - cs_j}:
//   dx_j  = D dy_j + dt_j (sum_{i>=j} L_ij (C_i . B_j) dy_i + f_j G1 B_j)
//   dB_j  = dt_j (sum_{i>=j} L_ij (dy_i . x_j) C_i + f_j G1^T x_j)
//   dC_i  = e_i S0^T dy_i + sum_{j<=i} L_ij dt_j (dy_i . x_j) B_j
//   G0    = sum_i e_i dy_i C_i^T + e^{cs_Q} G1          (dL/dS0, the previous chunk's G1)
//   ddt_j = sum_{i>=j} L_ij (C_i . B_j)(dy_i . x_j) + f_j x_j . (G1 B_j)   (the explicit dt_j)
//           + A sum_{k>=j} dcs_k                                          (through cs)
//   dcs_i = e_i dy_i . (S0 C_i) + sum_j W_ij - sum_k W_ki - f_i dt_i x_i . (G1 B_i)
//           + [i = last] (e^{cs_Q} <G1, S0> + sum_j f_j dt_j x_j . (G1 B_j)),
//   W_ij  = L_ij (C_i . B_j)(dy_i . x_j) dt_j (j <= i),
//   dA   += sum_j dt_j sum_{k>=j} dcs_k,  dz_j = ddt_j sigmoid(z_j), z = dt_raw + dt_bias.
//
// Three launches:
//   1. bwd_states_kernel: one workgroup per (row, head) walks the chunks
//      forward and stores the state entering each one (fp32, in the
//      workspace).
//   2. bwd_chunks_kernel: one workgroup per (row, head) walks the chunks in
//      reverse; the adjoint G, the entering state and every chunk operand
//      live in LDS, and each product above is a loop over LDS rows.  dB and
//      dC are written per head, the per-head scalars per (row, head).
//   3. bwd_reduce_kernel: dB, dC summed over the heads of each group and
//      dA, dD, ddt_bias over the rows, in a fixed order (no float atomics,
//      repeat runs are bitwise identical).
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kQ = 32;      // tokens per backward chunk
constexpr int kT = 256;     // threads per workgroup
constexpr int kP = kHeadDim, kN = kDState;
constexpr int kPN = kP * kN;

template <typename T> __device__ __forceinline__ float ld(const void *base, int64_t i) {
  return to_f32<T>(reinterpret_cast<const T *>(base)[i]);
}

// dt and the inclusive cumulative log-decay of one chunk (nv valid tokens),
// by wave 0; tokens past the end get dt = 0.
template <typename T>
__device__ __forceinline__ void chunk_dt(const BwdParams &p, int b, int h, int t0, int nv, float *s_dt, float *s_cs,
                                         float *s_z) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float z = 0.f, d = 0.f;
    if (lane < nv) {
      z = ld<T>(p.dt, ((int64_t)b * p.L + t0 + lane) * p.H + h) + (p.dt_bias ? p.dt_bias[h] : 0.f);
      d = softplus_f32(z);
    }
    float incl = d * p.A[h];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane < kQ) {
      s_dt[lane] = d;
      s_cs[lane] = incl;
      s_z[lane] = z;
    }
  }
}

// -------------------------------------------------------------------------
// 1. the state entering every chunk
// -------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void bwd_states_kernel(BwdParams p) {
  __shared__ float sX[kQ * kP], sB[kQ * kN], s_dt[kQ], s_cs[kQ], s_z[kQ];
  const int b = blockIdx.x / p.H, h = blockIdx.x % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x;
  float *states = p.ws_states + ((int64_t)b * p.H + h) * p.nchunks * kPN;
  // this thread's 32 state values: row p = tid / 4, columns n = 32 (tid % 4) + 0..31
  const int pr = tid >> 2, n0 = 32 * (tid & 3);
  float s[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) s[k] = p.init ? p.init[((int64_t)b * p.H + h) * kPN + pr * kN + n0 + k] : 0.f;
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
#pragma unroll
    for (int k = 0; k < 32; ++k) states[(int64_t)c * kPN + pr * kN + n0 + k] = s[k];
    for (int e = tid; e < kQ * kP; e += kT) {
      const int j = e / kP, q = e % kP;
      sX[e] = j < nv ? ld<T>(p.x, (((int64_t)b * p.L + t0 + j) * p.H + h) * kP + q) : 0.f;
    }
    for (int e = tid; e < kQ * kN; e += kT) {
      const int j = e / kN, q = e % kN;
      sB[e] = j < nv ? ld<T>(p.B, (((int64_t)b * p.L + t0 + j) * p.G + g) * kN + q) : 0.f;
    }
    chunk_dt<T>(p, b, h, t0, nv, s_dt, s_cs, s_z);
    __syncthreads();
    const float last = s_cs[kQ - 1], dec = __expf(last);
#pragma unroll
    for (int k = 0; k < 32; ++k) s[k] *= dec;
    for (int j = 0; j < nv; ++j) {
      const float wx = __expf(last - s_cs[j]) * s_dt[j] * sX[j * kP + pr];
#pragma unroll
      for (int k = 0; k < 32; ++k) s[k] = fmaf(wx, sB[j * kN + n0 + k], s[k]);
    }
    __syncthreads();
  }
}

// -------------------------------------------------------------------------
// 2. the chunks in reverse
// -------------------------------------------------------------------------
// Rows are padded by one float (129 and 65 floats), so lanes that walk down
// a column of one of these tiles hit different LDS banks.
constexpr int kNP = kN + 1, kPP = kP + 1;
__device__ __forceinline__ int gi(int q, int n) { return q * kNP + n; }   // G, S0: [p][n]
__device__ __forceinline__ int bi(int j, int n) { return j * kNP + n; }   // B, C: [token][n]
__device__ __forceinline__ int xi(int j, int q) { return j * kPP + q; }   // X, DY, GB, S0C: [token][p]

struct BwdSmem {
  float G[kP * kNP];   // adjoint dL/dS leaving the chunk (G1), then entering (G0)
  float S0[kP * kNP];  // state entering the chunk
  float X[kQ * kPP], DY[kQ * kPP], B[kQ * kNP], C[kQ * kNP];
  float CB[kQ * kQ], DYX[kQ * kQ];                 // C_i . B_j, dy_i . x_j
  float Lm[kQ * kQ];                               // e^{cs_i - cs_j} for j <= i, else 0
  float GB[kQ * kPP];                              // (G1 B_j)[p]
  float XG[kQ * kN];                               // (G1^T x_j)[n]
  float S0C[kQ * kPP];                             // (S0 C_i)[p]
  float dt[kQ], cs[kQ], z[kQ], ei[kQ], fj[kQ], dcs[kQ], ddt[kQ], xgb[kQ], red[kT / 64];
};

template <typename T>
__global__ __launch_bounds__(kT) void bwd_chunks_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  BwdSmem &s = *reinterpret_cast<BwdSmem *>(smem_raw);
  const int b = blockIdx.x / p.H, h = blockIdx.x % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x;
  const float Ah = p.A[h], Dh = p.D ? p.D[h] : 0.f;
  const float *states = p.ws_states + ((int64_t)b * p.H + h) * p.nchunks * kPN;
  for (int e = tid; e < kPN; e += kT)
    s.G[gi(e / kN, e % kN)] = p.dfinal ? p.dfinal[((int64_t)b * p.H + h) * kPN + e] : 0.f;
  float accA = 0.f, accD = 0.f, accBias = 0.f;
  __syncthreads();

  for (int c = p.nchunks - 1; c >= 0; --c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
    // operands of the chunk (rows past the end are zero; their dt is 0)
    for (int e = tid; e < kPN; e += kT) s.S0[gi(e / kN, e % kN)] = states[(int64_t)c * kPN + e];
    for (int e = tid; e < kQ * kP; e += kT) {
      const int j = e / kP, q = e % kP;
      const int64_t o = (((int64_t)b * p.L + t0 + j) * p.H + h) * kP + q;
      s.X[xi(j, q)] = j < nv ? ld<T>(p.x, o) : 0.f;
      s.DY[xi(j, q)] = j < nv ? ld<T>(p.dy, o) : 0.f;
    }
    for (int e = tid; e < kQ * kN; e += kT) {
      const int j = e / kN, q = e % kN;
      const int64_t o = (((int64_t)b * p.L + t0 + j) * p.G + g) * kN + q;
      s.B[bi(j, q)] = j < nv ? ld<T>(p.B, o) : 0.f;
      s.C[bi(j, q)] = j < nv ? ld<T>(p.C, o) : 0.f;
    }
    chunk_dt<T>(p, b, h, t0, nv, s.dt, s.cs, s.z);
    __syncthreads();
    for (int e = tid; e < kQ * kQ; e += kT) {
      const int i = e / kQ, j = e % kQ;
      s.Lm[e] = j <= i ? __expf(s.cs[i] - s.cs[j]) : 0.f;
    }
    if (tid < kQ) {
      s.ei[tid] = __expf(s.cs[tid]);
      s.fj[tid] = __expf(s.cs[kQ - 1] - s.cs[tid]);
    }

    // first products: CB, dyX (Q x Q), G1 B (Q x P), G1^T x (Q x N), S0 C (Q x P), <G1, S0>
    for (int e = tid; e < kQ * kQ; e += kT) {
      const int i = e / kQ, j = e % kQ;
      float cb = 0.f, dx = 0.f;
      for (int n = 0; n < kN; ++n) cb = fmaf(s.C[bi(i, n)], s.B[bi(j, n)], cb);
      for (int q = 0; q < kP; ++q) dx = fmaf(s.DY[xi(i, q)], s.X[xi(j, q)], dx);
      s.CB[e] = cb;
      s.DYX[e] = dx;
    }
    for (int e = tid; e < kQ * kP; e += kT) {
      const int j = e / kP, q = e % kP;
      float gb = 0.f, sc = 0.f;
      for (int n = 0; n < kN; ++n) {
        gb = fmaf(s.G[gi(q, n)], s.B[bi(j, n)], gb);
        sc = fmaf(s.S0[gi(q, n)], s.C[bi(j, n)], sc);
      }
      s.GB[xi(j, q)] = gb;
      s.S0C[xi(j, q)] = sc;
    }
    for (int e = tid; e < kQ * kN; e += kT) {
      const int j = e / kN, n = e % kN;
      float xg = 0.f;
      for (int q = 0; q < kP; ++q) xg = fmaf(s.X[xi(j, q)], s.G[gi(q, n)], xg);
      s.XG[e] = xg;
    }
    float gs = 0.f;  // <G1, S0>
    for (int e = tid; e < kPN; e += kT) gs = fmaf(s.G[gi(e / kN, e % kN)], s.S0[gi(e / kN, e % kN)], gs);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gs += __shfl_xor(gs, off, 64);
    if ((tid & 63) == 0) s.red[tid >> 6] = gs;
    __syncthreads();
    const float G1S0 = s.red[0] + s.red[1] + s.red[2] + s.red[3];
    const float eQ = s.ei[kQ - 1];

    // per-token scalars: the explicit dt gradient and dcs (one thread per token)
    if (tid < kQ) {
      const int j = tid;
      const float fj = s.fj[j];
      float xgb = 0.f;  // x_j . (G1 B_j)
      for (int q = 0; q < kP; ++q) xgb = fmaf(s.X[xi(j, q)], s.GB[xi(j, q)], xgb);
      s.xgb[j] = xgb;
      float dexp = fj * xgb;  // explicit: f_j x_j . G1 B_j + sum_{i>=j} L_ij CB_ij dyX_ij
      float col = 0.f;        // sum_{i>=j} W_ij
      for (int i = j; i < kQ; ++i) {
        const float m = s.Lm[i * kQ + j] * s.CB[i * kQ + j] * s.DYX[i * kQ + j];
        dexp += m;
        col = fmaf(m, s.dt[j], col);
      }
      float row = 0.f;        // sum_{k<=j} W_jk
      for (int k = 0; k <= j; ++k)
        row = fmaf(s.Lm[j * kQ + k] * s.CB[j * kQ + k] * s.DYX[j * kQ + k], s.dt[k], row);
      float ey = 0.f;         // dy_j . (S0 C_j)
      for (int q = 0; q < kP; ++q) ey = fmaf(s.DY[xi(j, q)], s.S0C[xi(j, q)], ey);
      float dcs = s.ei[j] * ey + row - col - fj * s.dt[j] * xgb;
      s.ddt[j] = dexp;
      s.dcs[j] = dcs;
    }
    __syncthreads();
    if (tid == 0) {
      float tot = eQ * G1S0;
      for (int j = 0; j < kQ; ++j) tot = fmaf(s.fj[j] * s.dt[j], s.xgb[j], tot);
      s.dcs[kQ - 1] += tot;
      // through cs: ddt_j += A sum_{k>=j} dcs_k; dA += dt_j sum_{k>=j} dcs_k
      float suf = 0.f;
      for (int j = kQ - 1; j >= 0; --j) {
        suf += s.dcs[j];
        s.ddt[j] = fmaf(Ah, suf, s.ddt[j]);
        accA = fmaf(s.dt[j], suf, accA);
      }
    }
    // outputs of the chunk: dx, dB, dC, ddt_raw; dD
    for (int e = tid; e < kQ * kP; e += kT) {
      const int j = e / kP, q = e % kP;
      if (j >= nv) continue;
      float acc = 0.f;
      for (int i = j; i < kQ; ++i) acc = fmaf(s.Lm[i * kQ + j] * s.CB[i * kQ + j], s.DY[xi(i, q)], acc);
      const float v = fmaf(Dh, s.DY[xi(j, q)], s.dt[j] * fmaf(s.fj[j], s.GB[xi(j, q)], acc));
      reinterpret_cast<T *>(p.dx)[(((int64_t)b * p.L + t0 + j) * p.H + h) * kP + q] = from_f32<T>(v);
    }
    for (int e = tid; e < kQ * kN; e += kT) {
      const int j = e / kN, n = e % kN;
      if (j >= nv) continue;
      float ab = 0.f, ac = 0.f;
      for (int i = j; i < kQ; ++i) ab = fmaf(s.Lm[i * kQ + j] * s.DYX[i * kQ + j], s.C[bi(i, n)], ab);
      for (int k = 0; k <= j; ++k) ac = fmaf(s.Lm[j * kQ + k] * s.dt[k] * s.DYX[j * kQ + k], s.B[bi(k, n)], ac);
      float dcv = 0.f;  // e_j (S0^T dy_j)[n]
      for (int q = 0; q < kP; ++q) dcv = fmaf(s.S0[gi(q, n)], s.DY[xi(j, q)], dcv);
      const int64_t o = (((int64_t)b * p.L + t0 + j) * p.H + h) * kN + n;   // per-head partials
      p.ws_dB[o] = s.dt[j] * fmaf(s.fj[j], s.XG[e], ab);
      p.ws_dC[o] = fmaf(s.ei[j], dcv, ac);
    }
    if (tid < 64) {
      float dd = 0.f;
      for (int j = tid; j < kQ; j += 64) dd += s.DYX[j * kQ + j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dd += __shfl_xor(dd, off, 64);
      accD += dd;  // every lane of wave 0 holds the chunk's sum
    }
    __syncthreads();  // ddt complete
    if (tid < kQ && tid < nv) {
      const float dz = s.ddt[tid] * __builtin_amdgcn_rcpf(1.f + __expf(-s.z[tid]));
      reinterpret_cast<T *>(p.ddt)[((int64_t)b * p.L + t0 + tid) * p.H + h] = from_f32<T>(dz);
    }
    if (tid < 64) {
      float dz = 0.f;
      if (tid < kQ && tid < nv) dz = s.ddt[tid] * __builtin_amdgcn_rcpf(1.f + __expf(-s.z[tid]));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dz += __shfl_xor(dz, off, 64);
      accBias += dz;
    }
    // G0 = sum_i e_i dy_i C_i^T + e^{cs_Q} G1, in place (every read of G1 is done)
    for (int e = tid; e < kPN; e += kT) {
      const int q = e / kN, n = e % kN;
      float acc = eQ * s.G[gi(q, n)];
      for (int i = 0; i < kQ; ++i) acc = fmaf(s.ei[i] * s.DY[xi(i, q)], s.C[bi(i, n)], acc);
      s.G[gi(q, n)] = acc;
    }
    __syncthreads();
  }
  if (p.dinit)
    for (int e = tid; e < kPN; e += kT) p.dinit[((int64_t)b * p.H + h) * kPN + e] = s.G[gi(e / kN, e % kN)];
  if (tid == 0) {
    p.ws_scalars[((int64_t)b * p.H + h) * 3 + 0] = accA;
    p.ws_scalars[((int64_t)b * p.H + h) * 3 + 1] = accD;
    p.ws_scalars[((int64_t)b * p.H + h) * 3 + 2] = accBias;
  }
}

// -------------------------------------------------------------------------
// 3. fixed-order sums: dB, dC over the heads of a group; the per-head
//    scalars over the rows
// -------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void bwd_reduce_kernel(BwdParams p) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  const int hpg = p.H / p.G;
  const int64_t total = (int64_t)p.batch * p.L * p.G * kN;
  if (e < total) {
    const int n = (int)(e % kN);
    const int64_t r = e / kN;
    const int gi = (int)(r % p.G);
    const int64_t bt = r / p.G;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < hpg; ++k) {
      const int64_t o = (bt * p.H + gi * hpg + k) * kN + n;
      sb += p.ws_dB[o];
      sc += p.ws_dC[o];
    }
    reinterpret_cast<T *>(p.dB)[e] = from_f32<T>(sb);
    reinterpret_cast<T *>(p.dC)[e] = from_f32<T>(sc);
  }
  if (e < p.H) {
    float a = 0.f, d = 0.f, bi = 0.f;
    for (int b = 0; b < p.batch; ++b) {
      a += p.ws_scalars[((int64_t)b * p.H + e) * 3 + 0];
      d += p.ws_scalars[((int64_t)b * p.H + e) * 3 + 1];
      bi += p.ws_scalars[((int64_t)b * p.H + e) * 3 + 2];
    }
    p.dA[e] = a;
    if (p.dD) p.dD[e] = d;
    if (p.ddt_bias) p.ddt_bias[e] = bi;
  }
}

template <typename T>
hipError_t launch_t(const BwdParams &p, hipStream_t stream) {
  const unsigned units = (unsigned)(p.batch * p.H);
  hipLaunchKernelGGL(bwd_states_kernel<T>, dim3(units), dim3(kT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(BwdSmem);
  e = set_max_dynamic_lds(reinterpret_cast<const void *>(bwd_chunks_kernel<T>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_chunks_kernel<T>, dim3(units), dim3(kT), lds, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = std::max<int64_t>((int64_t)p.batch * p.L * p.G * kN, p.H);
  hipLaunchKernelGGL(bwd_reduce_kernel<T>, dim3((unsigned)((total + kT - 1) / kT)), dim3(kT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t bwd_lds_bytes() { return sizeof(BwdSmem); }

BwdLayout bwd_layout(int batch, int L, int H, int G) {
  BwdLayout w{};
  const int64_t nchunks = (L + kQ - 1) / kQ;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  w.nchunks = (int)nchunks;
  w.states_off = take(sizeof(float) * (size_t)batch * H * nchunks * kPN);
  w.dB_off = take(sizeof(float) * (size_t)batch * L * H * kN);
  w.dC_off = take(sizeof(float) * (size_t)batch * L * H * kN);
  w.scalars_off = take(sizeof(float) * (size_t)batch * H * 3);
  w.bytes = off;
  (void)G;
  return w;
}

hipError_t launch_chunk_scan_bwd(const BwdParams &p, hipStream_t stream) {
  if (p.batch * p.H == 0) return hipSuccess;
  return p.bf16 ? launch_t<bf16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace ssd
