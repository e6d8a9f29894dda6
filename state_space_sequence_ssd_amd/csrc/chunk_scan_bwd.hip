// Backward pass of the chunked SSD scan on gfx950 (batch rows, fp32 sums).
// The training workload of the layer needs the gradient of
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
//      forward with the state in the matrix-core accumulators and stores the
//      state entering each chunk (fp32, in the workspace).
//   2. bwd_chunks_kernel: one workgroup per (row, head) walks the chunks in
//      reverse; the adjoint G, the entering state and every chunk operand
//      live in LDS (fp32), and each product above is a tile loop of matrix-
//      core products: bf16 ones for bf16 inputs (fp32 intermediates split
//      into bf16 hi + lo parts), fp32 ones for fp32 inputs.  dB and dC are
//      written per head, the per-head scalars per (row, head).
//   3. bwd_reduce_kernel: dB, dC summed over the heads of each group and
//      dA, dD, ddt_bias over the rows, in a fixed order (no float atomics,
//      repeat runs are bitwise identical).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kQ = 32;      // tokens per backward chunk
constexpr int kT = 256;     // threads per workgroup
constexpr int kP = kHeadDim, kN = kDState;
constexpr int kPN = kP * kN;

// Inclusive prefix (suffix) sums over the 32 lanes of a half-wave: DPP row
// shifts within each 16-lane row (a source outside the row reads 0), then the
// upper (lower) row adds the other row's total.  Lanes 32..63 get no
// meaningful value.
template <int kCtrl> __device__ __forceinline__ float dpp_shift(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float prefix32(float v) {
  v += dpp_shift<0x111>(v);  // row_shr:1
  v += dpp_shift<0x112>(v);  // row_shr:2
  v += dpp_shift<0x114>(v);  // row_shr:4
  v += dpp_shift<0x118>(v);  // row_shr:8
  const float row0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  return (threadIdx.x & 16) ? v + row0 : v;
}
__device__ __forceinline__ float suffix32(float v) {
  v += dpp_shift<0x101>(v);  // row_shl:1
  v += dpp_shift<0x102>(v);  // row_shl:2
  v += dpp_shift<0x104>(v);  // row_shl:4
  v += dpp_shift<0x108>(v);  // row_shl:8
  const float row1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  return (threadIdx.x & 16) ? v : v + row1;
}

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
    static_assert(kQ == 32, "one half-wave scans the chunk");
    const float incl = prefix32(d * p.A[h]);
    if (lane < kQ) {
      s_dt[lane] = d;
      s_cs[lane] = incl;
      s_z[lane] = z;
    }
  }
}

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 inputs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16): lane
// (l16, kq) holds 8 K values of its operand row / column, and the
// accumulator layout is that of v_mfma_f32_16x16x4_f32 (rows 4 kq .. +3,
// column l16).  Operands that are bf16 numbers (x, dy, B, C) convert exactly;
// fp32 intermediates (the adjoint, the entering state, the masked token
// products) go in as bf16 parts hi = bf16(v), lo = bf16(v - hi), two
// products, so each carries about 16 bits.
// The K values of lane group kq in a 32-wide k-step are, in slot order e,
// 4 kq + (e & 3) + 16 (e >> 2) (any order works as long as both operands of
// a product use it).  With rows padded to 4 (mod 64) floats, a column read
// by the four groups then touches rows 4 apart, 16 banks apart, and the
// wave's 64 lanes fall on 64 banks; 8 consecutive K values per group put the
// groups' rows 8 apart, 32 banks apart: a two-way conflict on every read.
struct F8 {
  float v[8];
};
// slots 0..7 of group kq from a row whose k-step starts at p (16-byte aligned)
__device__ __forceinline__ F8 ld8(const float *p, int kq) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p + 4 * kq);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4 * kq + 16);
  return F8{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
}
// ... from a column (K rows kStride floats apart) whose k-step starts at p
template <int kStride> __device__ __forceinline__ F8 ld8s(const float *p, int kq) {
  F8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = p[(4 * kq + (e & 3) + 16 * (e >> 2)) * kStride];
  return f;
}
__device__ __forceinline__ bf16x8 exact8(const F8 &f) {
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = pack2_bf16(f.v[2 * k], f.v[2 * k + 1]);
  return __builtin_bit_cast(bf16x8, o);
}
struct Split8 {
  bf16x8 hi, lo;
};
__device__ __forceinline__ Split8 split8(const F8 &f) {
  u32x4 h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[k] = pack2_bf16(f.v[2 * k], f.v[2 * k + 1]);
    l[k] = pack2_bf16(f.v[2 * k] - lo_bf16(h[k]), f.v[2 * k + 1] - hi_bf16(h[k]));
  }
  return Split8{__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, l)};
}
__device__ __forceinline__ f32x4 mfma32k(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// exact operand times split operand (lo part first), either side
__device__ __forceinline__ f32x4 mfma_es(bf16x8 a, const Split8 &b, f32x4 c) {
  return mfma32k(a, b.hi, mfma32k(a, b.lo, c));
}
__device__ __forceinline__ f32x4 mfma_se(const Split8 &a, bf16x8 b, f32x4 c) {
  return mfma32k(a.hi, b, mfma32k(a.lo, b, c));
}

// Chunk operands move as 16-byte pieces: every thread issues all of its loads
// of a chunk before the first one is used, so a chunk waits for one memory
// latency, not one per element.
template <typename T> constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte piece

template <typename T>
__device__ __forceinline__ u32x4 ld16(const void *base, int64_t elem) {
  return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const T *>(base) + elem);
}

// the fp32 values of one piece into LDS, in aligned groups of 4 floats:
// columns q .. q + 3 to dst0 and (bf16 pieces) q + 4 .. q + 7 to dst1
template <typename T> __device__ __forceinline__ void st_piece(float *dst0, float *dst1, u32x4 v, float scale);
template <> __device__ __forceinline__ void st_piece<float>(float *dst0, float *, u32x4 v, float scale) {
  f32x4 f;
#pragma unroll
  for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]) * scale;
  *reinterpret_cast<f32x4 *>(dst0) = f;
}
template <> __device__ __forceinline__ void st_piece<bf16_t>(float *dst0, float *dst1, u32x4 v, float scale) {
  f32x4 lo, hi;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    lo[2 * k] = __uint_as_float(v[k] << 16) * scale;
    lo[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u) * scale;
    hi[2 * k] = __uint_as_float(v[k + 2] << 16) * scale;
    hi[2 * k + 1] = __uint_as_float(v[k + 2] & 0xffff0000u) * scale;
  }
  *reinterpret_cast<f32x4 *>(dst0) = lo;
  *reinterpret_cast<f32x4 *>(dst1) = hi;
}

// rows of `width` elements of one chunk (token rows t0 .. t0 + kQ - 1, row r
// at element offset r * row_st); piece i of this thread covers row
// (v * kVec) / width, columns (v * kVec) % width .., v = tid + kT i.  Rows
// past nv read nothing and hold zeros.
template <typename T, int width, int kThreads = kT>
struct ChunkRows {
  static constexpr int kTotal = kQ * width / kVec<T>;                  // pieces of the chunk
  static constexpr int kPieces = (kTotal + kThreads - 1) / kThreads;  // per thread
  u32x4 v[kPieces];
  __device__ __forceinline__ void load(const void *base, int64_t first, int64_t row_st, int nv, int tid) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + kThreads * i, e = pc * kVec<T>, j = e / width, q = e % width;
      v[i] = (pc < kTotal && j < nv) ? ld16<T>(base, first + j * row_st + q) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // into an LDS tile: element (j, q) at tile[idx(j, q)], 4-float groups
  // aligned and contiguous; scale(j) weights row j
  template <typename FI, typename F>
  __device__ __forceinline__ void store_at(float *tile, int tid, FI idx, F scale) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + kThreads * i, e = pc * kVec<T>, j = e / width, q = e % width;
      if (pc < kTotal) st_piece<T>(tile + idx(j, q), tile + idx(j, q + 4), v[i], scale(j));
    }
  }
  // ... with row pitch `pitch` floats
  template <int pitch, typename F>
  __device__ __forceinline__ void store(float *tile, int tid, F scale) const {
    store_at(tile, tid, [](int j, int q) { return j * pitch + q; }, scale);
  }
};

// NS k-steps of matrix-core products: load(s) reads step s's operands from
// LDS into an R, mma(R) issues its products.  Step s + 1's reads go out
// while step s's products run, so the matrix core does not wait for each
// step's reads (the last step's operands are read twice rather than
// branching).
template <int NS, typename R, typename FL, typename FM>
__device__ __forceinline__ void pipelined(FL load, FM mma) {
  R cur = load(0);
#pragma unroll 2
  for (int st = 0; st < NS; ++st) {
    const R nxt = load(st + 1 < NS ? st + 1 : NS - 1);
    mma(cur);
    cur = nxt;
    // keeps each step's reads in their own iteration: without it the
    // compiler folds the rotation back into read-then-multiply
    asm volatile("" ::: "memory");
  }
}

// -------------------------------------------------------------------------
// 1. the state entering every chunk
// -------------------------------------------------------------------------
// S <- e^{cs_Q} S + sum_j w_j x_j B_j^T on the fp32 matrix cores: the state
// (64 x 128) is 32 tiles of 16 x 16, eight per wave, kept in the
// accumulators; per chunk each tile takes 8 steps of v_mfma_f32_16x16x4_f32
// (k = token).  Lane roles: operand row l16, k slot kq; the accumulator
// holds rows 4 kq .. 4 kq + 3, column l16.
// The tiles are read with the token (k) on the lane's k slot and the column
// on its 16-lane index: rows padded to 16 (mod 64) floats put the four k
// slots on four different 16-bank groups.
// The workspace keeps each chunk's entering state in the order the states
// pass holds it: float4 number (8 w + t) 64 + lane is rows 16 w + 4 kq .. + 3
// of column 16 t + l16 (wave w, tile t, lane = 16 kq + l16), so every store
// is a whole 16-byte vector and each store instruction writes 1 KiB in a
// row.  Only the reverse pass reads it back (state_elem gives the element).
__device__ __forceinline__ void store_state(float *dst, const f32x4 *acc, int wave, int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4 *>(dst + 4 * ((8 * wave + t) * 64 + lane)) = acc[t];
}
// bf16 inputs: the same order with each float4 rounded to four bf16 (8 bytes,
// 512 B per store instruction).  The reverse pass's products with the
// entering state then take it as one bf16 operand, as the forward pass's
// state->output product takes its bf16 copy of the state.
__device__ __forceinline__ void store_state_bf16(bf16_t *dst, const f32x4 *acc, int wave, int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u32x2 v;
    v[0] = pack2_bf16(acc[t][0], acc[t][1]);
    v[1] = pack2_bf16(acc[t][2], acc[t][3]);
    *reinterpret_cast<u32x2 *>(dst + 4 * ((8 * wave + t) * 64 + lane)) = v;
  }
}
// row p and column n of float4 number f of a stored state (its element r is row p + r)
__device__ __forceinline__ void state_elem(int f, int &p, int &n) {
  const int w = f >> 9, t = (f >> 6) & 7, ln = f & 63;
  p = 16 * w + 4 * (ln >> 4);
  n = 16 * t + (ln & 15);
}

constexpr int kXSP = kP + 16;   // padded rows of the staged x (w x) and B tiles
constexpr int kBSP = kN + 16;
template <typename T>
__global__ __launch_bounds__(kT) void bwd_states_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) float sX[kQ * kXSP], sB[kQ * kBSP];
  __shared__ float s_dt[kQ], s_cs[kQ], s_z[kQ];
  const int b = blockIdx.x / p.H, h = blockIdx.x % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, kq = lane >> 4;
  float *states = p.ws_states + ((int64_t)b * p.H + h) * p.nchunks * kPN;
  // this wave's tiles: rows p in [16 wave, +16), columns n in [16 t, +16), t = 0..7
  f32x4 acc[8];
  const float *h0 = p.init ? p.init + ((int64_t)b * p.H + h) * kPN : nullptr;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = h0 ? h0[(16 * wave + 4 * kq + r) * kN + 16 * t + l16] : 0.f;
  // B and x of chunk c + 1 are loaded while chunk c is multiplied
  ChunkRows<T, kN> rb;
  ChunkRows<T, kP> rx;
  const auto load_chunk = [&](int c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
    rb.load(p.B, (((int64_t)b * p.L + t0) * p.G + g) * kN, (int64_t)p.G * kN, nv, tid);
    rx.load(p.x, (((int64_t)b * p.L + t0) * p.H + h) * kP, (int64_t)p.H * kP, nv, tid);
  };
  if (p.nchunks > 0) load_chunk(0);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
    // the state entering this chunk, in the accumulators' own order
    store_state(states + (int64_t)c * kPN, acc, wave, lane);
    chunk_dt<T>(p, b, h, t0, nv, s_dt, s_cs, s_z);
    rb.template store<kBSP>(sB, tid, [](int) { return 1.f; });
    __syncthreads();  // dt, cs
    const float last = s_cs[kQ - 1];
    rx.template store<kXSP>(sX, tid, [&](int j) { return __expf(last - s_cs[j]) * s_dt[j]; });  // w_j x_j
    __syncthreads();
    if (c + 1 < p.nchunks) load_chunk(c + 1);
    const float dec = __expf(last);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= dec;
#pragma unroll
    for (int k0 = 0; k0 < kQ; k0 += 4) {
      const float a = sX[(k0 + kq) * kXSP + 16 * wave + l16];  // (w x)^T: row p, k = token
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = mfma16(a, sB[(k0 + kq) * kBSP + 16 * t + l16], acc[t]);
    }
    __syncthreads();  // the tiles are rewritten by the next chunk
  }
}

// bf16 inputs: the same recurrence on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16: the chunk's 32 tokens are one k-step).  B is
// exact in bf16; w_j x_j is split into bf16 parts hi = bf16(v) and lo =
// bf16(v - hi), so the two products carry w x to about 2^-16 of its size,
// far below the rounding of the bf16 inputs themselves.  The tiles stay
// token-major in LDS (rows padded by 32 bytes) and the operands, whose K runs
// over tokens, come from the LDS transpose read: in each 16-lane group lane s
// points at token row k0 + s / 4, columns c0 + 4 (s % 4) .. + 3, and receives
// tokens k0 .. k0 + 3 of column c0 + s.  Group kq takes tokens 4 kq .. + 3
// and 16 + 4 kq .. + 3 (the same order in both operands), so one read by the
// four groups covers 16 consecutive rows; with rows 8 or 40 banks apart (288-
// and 160-byte rows) those fall on distinct banks, where tokens 8 kq .. + 7
// put rows 8 apart on the same banks.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
constexpr int kXR = 2 * kP + 32, kBR = 2 * kN + 32;  // bytes per staged row
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t *tile, int pitch, int k0, int c0, int lane) {
  const int s = lane & 15;
  const uint8_t *a = tile + (k0 + (s >> 2)) * pitch + 2 * (c0 + 4 * (s & 3));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)a);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a + 16 * pitch));
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], h[0], h[1]});
}
__global__ __launch_bounds__(kT) void bwd_states_bf16_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sXh[kQ * kXR], sXl[kQ * kXR], sB[kQ * kBR];
  __shared__ float s_dt[kQ], s_cs[kQ], s_z[kQ];
  const int b = blockIdx.x / p.H, h = blockIdx.x % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, kq = lane >> 4;
  bf16_t *states = reinterpret_cast<bf16_t *>(p.ws_states) + ((int64_t)b * p.H + h) * p.nchunks * kPN;
  // this wave's tiles: rows p in [16 wave, +16), columns n in [16 t, +16), t = 0..7
  f32x4 acc[8];
  const float *h0 = p.init ? p.init + ((int64_t)b * p.H + h) * kPN : nullptr;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = h0 ? h0[(16 * wave + 4 * kq + r) * kN + 16 * t + l16] : 0.f;
  ChunkRows<bf16_t, kN> rb;
  ChunkRows<bf16_t, kP> rx;
  const auto load_chunk = [&](int c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
    rb.load(p.B, (((int64_t)b * p.L + t0) * p.G + g) * kN, (int64_t)p.G * kN, nv, tid);
    rx.load(p.x, (((int64_t)b * p.L + t0) * p.H + h) * kP, (int64_t)p.H * kP, nv, tid);
  };
  if (p.nchunks > 0) load_chunk(0);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
    store_state_bf16(states + (int64_t)c * kPN, acc, wave, lane);
    chunk_dt<bf16_t>(p, b, h, t0, nv, s_dt, s_cs, s_z);
#pragma unroll
    for (int i = 0; i < rb.kPieces; ++i) {
      const int pc = tid + kT * i, e = pc * 8, j = e / kN, q = e % kN;
      if (pc < rb.kTotal) *reinterpret_cast<u32x4 *>(sB + j * kBR + 2 * q) = rb.v[i];
    }
    __syncthreads();  // dt, cs
    const float last = s_cs[kQ - 1];
#pragma unroll
    for (int i = 0; i < rx.kPieces; ++i) {
      const int pc = tid + kT * i, e = pc * 8, j = e / kP, q = e % kP;
      if (pc < rx.kTotal) {
        const float w = __expf(last - s_cs[j]) * s_dt[j];
        u32x4 hv, lv;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v0 = lo_bf16(rx.v[i][k]) * w, v1 = hi_bf16(rx.v[i][k]) * w;
          hv[k] = pack2_bf16(v0, v1);
          lv[k] = pack2_bf16(v0 - lo_bf16(hv[k]), v1 - hi_bf16(hv[k]));
        }
        *reinterpret_cast<u32x4 *>(sXh + j * kXR + 2 * q) = hv;
        *reinterpret_cast<u32x4 *>(sXl + j * kXR + 2 * q) = lv;
      }
    }
    __syncthreads();
    if (c + 1 < p.nchunks) load_chunk(c + 1);
    const float dec = __expf(last);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= dec;
    // A = (w x)^T (rows p, K = tokens), B = B (K = tokens, columns n)
    const bf16x8 ah = tr_frag(sXh, kXR, 4 * kq, 16 * wave, lane);
    const bf16x8 al = tr_frag(sXl, kXR, 4 * kq, 16 * wave, lane);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8 bt = tr_frag(sB, kBR, 4 * kq, 16 * t, lane);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bt, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bt, acc[t], 0, 0, 0);
    }
    __syncthreads();  // the tiles are rewritten by the next chunk
  }
}

// -------------------------------------------------------------------------
// 2. the chunks in reverse
// -------------------------------------------------------------------------
// Every product of the chunked formulas runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: fp32 products, fp32 sums).  Rows of the LDS tiles
// are padded to 4 (mod 64) floats, so the 16 rows x 4 k values of one
// operand read (rows on the lane's 16-lane index) fall on 64 different
// banks.  (An XOR swizzle that also spreads the reads with the rows on the
// k slot cost more in address arithmetic than the bank conflicts it removed.)
constexpr int kNP = kN + 4, kPP = kP + 4, kQP = kQ + 4;
__device__ __forceinline__ int gi(int q, int n) { return q * kNP + n; }   // G, S0: [p][n]
__device__ __forceinline__ int bi(int j, int n) { return j * kNP + n; }   // B, C: [token][n]
__device__ __forceinline__ int xi(int j, int q) { return j * kPP + q; }   // X, DY: [token][p]
__device__ __forceinline__ int qi(int i, int j) { return i * kQP + j; }   // CB, DYX, Lm, W: [token][token]

// Eight waves (two per SIMD, so one wave's LDS waits are covered by the
// other's matrix-core work).  Wave w's tiles, in 16 x 16 blocks:
//   token x token (C B^T for w < 4, dy x^T for w >= 4): rows 16 ((w % 4) / 2), columns 16 (w % 2)
//   G1 B, S0 C, dx: token rows 16 mj (mj = w / 4), p columns 16 qb (qb = w % 4)
//   x G1, dB, dC: token rows 16 mj, n columns 16 (2 qb + t), t < 2
//   G0: p rows 16 qb, n columns 16 (4 mj + t), t < 4
constexpr int kTC = 512;
struct BwdSmem {
  float G[kP * kNP];   // adjoint dL/dS leaving the chunk (G1), then entering (G0)
  float S0[kP * kNP];  // state entering the chunk
  float X[kQ * kPP], DY[kQ * kPP], B[kQ * kNP], C[kQ * kNP];
  float CB[kQ * kQP], DYX[kQ * kQP];               // C_i . B_j, dy_i . x_j
  float Lm[kQ * kQP];                              // e^{cs_i - cs_j} for j <= i, else 0
  float xgb_part[4][kQ];                           // per 32-column block: x_j . (G1 B_j)
  float ey_part[4][kQ];                            // per 16-column block: dy_j . (S0 C_j)
  float wcol[16][kQ], wrow[16][kQ];                // per 2-token part: column / dt-weighted row sums of W
  float dt[kQ], cs[kQ], z[kQ], ei[kQ], fj[kQ], red[kTC / 64];
};

template <typename T>
__global__ __launch_bounds__(kTC) void bwd_chunks_kernel(BwdParams p) {
  constexpr bool kBf = std::is_same<T, bf16_t>::value;  // bf16 inputs: the bf16 matrix cores
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  BwdSmem &s = *reinterpret_cast<BwdSmem *>(smem_raw);
  const int b = blockIdx.x / p.H, h = blockIdx.x % p.H, g = h / (p.H / p.G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, kq = lane >> 4;
  const float Ah = p.A[h], Dh = p.D ? p.D[h] : 0.f;
  const int64_t st0 = ((int64_t)b * p.H + h) * p.nchunks * kPN;  // this (row, head)'s states
  for (int e = tid; e < kPN; e += kTC)
    s.G[gi(e / kN, e % kN)] = p.dfinal ? p.dfinal[((int64_t)b * p.H + h) * kPN + e] : 0.f;
  float accA = 0.f, accD = 0.f, accBias = 0.f;
  const bool has_cb = wave < 4;                             // C B^T (else dy x^T)
  const int mi = (wave & 3) >> 1, ni = wave & 1;            // its token x token block
  const int mj = wave >> 2, qb = wave & 3, nb0 = 2 * qb, gn0 = 4 * mj;
  const int jr = 16 * mj + l16;                             // the lane's operand row in the token blocks
  __syncthreads();

  for (int c = p.nchunks - 1; c >= 0; --c) {
    const int t0 = c * kQ, nv = min(kQ, p.L - t0);
    // operands of the chunk (rows past the end are zero; their dt is 0)
    {
      constexpr int kS0 = kPN / 4 / kTC;
      f32x4 s0[kS0];
      if constexpr (kBf) {
        // four bf16 per float4 number (the bf16 states pass's format)
        const bf16_t *states = reinterpret_cast<const bf16_t *>(p.ws_states) + st0 + (int64_t)c * kPN;
        u32x2 sb[kS0];
#pragma unroll
        for (int i = 0; i < kS0; ++i) sb[i] = *reinterpret_cast<const u32x2 *>(states + 4 * (tid + kTC * i));
#pragma unroll
        for (int i = 0; i < kS0; ++i) {
          s0[i][0] = lo_bf16(sb[i][0]);
          s0[i][1] = hi_bf16(sb[i][0]);
          s0[i][2] = lo_bf16(sb[i][1]);
          s0[i][3] = hi_bf16(sb[i][1]);
        }
      } else {
        const float *states = p.ws_states + st0 + (int64_t)c * kPN;
#pragma unroll
        for (int i = 0; i < kS0; ++i) s0[i] = *reinterpret_cast<const f32x4 *>(states + 4 * (tid + kTC * i));
      }
      ChunkRows<T, kP, kTC> rx, rdy;
      ChunkRows<T, kN, kTC> rb, rc;
      const int64_t xo = (((int64_t)b * p.L + t0) * p.H + h) * kP, bo = (((int64_t)b * p.L + t0) * p.G + g) * kN;
      rx.load(p.x, xo, (int64_t)p.H * kP, nv, tid);
      rdy.load(p.dy, xo, (int64_t)p.H * kP, nv, tid);
      rb.load(p.B, bo, (int64_t)p.G * kN, nv, tid);
      rc.load(p.C, bo, (int64_t)p.G * kN, nv, tid);
      chunk_dt<T>(p, b, h, t0, nv, s.dt, s.cs, s.z);
#pragma unroll
      for (int i = 0; i < kS0; ++i) {
        int sp, sn;
        state_elem(tid + kTC * i, sp, sn);
#pragma unroll
        for (int r = 0; r < 4; ++r) s.S0[gi(sp + r, sn)] = s0[i][r];
      }
      const auto one = [](int) { return 1.f; };
      rx.store_at(s.X, tid, xi, one);
      rdy.store_at(s.DY, tid, xi, one);
      rb.store_at(s.B, tid, bi, one);
      rc.store_at(s.C, tid, bi, one);
    }
    __syncthreads();
    for (int e = tid; e < kQ * kQ; e += kTC) {
      const int i = e / kQ, j = e % kQ;
      s.Lm[qi(i, j)] = j <= i ? __expf(s.cs[i] - s.cs[j]) : 0.f;
    }
    if (tid < kQ) {
      s.ei[tid] = __expf(s.cs[tid]);
      s.fj[tid] = __expf(s.cs[kQ - 1] - s.cs[tid]);
    }

    // ---- phase 1: C B^T or dy x^T (one 16 x 16 block), G1 B and S0 C (rows
    // j, columns p), x G1 (rows j, columns n) ----
    f32x4 gb, s0c, xg[2];  // G1 B and x G1 are kept for dx and dB
    {
      f32x4 tt = f32x4{};  // the token x token block
      gb = s0c = xg[0] = xg[1] = f32x4{};
      if constexpr (kBf) {
        // over n: 4 k-steps of 32 (rows of every tile, 8 consecutive n per lane)
#pragma unroll
        for (int st = 0; st < kN / 32; ++st) {
          const int n0 = 32 * st;
          if (has_cb)
            tt = mfma32k(exact8(ld8(&s.C[bi(16 * mi + l16, n0)], kq)), exact8(ld8(&s.B[bi(16 * ni + l16, n0)], kq)), tt);
          gb = mfma_es(exact8(ld8(&s.B[bi(jr, n0)], kq)), split8(ld8(&s.G[gi(16 * qb + l16, n0)], kq)), gb);
          // S0 holds the bf16 states pass's values, exact in bf16: one product
          s0c = mfma32k(exact8(ld8(&s.C[bi(jr, n0)], kq)), exact8(ld8(&s.S0[gi(16 * qb + l16, n0)], kq)), s0c);
        }
        // over p: 2 k-steps of 32; G1's columns are read down the p rows
#pragma unroll
        for (int st = 0; st < kP / 32; ++st) {
          const int p0 = 32 * st;
          if (!has_cb)
            tt = mfma32k(exact8(ld8(&s.DY[xi(16 * mi + l16, p0)], kq)), exact8(ld8(&s.X[xi(16 * ni + l16, p0)], kq)), tt);
          const bf16x8 xr = exact8(ld8(&s.X[xi(jr, p0)], kq));
#pragma unroll
          for (int t = 0; t < 2; ++t)
            xg[t] = mfma_es(xr, split8(ld8s<kNP>(&s.G[gi(p0, 16 * (nb0 + t) + l16)], kq)), xg[t]);
        }
      } else {
      // contractions over n: C B^T (waves 0..3), B G1^T, C S0^T
      struct RN { float c_i, b_j, b_r, c_r, g, s0; };
      pipelined<kN / 4, RN>(
          [&](int st) {
            const int k = 4 * st + kq;
            RN o;
            o.c_i = has_cb ? s.C[bi(16 * mi + l16, k)] : 0.f;
            o.b_j = has_cb ? s.B[bi(16 * ni + l16, k)] : 0.f;
            o.b_r = s.B[bi(jr, k)];
            o.c_r = s.C[bi(jr, k)];
            o.g = s.G[gi(16 * qb + l16, k)];
            o.s0 = s.S0[gi(16 * qb + l16, k)];
            return o;
          },
          [&](const RN &o) {
            if (has_cb) tt = mfma16(o.c_i, o.b_j, tt);
            gb = mfma16(o.b_r, o.g, gb);
            s0c = mfma16(o.c_r, o.s0, s0c);
          });
      // contractions over p: dy x^T (waves 4..7), x G1
      struct RP { float dy_i, x_j, x_r, g[2]; };
      pipelined<kP / 4, RP>(
          [&](int st) {
            const int k = 4 * st + kq;
            RP o;
            o.dy_i = has_cb ? 0.f : s.DY[xi(16 * mi + l16, k)];
            o.x_j = has_cb ? 0.f : s.X[xi(16 * ni + l16, k)];
            o.x_r = s.X[xi(jr, k)];
#pragma unroll
            for (int t = 0; t < 2; ++t) o.g[t] = s.G[gi(k, 16 * (nb0 + t) + l16)];
            return o;
          },
          [&](const RP &o) {
            if (!has_cb) tt = mfma16(o.dy_i, o.x_j, tt);
#pragma unroll
            for (int t = 0; t < 2; ++t) xg[t] = mfma16(o.x_r, o.g[t], xg[t]);
          });
      }
      float *ttd = has_cb ? s.CB : s.DYX;
#pragma unroll
      for (int r = 0; r < 4; ++r) ttd[qi(16 * mi + 4 * kq + r, 16 * ni + l16)] = tt[r];
      // per-token partial dot products over this wave's columns: the lane
      // holds rows j = 16 mj + 4 kq + r, column l16 of each block; its blocks
      // are summed in the lane, then over the 16 lanes of the row
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * mj + 4 * kq + r;
        float ve = s0c[r] * s.DY[xi(j, 16 * qb + l16)], vx = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) vx = fmaf(xg[t][r], s.B[bi(j, 16 * (nb0 + t) + l16)], vx);
        ve = row_sum16(ve);
        vx = row_sum16(vx);
        if (l16 == 0) {
          s.ey_part[qb][j] = ve;
          s.xgb_part[qb][j] = vx;
        }
      }
    }
    {
      // <G1, S0>, 16-byte reads
      f32x4 acc4 = f32x4{};
#pragma unroll
      for (int i = 0; i < kPN / 4 / kTC; ++i) {
        const int e = 4 * (tid + kTC * i);
        const f32x4 gv = *reinterpret_cast<const f32x4 *>(&s.G[gi(e / kN, e % kN)]);
        const f32x4 sv = *reinterpret_cast<const f32x4 *>(&s.S0[gi(e / kN, e % kN)]);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc4[k] = fmaf(gv[k], sv[k], acc4[k]);
      }
      const float gs = wave_sum((acc4[0] + acc4[1]) + (acc4[2] + acc4[3]));
      if (lane == 0) s.red[wave] = gs;
    }
    __syncthreads();

    // ---- phase 2: per-token scalars ----
    {
      // W_ij = Lm_ij CB_ij DYX_ij: thread (part, j) sums column j over rows
      // i in [2 part, +2) and row j over columns k in [2 part, +2), weighted by dt_k
      const int j = tid & 31, part = tid >> 5;
      float cp = 0.f, rp = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 2 * part + u;
        cp = fmaf(s.Lm[qi(i, j)] * s.CB[qi(i, j)], s.DYX[qi(i, j)], cp);
        rp = fmaf(s.Lm[qi(j, i)] * s.CB[qi(j, i)] * s.DYX[qi(j, i)], s.dt[i], rp);
      }
      s.wcol[part][j] = cp;
      s.wrow[part][j] = rp;
    }
    __syncthreads();
    float G1S0 = 0.f;
#pragma unroll
    for (int w = 0; w < kTC / 64; ++w) G1S0 += s.red[w];
    const float eQ = s.ei[kQ - 1];
    if (wave == 0) {
      const int j = lane & 31;
      float dcs = 0.f, dexp = 0.f, tot_part = 0.f, dtj = 0.f;
      if (lane < 32) {
        float acc = 0.f, row = 0.f;  // sum_{i>=j} W_ij and sum_{k<=j} W_jk dt_k
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          acc += s.wcol[t][j];
          row += s.wrow[t][j];
        }
        const float fj = s.fj[j];
        dtj = s.dt[j];
        float xgb = 0.f, ey = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          xgb += s.xgb_part[t][j];
          ey += s.ey_part[t][j];
        }
        dexp = fmaf(fj, xgb, acc);                               // f_j x_j.(G1 B_j) + sum_{i>=j} W_ij
        dcs = s.ei[j] * ey + row - dtj * acc - fj * dtj * xgb;
        tot_part = fj * dtj * xgb;
      }
      // the last token also carries e^{cs_Q} <G1, S0> + sum_j f_j dt_j x_j.(G1 B_j)
      const float tot = half_wave_sum(tot_part);
      if (lane == kQ - 1) dcs += fmaf(eQ, G1S0, tot);
      // suffix sums over the chunk's tokens: suf_j = sum_{k>=j} dcs_k
      const float suf = suffix32(lane < 32 ? dcs : 0.f);
      const float da = half_wave_sum(lane < 32 ? dtj * suf : 0.f);
      accA += da;  // lanes 0..31 hold the chunk's sum
      if (lane < 32) {
        const float ddt = fmaf(Ah, suf, dexp);
        float dz = 0.f;
        if (j < nv) {
          dz = ddt * __builtin_amdgcn_rcpf(1.f + __expf(-s.z[j]));
          reinterpret_cast<T *>(p.ddt)[((int64_t)b * p.L + t0 + j) * p.H + h] = from_f32<T>(dz);
        }
        accBias += half_wave_sum(dz);
        accD += half_wave_sum(s.DYX[qi(j, j)]);
      }
    }

    // ---- phase 3: dx, dB, dC (this wave's blocks) and G0 (rows p in [16 qb, +16)) ----
    {
      // dx[j][q] = D dy_j[q] + dt_j (f_j (G1 B_j)[q] + sum_{i>=j} Lm_ij CB_ij dy_i[q]);
      // dB[j][n] = dt_j (f_j (x_j G1)[n] + sum_{i>=j} Lm_ij DYX_ij C_i[n]);
      // dC[j][n] = e_j (S0^T dy_j)[n] + sum_{k<=j} Lm_jk dt_k DYX_jk B_k[n];
      // G0[q][n] = e^{cs_Q} G1[q][n] + sum_i e_i dy_i[q] C_i[n], in place: this wave
      // reads and writes only its own blocks of G, and no other product reads G now
      f32x4 ax = f32x4{}, ab[2], ac[2], g0[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) ab[t] = ac[t] = f32x4{};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) g0[t][r] = eQ * s.G[gi(16 * qb + 4 * kq + r, 16 * (gn0 + t) + l16)];
      if constexpr (kBf) {
        // over the chunk's 32 tokens: one k-step, 8 tokens per lane group
        const F8 lm = ld8s<kQP>(&s.Lm[qi(0, jr)], kq), cb = ld8s<kQP>(&s.CB[qi(0, jr)], kq),
                 dyx = ld8s<kQP>(&s.DYX[qi(0, jr)], kq), dy = ld8s<kPP>(&s.DY[xi(0, 16 * qb + l16)], kq);
        const F8 lr = ld8(&s.Lm[qi(jr, 0)], kq), dr = ld8(&s.DYX[qi(jr, 0)], kq), dtk = ld8(&s.dt[0], kq),
                 ek = ld8(&s.ei[0], kq);
        F8 lcb, ldyx, ldt, edy;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lcb.v[e] = lm.v[e] * cb.v[e];
          ldyx.v[e] = lm.v[e] * dyx.v[e];
          ldt.v[e] = lr.v[e] * dtk.v[e] * dr.v[e];
          edy.v[e] = ek.v[e] * dy.v[e];
        }
        ax = mfma_se(split8(lcb), exact8(dy), ax);
        const Split8 sdyx = split8(ldyx), sdt = split8(ldt), sedy = split8(edy);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          ab[t] = mfma_se(sdyx, exact8(ld8s<kNP>(&s.C[bi(0, 16 * (nb0 + t) + l16)], kq)), ab[t]);
          ac[t] = mfma_se(sdt, exact8(ld8s<kNP>(&s.B[bi(0, 16 * (nb0 + t) + l16)], kq)), ac[t]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          g0[t] = mfma_se(sedy, exact8(ld8s<kNP>(&s.C[bi(0, 16 * (gn0 + t) + l16)], kq)), g0[t]);
        // ... and over p (2 k-steps): the e_j S0^T dy_j term of dC
        const float ej = s.ei[jr];
#pragma unroll
        for (int st = 0; st < kP / 32; ++st) {
          const int p0 = 32 * st;
          F8 a = ld8(&s.DY[xi(jr, p0)], kq);
#pragma unroll
          for (int e = 0; e < 8; ++e) a.v[e] *= ej;
          const Split8 sa = split8(a);
#pragma unroll
          for (int t = 0; t < 2; ++t)
            ac[t] = mfma_se(sa, exact8(ld8s<kNP>(&s.S0[gi(p0, 16 * (nb0 + t) + l16)], kq)), ac[t]);  // S0 exact
        }
      } else {
      // contractions over the chunk's tokens (k); dy_k[16 qb + l16] is both the
      // B operand of dx and, times e_k, the A operand of G0
      struct RQ { float lcb, ldyx, ldt, ek, dy, cb[2], cg[4], bb[2]; };
      pipelined<kQ / 4, RQ>(
          [&](int st) {
            const int k = 4 * st + kq;
            RQ o;
            const float lkj = s.Lm[qi(k, jr)];
            o.lcb = lkj * s.CB[qi(k, jr)];
            o.ldyx = lkj * s.DYX[qi(k, jr)];
            o.ldt = s.Lm[qi(jr, k)] * s.dt[k] * s.DYX[qi(jr, k)];
            o.ek = s.ei[k];
            o.dy = s.DY[xi(k, 16 * qb + l16)];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              o.cb[t] = s.C[bi(k, 16 * (nb0 + t) + l16)];
              o.bb[t] = s.B[bi(k, 16 * (nb0 + t) + l16)];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) o.cg[t] = s.C[bi(k, 16 * (gn0 + t) + l16)];
            return o;
          },
          [&](const RQ &o) {
            ax = mfma16(o.lcb, o.dy, ax);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              ab[t] = mfma16(o.ldyx, o.cb[t], ab[t]);
              ac[t] = mfma16(o.ldt, o.bb[t], ac[t]);
            }
            const float edy = o.ek * o.dy;
#pragma unroll
            for (int t = 0; t < 4; ++t) g0[t] = mfma16(edy, o.cg[t], g0[t]);
          });
      // ... and over p: the e_j S0^T dy_j term of dC
      const float ej = s.ei[jr];
      struct RS { float edy, s0[2]; };
      pipelined<kP / 4, RS>(
          [&](int st) {
            const int q = 4 * st + kq;
            RS o;
            o.edy = ej * s.DY[xi(jr, q)];
#pragma unroll
            for (int t = 0; t < 2; ++t) o.s0[t] = s.S0[gi(q, 16 * (nb0 + t) + l16)];
            return o;
          },
          [&](const RS &o) {
#pragma unroll
            for (int t = 0; t < 2; ++t) ac[t] = mfma16(o.edy, o.s0[t], ac[t]);
          });
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) s.G[gi(16 * qb + 4 * kq + r, 16 * (gn0 + t) + l16)] = g0[t][r];
      // outputs: the lane holds rows j = 16 mj + 4 kq + r, column l16 of each block
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * mj + 4 * kq + r;
        if (j >= nv) continue;
        const float dtj = s.dt[j], fj = s.fj[j];
        const int q = 16 * qb + l16;
        const float v = fmaf(Dh, s.DY[xi(j, q)], dtj * fmaf(fj, gb[r], ax[r]));
        reinterpret_cast<T *>(p.dx)[(((int64_t)b * p.L + t0 + j) * p.H + h) * kP + q] = from_f32<T>(v);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int n = 16 * (nb0 + t) + l16;
          const int64_t o = (((int64_t)b * p.L + t0 + j) * p.H + h) * kN + n;   // per-head partials
          p.ws_dB[o] = dtj * fmaf(fj, xg[t][r], ab[t][r]);
          p.ws_dC[o] = ac[t][r];
        }
      }
    }
    __syncthreads();  // G0 complete; the chunk's tiles are rewritten by the next chunk
  }
  if (p.dinit)
    for (int e = tid; e < kPN; e += kTC) p.dinit[((int64_t)b * p.H + h) * kPN + e] = s.G[gi(e / kN, e % kN)];
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
// four consecutive outputs (element e, a multiple of 4) in one store
template <typename T> __device__ __forceinline__ void store4(void *base, int64_t e, f32x4 v);
template <> __device__ __forceinline__ void store4<float>(void *base, int64_t e, f32x4 v) {
  *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(base) + e) = v;
}
template <> __device__ __forceinline__ void store4<bf16_t>(void *base, int64_t e, f32x4 v) {
  *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16_t *>(base) + e) = u32x2{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
}

// Each thread sums 4 consecutive n of one (row, token, group) over the
// group's heads, in head order: 16-byte loads of the partials (read once,
// non-temporal) and one store per output vector.
template <typename T>
__global__ __launch_bounds__(kT) void bwd_reduce_kernel(BwdParams p) {
  const int64_t tid = (int64_t)blockIdx.x * kT + threadIdx.x;
  const int hpg = p.H / p.G;
  const int64_t total4 = (int64_t)p.batch * p.L * p.G * kN / 4;
  if (tid < total4) {
    const int64_t e = 4 * tid;
    const int n = (int)(e % kN);
    const int64_t r = e / kN;
    const int gi = (int)(r % p.G);
    const int64_t bt = r / p.G;
    f32x4 sb = f32x4{}, sc = f32x4{};
    for (int k = 0; k < hpg; ++k) {
      const int64_t o = (bt * p.H + gi * hpg + k) * kN + n;
      sb += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.ws_dB + o));
      sc += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.ws_dC + o));
    }
    store4<T>(p.dB, e, sb);
    store4<T>(p.dC, e, sc);
  }
  const int64_t e = tid;
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
  if constexpr (std::is_same<T, bf16_t>::value)
    hipLaunchKernelGGL(bwd_states_bf16_kernel, dim3(units), dim3(kT), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_states_kernel<T>, dim3(units), dim3(kT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(BwdSmem);
  e = set_max_dynamic_lds(reinterpret_cast<const void *>(bwd_chunks_kernel<T>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_chunks_kernel<T>, dim3(units), dim3(kTC), lds, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = std::max<int64_t>((int64_t)p.batch * p.L * p.G * kN / 4, p.H);
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
