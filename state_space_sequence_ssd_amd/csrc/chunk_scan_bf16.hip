// Chunked SSD prefill, bf16 inputs: the fused MFMA chunk kernel for gfx950.
//
// Per head, a chunk of Q = 128 tokens with inclusive in-chunk cumulative
// log-decay cs_i = sum_{k<=i} dt_k A (scalar-times-identity transition of
// Mamba-2: "Mamba-3: an inference-first state space model"; the block form
// is the state space duality of "AI Engineering EP6", sec. 8 and 10; chunk
// 128 from "Nemotron-H style Hybrid Mamba-Transformer 3B feasibility
// study", sec. 1.4) is
//
//   G      = B C^T                                   (C B^T, K = d_state)
//   M[i][j] = G[j][i] exp(cs_i - cs_j) dt_j  (j <= i)
//   y      = exp(cs_i) (C_i H_prev^T)  +  sum_j M[i][j] x_j  +  D x_i
//   H      = exp(cs_last) H_prev  +  sum_j w_j x_j B_j^T,  w_j = exp(cs_last - cs_j) dt_j
//
// and every exponent is a difference cs_i - cs_j with j <= i (<= 0).
//
// One workgroup runs one segment of one sequence for one head with 4 waves
// (one per SIMD).  Wave w owns output rows i in [32w, 32w+32): its w+1 causal
// C B^T tiles, turned into the decay-masked M in registers and fed straight
// back as the MFMA operand of the intra-chunk product (the accumulator holds
// 4+4 rows per lane, used as a permuted K order that the other operand
// follows), its state->output tiles, and a share of the 8 state tiles dealt
// 4/3/1/0 so every wave runs 60-64 MFMAs per chunk.  All products are
// v_mfma_f32_32x32x16_bf16.
//
// Memory path, MI355X-specific:
//   * x and B arrive by global->LDS direct loads (global_load_lds_dwordx4)
//     into token-major tiles whose 16-byte blocks are XOR-swizzled per row;
//     no VGPR staging and no transposing copies.  Each tile is reloaded as
//     soon as its last reader is done: B (read only in the k-loop) by the
//     last wave out of the k-loop, x after barrier A.
//   * operands whose contraction runs over tokens (B^T and x^T) are read
//     straight from those token-major tiles with the LDS transpose read
//     ds_read_b64_tr_b16: in each 16-lane group, lane s points at row
//     k0 + s/4, columns c0 + 4(s%4)..+3, and lane i then holds rows
//     k0..k0+3 of column c0 + i -- four K values of its MFMA column.
//   * the running state stays on chip: fp32 in the owning waves' MFMA
//     accumulators, bf16 in LDS as the operand of the state->output product.
//   * C goes global -> registers (each wave its own 32 rows), one fragment of
//     the next chunk per k-step, right after the step that used the current
//     one.
//   * y is staged through an LDS tile of its own, so every store writes whole
//     128-byte rows while the next x tile is landing.
#include <type_traits>

#include "scan_items.h"

namespace ssd {

namespace {

constexpr int kThr = 256;  // 4 waves, one per SIMD

typedef short s16x4 __attribute__((ext_vector_type(4)));
// LDS pointers stay in address space 3 from the kernel entry on: no generic
// pointer (and no null check per access) between a tile and its ds_* / direct loads.
#define SSD_LDS __attribute__((address_space(3)))
typedef SSD_LDS s16x4 lds_s16x4;
typedef SSD_LDS void lds_void;
typedef SSD_LDS uint8_t lds_u8;
typedef SSD_LDS float lds_f32;
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <class T> __device__ __forceinline__ T lds_ld(const lds_u8 *p) { return *reinterpret_cast<const SSD_LDS T *>(p); }
template <class T> __device__ __forceinline__ void lds_st(lds_u8 *p, T v) { *reinterpret_cast<SSD_LDS T *>(p) = v; }

// Row swizzles of the 16-byte blocks: conflict-free for 8 (or 16) lanes on
// consecutive rows of one block, and for the transpose reads (4 consecutive
// rows x 2 adjacent blocks).
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }
__device__ __forceinline__ int swz8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
// byte offset of element (row, col) in a 256-byte-row tile (128 bf16) / 128-byte-row tile (64 bf16)
__device__ __forceinline__ int off256(int row, int col) {
  return row * 256 + ((((col >> 3) ^ swz16(row))) << 4) + ((col & 7) << 1);
}
__device__ __forceinline__ int off128(int row, int col) {
  return row * 128 + ((((col >> 3) ^ swz8(row))) << 4) + ((col & 7) << 1);
}

// Per-token arrays of one chunk (cs, dt, w, v), then exp(cs_last), cs_last and
// the counter of waves done with the chunk's B tile.
constexpr int kSmallBytes = 4 * kChunk * 4 + 16;
struct Smem {
  uint8_t B[kChunk * 256];    // B[j][n], token-major
  uint8_t X[kChunk * 128];    // x[j][p], token-major
  uint8_t H[kHeadDim * 256];  // running state H[p][n] in bf16
  // y[i][p] staging between barriers A and B, 128-byte rows like the x tile.
  // Its last kSmallBytes are the per-token arrays: they lie in rows that only
  // the dt wave stages, and it rewrites them after reading its y rows back.
  uint8_t Y[kChunk * 128];
};
constexpr int kSmallOff = kChunk * 128 - kSmallBytes;
// two workgroups per CU: each fits in half of the 160 KiB LDS
static_assert(sizeof(Smem) <= 80 * 1024, "LDS budget of one of two workgroups per CU");
static_assert(kSmallOff % 16 == 0, "per-token arrays 16-byte aligned");

struct Lds {
  lds_u8 *B, *X, *H, *Y;
  lds_f32 *cs, *dt, *w, *v, *misc;
};


// state tiles (n-block nb, p-block pb) of H^T owned by wave w in the full pass
// dealt by p-block, so each wave scales one x fragment per k-step
constexpr int kNS[4] = {4, 3, 1, 0};
constexpr int kSnb[4][4] = {{0, 1, 2, 3}, {0, 1, 2, 0}, {3, 0, 0, 0}, {0, 0, 0, 0}};
constexpr int kSpb[4][4] = {{0, 0, 0, 0}, {1, 1, 1, 0}, {1, 0, 0, 0}, {0, 0, 0, 0}};
constexpr int kDtWave = 3;  // the wave that computes the next chunk's dt / cumsum (no state tiles)
// the per-token arrays overlay staging rows of the dt wave only
static_assert(kSmallOff >= 32 * kDtWave * 128 && 32 * (kDtWave + 1) == kChunk, "arrays in the dt wave's y rows");

template <bool kFull, int W> struct Cfg {
  static constexpr int NCB = kFull ? W + 1 : 0;
  static constexpr int NS = kFull ? kNS[W] : 2;
  // state-only pass: wave w owns n-blocks 2(w%2), 2(w%2)+1 of p-block w/2
  __host__ __device__ static constexpr int nb(int t) { return kFull ? kSnb[W][t] : 2 * (W % 2) + t; }
  __host__ __device__ static constexpr int spb(int t) { return kFull ? kSpb[W][t] : W / 2; }
  __host__ __device__ static constexpr bool uses_spb(int q) {
    for (int t = 0; t < NS; ++t)
      if (spb(t) == q) return true;
    return false;
  }
  // distinct n-blocks of the state tiles: one B^T fragment each per k-step.
  // slots.s[t] = fragment slot of tile t, slots.nb[u] = n-block of slot u.
  struct Slots {
    int s[4], nb[4], n;
  };
  __host__ __device__ static constexpr Slots make_slots() {
    Slots r{{0, 0, 0, 0}, {0, 0, 0, 0}, 0};
    for (int t = 0; t < NS; ++t) {
      int u = 0;
      while (u < r.n && r.nb[u] != nb(t)) ++u;
      if (u == r.n) r.nb[r.n++] = nb(t);
      r.s[t] = u;
    }
    return r;
  }
  static constexpr Slots kSlots = make_slots();
  static constexpr int NNB = kSlots.n;
  __host__ __device__ static constexpr int slot(int t) { return kSlots.s[t]; }
  __host__ __device__ static constexpr int slot_nb(int u) { return kSlots.nb[u]; }
  // every tile's slot holds its own n-block, and slots are all distinct
  __host__ __device__ static constexpr bool slots_ok() {
    for (int t = 0; t < NS; ++t)
      if (slot(t) >= NNB || slot_nb(slot(t)) != nb(t)) return false;
    for (int u = 0; u < NNB; ++u)
      for (int v = 0; v < u; ++v)
        if (slot_nb(u) == slot_nb(v)) return false;
    return true;
  }
};
static_assert(Cfg<true, 0>::slots_ok() && Cfg<true, 0>::NNB == 4, "state tile slots");
static_assert(Cfg<true, 1>::slots_ok() && Cfg<true, 1>::NNB == 3, "state tile slots");
static_assert(Cfg<true, 2>::slots_ok() && Cfg<true, 2>::NNB == 1, "state tile slots");
static_assert(Cfg<true, 3>::slots_ok() && Cfg<true, 3>::NNB == 0, "state tile slots");
static_assert(Cfg<false, 0>::slots_ok() && Cfg<false, 0>::NNB == 2, "state tile slots");
static_assert(Cfg<false, 3>::slots_ok() && Cfg<false, 3>::NNB == 2, "state tile slots");

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 tr_read(const lds_u8 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  return __builtin_bit_cast(u32x2, v);
}

// w_j x_j for the 8 K values of a fragment (K rows k0..k0+7 in element order),
// rounded to bf16 as the MFMA operand.
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 x, f32x4 wa, f32x4 wb) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  u32x4 o;
  o[0] = pack2_bf16(lo_bf16(u[0]) * wa[0], hi_bf16(u[0]) * wa[1]);
  o[1] = pack2_bf16(lo_bf16(u[1]) * wa[2], hi_bf16(u[1]) * wa[3]);
  o[2] = pack2_bf16(lo_bf16(u[2]) * wb[0], hi_bf16(u[2]) * wb[1]);
  o[3] = pack2_bf16(lo_bf16(u[3]) * wb[2], hi_bf16(u[3]) * wb[3]);
  return __builtin_bit_cast(bf16x8, o);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS traffic).
__device__ __forceinline__ float wave_incl_scan(float x) {
#define SSD_DPP_ADD(ctrl, rmask, bc)                                                              \
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xF, bc))
  SSD_DPP_ADD(0x111, 0xF, true);   // row_shr:1
  SSD_DPP_ADD(0x112, 0xF, true);   // row_shr:2
  SSD_DPP_ADD(0x114, 0xF, true);   // row_shr:4
  SSD_DPP_ADD(0x118, 0xF, true);   // row_shr:8
  SSD_DPP_ADD(0x142, 0xA, false);  // row_bcast:15 -> rows 1, 3
  SSD_DPP_ADD(0x143, 0xC, false);  // row_bcast:31 -> rows 2, 3
#undef SSD_DPP_ADD
  return x;
}

// softplus(z) = log(1 + e^z) with log1p accuracy (u = 1 + e rounded; the
// factor e / (u - 1) corrects the rounding of u).
__device__ __forceinline__ float softplus_fast(float z) {
  if (z > 20.f) return z;
  const float e = __expf(z);
  const float u = 1.f + e;
  return u == 1.f ? e : __logf(u) * (e / (u - 1.f));
}

// dt, cs, w = exp(cs_last - cs) dt and v = exp(cs_r - cs) dt (r = end of the
// token's 32-block) of one chunk, by one wave (tokens 2 lane, 2 lane + 1),
// held in registers until store() puts them in LDS.
struct ChunkDt {
  f32x2 cs, dt, w, v;
  float dec, total;
  __device__ __forceinline__ void store(lds_f32 *cs_, lds_f32 *dt_, lds_f32 *w_, lds_f32 *v_, lds_f32 *misc) const {
    const int j0 = 2 * (threadIdx.x & 63);
    *reinterpret_cast<SSD_LDS f32x2 *>(cs_ + j0) = cs;
    *reinterpret_cast<SSD_LDS f32x2 *>(dt_ + j0) = dt;
    *reinterpret_cast<SSD_LDS f32x2 *>(w_ + j0) = w;
    *reinterpret_cast<SSD_LDS f32x2 *>(v_ + j0) = v;
    if ((threadIdx.x & 63) == 0) {
      misc[0] = dec;
      misc[1] = total;
      misc[2] = 0.f;  // the B-load counter of the chunk (all bits zero)
    }
  }
};
__device__ __forceinline__ ChunkDt chunk_dt_wave(uint32_t raw, int nv, float bias, float A) {
  const int lane = threadIdx.x & 63;
  const int j0 = 2 * lane;
  const float d0 = j0 < nv ? softplus_fast(lo_bf16(raw) + bias) : 0.f;
  const float d1 = j0 + 1 < nv ? softplus_fast(hi_bf16(raw) + bias) : 0.f;
  const float a1 = d1 * A;
  const float incl = wave_incl_scan(d0 * A + a1);
  const float cs1 = incl, cs0 = incl - a1;
  const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
  // cs at the last token of this lane's 32-token block: lanes 15, 31, 47, 63
  const float e0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 15));
  const float e1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 31));
  const float e2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 47));
  const int blk = lane >> 4;
  const float cr = blk == 0 ? e0 : blk == 1 ? e1 : blk == 2 ? e2 : total;
  ChunkDt r;
  r.cs = f32x2{cs0, cs1};
  r.dt = f32x2{d0, d1};
  r.w = f32x2{__expf(total - cs0) * d0, __expf(total - cs1) * d1};
  r.v = f32x2{__expf(cr - cs0) * d0, __expf(cr - cs1) * d1};
  r.dec = __expf(total);
  r.total = total;
  return r;
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses are
// complete, its global loads (and direct loads to LDS) may still be in
// flight.  The empty asm keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Lane id through an empty asm: values derived from it are recomputed in
// every chunk instead of being hoisted out of the chunk loop, where dozens of
// loop-invariant addresses and masks would hold registers for the whole kernel.
__device__ __forceinline__ int opaque_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}
// A value the compiler cannot see through: x XOR (an opaque zero).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Where one lane sits in the MFMA layouts, and the per-lane LDS byte offsets
// of its operands at k-step 0.  The swizzles only look at the low 4 (B tile) /
// 3 (x tile) bits of a row, so the transpose read k-step s later, 16 rows
// further, is + 4096 s in B and + 2048 s in x (an immediate offset), and the
// row-major 16-byte read of column block 2s + hh is the step-0 offset XOR 32 s.
template <int NCB> struct LaneGeo {
  int lane, l32, hh, g16, s16;
  uint32_t oBt[4][2], oXt[2][2], oBr[NCB > 0 ? NCB : 1], oH[2], oYd[2];
  template <class Cf> __device__ __forceinline__ void init(int ln) {
    lane = ln;
    l32 = ln & 31;
    hh = ln >> 5;
    g16 = ln >> 4;
    s16 = ln & 15;
    const int trr = 8 * hh + (s16 >> 2);            // transpose-read row at step 0
    const int trc = 16 * (g16 & 1) + 4 * (s16 & 3);  // ... and column within a 32-block
#pragma unroll
    for (int u = 0; u < Cf::NNB; ++u) {
      oBt[u][0] = off256(trr, 32 * Cf::slot_nb(u) + trc);
      oBt[u][1] = off256(trr + 4, 32 * Cf::slot_nb(u) + trc);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      oXt[u][0] = off128(trr, 32 * u + trc);
      oXt[u][1] = off128(trr + 4, 32 * u + trc);
      oH[u] = off256(32 * u + l32, 8 * hh);
      // x^T reads of the intra-chunk product: rows 32 jb + 16 s2 + 4 hh + s16/4 (+8)
      oYd[u] = off128(4 * hh + (s16 >> 2), 32 * u + trc);
    }
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) oBr[jb] = off256(32 * jb + l32, 8 * hh);
  }
};

__device__ __forceinline__ bf16x8 trd(const lds_u8 *tile, uint32_t lo, uint32_t hi) {
  const u32x2 a = tr_read(tile + lo);
  const u32x2 b = tr_read(tile + hi);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

template <bool kFull, bool kConv, int W>
__device__ __forceinline__ void run_wave(const ScanParams &p, const ScanPlan &plan, char *ws, const Item &it,
                                         int item, int h, int g, const Lds &sm) {
  using Cf = Cfg<kFull, W>;
  constexpr int NCB = Cf::NCB, NS = Cf::NS;
  constexpr int NX = (Cf::uses_spb(0) ? 1 : 0) + (Cf::uses_spb(1) ? 1 : 0);
  constexpr int NNB = Cf::NNB;
  constexpr int NF = NX + NNB + (kFull ? NCB + 2 : 0);

  const bf16_t *xg = reinterpret_cast<const bf16_t *>(p.x) + it.boff * p.x_sb + h * kHeadDim;
  const bf16_t *Bg = reinterpret_cast<const bf16_t *>(p.B) + it.boff * p.B_sb + g * kDState;
  const bf16_t *Cg = reinterpret_cast<const bf16_t *>(p.C) + it.boff * p.C_sb + g * kDState;
  const bf16_t *dtg = reinterpret_cast<const bf16_t *>(p.dt) + it.boff * p.dt_sb + h;
  bf16_t *yg = reinterpret_cast<bf16_t *>(p.y) + it.boff * p.y_sb + h * kHeadDim;
  const uint32_t xst = (uint32_t)p.x_st, bst = (uint32_t)p.B_st, cst = (uint32_t)p.C_st;
  const uint32_t dst = (uint32_t)p.dt_st, yst = (uint32_t)p.y_st;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;
  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;

  // B rows [r0, r0 + 4 N) / this wave's x rows of one chunk -> LDS by direct
  // loads, 4 B rows (8 x rows) per instruction.  Rows past the segment end
  // repeat its last row (finite values whose every use is cancelled: dt = 0
  // there).  A whole chunk takes one per-lane 32-bit byte offset per tile,
  // the row step in the (uniform) base address.
  auto issue_b = [&](int ln, int c0, int nv, int r0, auto n_instr) {
    constexpr int N = decltype(n_instr)::value;
    if (nv == kChunk) {
      const char *bc = reinterpret_cast<const char *>(Bg + (int64_t)c0 * p.B_st);
      const uint32_t ob = (r0 + (ln >> 4)) * bst * 2;
      uint32_t cb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cb[i] = ob + 16 * ((ln & 15) ^ swz16(r0 + (ln >> 4) + 4 * i));
#pragma unroll
      for (int i = 0; i < N; ++i)
        __builtin_amdgcn_global_load_lds(bc + (size_t)(8 * i) * bst + cb[i & 3],
                                         (lds_void *)(sm.B + (r0 + 4 * i) * 256), 16, 0, 0);
      return;
    }
    const int last = nv - 1;
    const bf16_t *bc = Bg + (int64_t)c0 * p.B_st;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + 4 * i + (ln >> 4);
      const int blk = (ln & 15) ^ swz16(r);
      __builtin_amdgcn_global_load_lds(bc + (uint32_t)min(r, last) * bst + 8 * blk,
                                       (lds_void *)(sm.B + (r0 + 4 * i) * 256), 16, 0, 0);
    }
  };
  auto issue_x = [&](int ln, int c0, int nv) {
    if (nv == kChunk) {
      const char *xc = reinterpret_cast<const char *>(xg + (int64_t)c0 * p.x_st);
      const uint32_t ox = (32 * W + (ln >> 3)) * xst * 2 + 16 * ((ln & 7) ^ swz8(ln >> 3));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(xc + (size_t)(16 * i) * xst + ox,
                                         (lds_void *)(sm.X + (32 * W + 8 * i) * 128), 16, 0, 0);
      return;
    }
    const int last = nv - 1;
    const bf16_t *xc = xg + (int64_t)c0 * p.x_st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * W + 8 * i + (ln >> 3);
      const int blk = (ln & 7) ^ swz8(r);
      __builtin_amdgcn_global_load_lds(xc + (uint32_t)min(r, last) * xst + 8 * blk,
                                       (lds_void *)(sm.X + (32 * W + 8 * i) * 128), 16, 0, 0);
    }
  };
  // kConv: the x tile is conv1d(4) + SiLU of the raw conv input.  The raw
  // rows land in the tile by the same direct loads as post-conv rows would
  // (issue_x); once a wave's own loads have landed it convolves its 32 rows
  // in place, with the conv kernel's arithmetic (fp32 taps in the same order,
  // the same SiLU, bf16 round to nearest even), so the tile ends up holding
  // exactly what a separate conv pass would have written.  Lane roles:
  // channels 2 cp, 2 cp + 1 (cp = lane % 32) of rows 16 rg .. 16 rg + 15 (rg =
  // lane / 32) of the wave's rows.  All of a wave's LDS reads precede its
  // writes, so in place is safe within the wave; the 3 rows before the wave's
  // first (another wave's, or before the chunk) come from global memory into
  // registers: the input, or before the sequence the conv state (or zero).
  // Rows past the segment end repeat its last token, as the direct loads do.
  uint32_t halo[kConv ? kConvWidth - 1 : 1];
  auto conv_halo_load = [&](int ln, int c0, int nv) {
    const int cp = ln & 31;
    const int first = it.seq0 - c0;  // chunk row of the sequence's first token (<= 0)
    const char *xc = reinterpret_cast<const char *>(xg + (int64_t)c0 * p.x_st) + 4 * cp;
    // one row past the sequence's conv state rows: row first - d sits d rows before it
    const char *st = p.conv_state
                         ? reinterpret_cast<const char *>(p.conv_state) +
                               (((int64_t)it.row * (kConvWidth - 1) + (kConvWidth - 1)) * p.conv_ch +
                                h * kHeadDim + 2 * cp) * 2
                         : nullptr;
#pragma unroll
    for (int k = 0; k < kConvWidth - 1; ++k) {
      const int r = min(32 * W - (kConvWidth - 1) + k, nv - 1);  // chunk row (negative: before the chunk)
      const bool before = r < first;
      const char *src = (before && st) ? st - (int64_t)(first - r) * p.conv_ch * 2
                                       : xc + max(r, first) * (int)xst * 2;
      const uint32_t v = *reinterpret_cast<const uint32_t *>(src);
      halo[k] = (before && !st) ? 0u : v;
    }
  };
  // the two channels' taps and biases: loaded ahead of the wait for the
  // tile, so the conv does not wait for them
  float cwt[kConv ? 2 : 1][4], cbias[kConv ? 2 : 1];
  auto conv_taps_load = [&](int ln) {
    const int ch = h * kHeadDim + 2 * (ln & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float4 wv = *reinterpret_cast<const float4 *>(p.conv_w + (int64_t)(ch + i) * kConvWidth);
      cwt[i][0] = wv.x; cwt[i][1] = wv.y; cwt[i][2] = wv.z; cwt[i][3] = wv.w;
      cbias[i] = p.conv_b ? p.conv_b[ch + i] : 0.f;
    }
  };
  // rows r0 + j0 .. r0 + j0 + 7 of this lane's group from raw[0..10] = rows
  // r0 + j0 - 3 .. r0 + j0 + 7
  auto conv_rows8 = [&](int ln, int j0, const uint32_t *raw) {
    const int cp = ln & 31, r0 = 32 * W + 16 * (ln >> 5);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float u[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        auto v = [&](int k) { return i ? hi_bf16(raw[k]) : lo_bf16(raw[k]); };
        float a = cbias[i];
        a = fmaf(cwt[i][0], v(j), a);
        a = fmaf(cwt[i][1], v(j + 1), a);
        a = fmaf(cwt[i][2], v(j + 2), a);
        a = fmaf(cwt[i][3], v(j + 3), a);
        u[i] = silu_f32(a);
      }
      lds_st<uint32_t>(sm.X + off128(r0 + j0 + j, 2 * cp), pack2_bf16(u[0], u[1]));
    }
  };
  // In two halves, each reading all it needs before writing: the group's
  // rows 8..15 first (reads rows 5..15), then rows 0..7 (reads rows 0..7,
  // untouched so far, and the 3 rows before the group, taken at the start:
  // group 1's are group 0's rows 13..15, which the first half overwrites).
  auto conv_in_place = [&](int ln) {
    const int cp = ln & 31, rg = ln >> 5;
    const int r0 = 32 * W + 16 * rg;
    uint32_t pre[kConvWidth - 1];
#pragma unroll
    for (int k = 0; k < kConvWidth - 1; ++k) {
      const uint32_t l = lds_ld<uint32_t>(sm.X + off128(max(r0 - (kConvWidth - 1) + k, 32 * W), 2 * cp));
      pre[k] = rg ? l : halo[k];
    }
    uint32_t raw[8 + kConvWidth - 1];
#pragma unroll
    for (int k = 0; k < 8 + kConvWidth - 1; ++k) raw[k] = lds_ld<uint32_t>(sm.X + off128(r0 + 5 + k, 2 * cp));
    conv_rows8(ln, 8, raw);
#pragma unroll
    for (int k = 0; k < kConvWidth - 1; ++k) raw[k] = pre[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) raw[kConvWidth - 1 + k] = lds_ld<uint32_t>(sm.X + off128(r0 + k, 2 * cp));
    conv_rows8(ln, 0, raw);
  };
  auto issue_tiles = [&](int ln, int c0, int nv) {
    issue_b(ln, c0, nv, 32 * W, std::integral_constant<int, 8>{});
    issue_x(ln, c0, nv);
    if (kConv) conv_halo_load(ln, c0, nv);
  };
  // C rows i of this wave's i-block: this lane's 8 k-steps of the MFMA operand
  u32x4 cf[8];
  // (uniform 64-bit base + per-lane 32-bit byte offset: scalar-base addressing)
  auto load_c = [&](int ln, int c0, int nv) {
    const int ci = 32 * W + (ln & 31);
    const char *cc = reinterpret_cast<const char *>(Cg + (int64_t)c0 * p.C_st);
    const uint32_t o = (uint32_t)min(ci, nv - 1) * cst * 2 + 16 * (ln >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) cf[s] = *reinterpret_cast<const u32x4 *>(cc + o + 32 * s);
  };
  // raw dt of tokens 2 lane, 2 lane + 1 (two bf16, packed by the caller)
  auto load_dt_raw = [&](int ln, int c0, int nv, uint32_t &lo, uint32_t &hi) {
    const char *dc = reinterpret_cast<const char *>(dtg + (int64_t)c0 * p.dt_st);
    lo = *reinterpret_cast<const bf16_t *>(dc + (uint32_t)min(2 * ln, nv - 1) * dst * 2);
    hi = *reinterpret_cast<const bf16_t *>(dc + (uint32_t)min(2 * ln + 1, nv - 1) * dst * 2);
  };

  // state tiles H^T (rows n = 32 nb + 8q + 4hh + 0..3, col p = 32 pb + l32)
  f32x16 hs[NS > 0 ? NS : 1];
  auto write_state_lds = [&](int ln) {
    const int l32 = ln & 31, hh = ln >> 5;
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 v;
        v[0] = pack2_bf16(hs[t][4 * q], hs[t][4 * q + 1]);
        v[1] = pack2_bf16(hs[t][4 * q + 2], hs[t][4 * q + 3]);
        lds_st<u32x2>(sm.H + off256(32 * Cf::spb(t) + l32, 32 * Cf::nb(t) + 8 * q + 4 * hh), v);
      }
  };
  {
    const int ln = threadIdx.x & 63, l32 = ln & 31, hh = ln >> 5;
    const float *entry = nullptr;
    if (kFull) {
      if (it.first) entry = p.init ? p.init + ((int64_t)it.row * p.H + h) * kPN : nullptr;
      else entry = ws_f32(plan, ws, plan.ws_entry_off) + ((int64_t)item * p.H + h) * kPN;
    }
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 e = make_float4(0.f, 0.f, 0.f, 0.f);
        if (entry)
          e = *reinterpret_cast<const float4 *>(entry + (32 * Cf::spb(t) + l32) * kDState + 32 * Cf::nb(t) + 8 * q +
                                                4 * hh);
        hs[t][4 * q + 0] = e.x; hs[t][4 * q + 1] = e.y;
        hs[t][4 * q + 2] = e.z; hs[t][4 * q + 3] = e.w;
      }
  }

  float logdecay = 0.f;
  const int ntok = it.tok1 - it.tok0;
  if (ntok > 0) {
    const int ln = threadIdx.x & 63;
    const int nv0 = min(kChunk, ntok);
    if (kFull) load_c(ln, it.tok0, nv0);
    if (W == kDtWave) {
      uint32_t lo, hi;
      load_dt_raw(ln, it.tok0, nv0, lo, hi);
      chunk_dt_wave(lo | (hi << 16), nv0, bias, Ah).store(sm.cs, sm.dt, sm.w, sm.v, sm.misc);
    }
    if (kFull) write_state_lds(ln);
    issue_tiles(ln, it.tok0, nv0);  // last, for the same reason as in the loop
    if (kConv) conv_taps_load(ln);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
    if (kConv) conv_in_place(ln);
    __syncthreads();
  }

  // Per chunk: k-loop (the last wave out of it loads the next B tile at the
  // end of its intra-chunk phase), intra-chunk product, barrier A (LDS only),
  // then the next x tile's loads, this chunk's state into H, y through the
  // staging tile, the next chunk's dt, and barrier B once every direct load
  // has landed.  The other workgroup on the CU runs while this one waits.
  // operand offsets once per segment (a few registers); the rest of the lane
  // geometry is re-derived in every chunk from an opaque lane id
  LaneGeo<NCB> LG;
  LG.template init<Cf>(threadIdx.x & 63);
  f32x16 yo[2];
  for (int c0 = it.tok0; c0 < it.tok1; c0 += kChunk) {
    struct {
      int lane, l32, hh;
    } L;
    L.lane = opaque_lane();
    L.l32 = L.lane & 31;
    L.hh = L.lane >> 5;
    // row-major operand bases, made opaque per chunk so that their eight
    // XOR-stepped addresses are formed in the k-loop, not hoisted
    uint32_t oBr[NCB > 0 ? NCB : 1], oH[2];
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) oBr[jb] = opaque(LG.oBr[jb]);
    oH[0] = opaque(LG.oH[0]);
    oH[1] = opaque(LG.oH[1]);
    const int ci = 32 * W + L.l32;  // this lane's chunk row i (full pass)
    const int nv = min(kChunk, it.tok1 - c0);
    const int c1 = c0 + kChunk;
    const bool has_next = c1 < it.tok1;
    const int cn = has_next ? c1 : c0;
    const int nvn = has_next ? min(kChunk, it.tok1 - c1) : nv;
    // the next chunk's raw dt: loaded now, packed (and so waited for) only
    // after the k-loop
    uint32_t raw_lo = 0, raw_hi = 0;
    if (W == kDtWave) load_dt_raw(L.lane, cn, nvn, raw_lo, raw_hi);

    const float dec = sm.misc[0];
    logdecay += sm.misc[1];
    const float cs_i = kFull ? sm.cs[ci] : 0.f;  // read now, used after the k-loop
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) hs[t][r] *= dec;

    f32x16 G[NCB > 0 ? NCB : 1];
#pragma unroll
    for (int t = 0; t < NCB; ++t) G[t] = f32x16{};
    yo[0] = f32x16{}; yo[1] = f32x16{};

    // k-loop: every accumulator chain of this wave, operands double-buffered
    auto load_frags = [&](int s, bf16x8 *f, f32x4 *wv) {
      int k = 0;
      if (NX > 0) {
        wv[0] = lds_ld<f32x4>((const lds_u8 *)&sm.w[16 * s + 8 * L.hh]);
        wv[1] = lds_ld<f32x4>((const lds_u8 *)&sm.w[16 * s + 8 * L.hh + 4]);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (Cf::uses_spb(q)) f[k++] = trd(sm.X, LG.oXt[q][0] + 2048 * s, LG.oXt[q][1] + 2048 * s);
#pragma unroll
      for (int u = 0; u < NNB; ++u) f[k++] = trd(sm.B, LG.oBt[u][0] + 4096 * s, LG.oBt[u][1] + 4096 * s);
      if (kFull) {
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb) f[k++] = lds_ld<bf16x8>(sm.B + (oBr[jb] ^ (32 * s)));
#pragma unroll
        for (int q = 0; q < 2; ++q) f[k++] = lds_ld<bf16x8>(sm.H + (oH[q] ^ (32 * s)));
      }
    };
    auto mfma_step = [&](int s, const bf16x8 *f, const f32x4 *wv) {
      int k = 0;
      bf16x8 xw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (Cf::uses_spb(q)) xw[q] = scale_frag(f[k++], wv[0], wv[1]);
#pragma unroll
      for (int t = 0; t < NS; ++t) hs[t] = mfma32(f[k + Cf::slot(t)], xw[Cf::spb(t)], hs[t]);
      k += NNB;
      if (kFull) {
        const bf16x8 cb = __builtin_bit_cast(bf16x8, cf[s]);
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb) G[jb] = mfma32(f[k++], cb, G[jb]);
#pragma unroll
        for (int q = 0; q < 2; ++q) yo[q] = mfma32(f[k++], cb, yo[q]);
      }
    };
    // The next chunk's C fragments are loaded one per k-step, into the one the
    // step has just used.  A fragment load touches 32 cache lines (one per
    // row); eight of them from each wave in one burst after the k-loop would
    // hold up the direct loads queued behind them.
    const char *ccn = reinterpret_cast<const char *>(Cg + (int64_t)cn * p.C_st);
    const uint32_t ocn = (uint32_t)min(ci, nvn - 1) * cst * 2 + 16 * L.hh;
    {
      bf16x8 fr[2][NF > 0 ? NF : 1];
      f32x4 wr[2][2];
      load_frags(0, fr[0], wr[0]);
      // the k-loop's MFMA stream goes first when the other workgroup's wave on
      // this SIMD also has work to issue
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < 7) load_frags(s + 1, fr[(s + 1) & 1], wr[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(s, fr[s & 1], wr[s & 1]);
        if (kFull) cf[s] = *reinterpret_cast<const u32x4 *>(ccn + ocn + 32 * s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // raw_next (loaded at the top of the chunk) is waited for here, before any
    // later load: a wait for it behind those would be a wait for all of them
    uint32_t raw_next = 0;
    if (W == kDtWave) {
      asm volatile("" : "+v"(raw_lo), "+v"(raw_hi));
      raw_next = raw_lo | (raw_hi << 16);
    }
    // B is only read in the k-loop.  The last wave to finish it loads the
    // whole next B tile at the end of its intra-chunk phase (after its last
    // LDS read: a read behind a direct load waits for it), ahead of barrier
    // A, so that only the x tile is left to load after the barrier.  (The
    // counter is zeroed with the per-token arrays of every chunk.)
    // (the count is only looked at after the intra-chunk phase)
    uint32_t done = 0;
    if (has_next && L.lane == 0)
      done = __hip_atomic_fetch_add(reinterpret_cast<SSD_LDS uint32_t *>(sm.misc + 2), 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP);

    if (kFull) {
      // y = exp(cs_i) (C H_prev^T) + M x: scale the state->output part, then the
      // intra-chunk product accumulates on top of it
      const float ecs = __expf(cs_i);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) yo[q][r] *= ecs;
      // decay mask and dt -> bf16 M operand (rows j, col i) in registers,
      // then y^T[p][i] += sum_j x[j][p] M[j][i]
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb) {
        // x^T (row p, k = j) in the accumulator's permuted K order: slots 0..3
        // are rows 16s + 4hh + 0..3, slots 4..7 rows 16s + 8 + 4hh + 0..3.
        // Read first, so that building this tile's mask hides the LDS latency.
        bf16x8 xf[2][2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t o = LG.oYd[q] + 128 * (32 * jb + 16 * s2);
            xf[s2][q] = trd(sm.X, o, o + 1024);
          }
        // ... and so are the per-token factors of the mask: v_j and cs at the
        // block end off the diagonal, cs_j and dt_j on it
        f32x4 fa[4], fb[4];
        float cs_r = 0.f;
        if (jb < W) {
          cs_r = sm.cs[32 * jb + 31];
#pragma unroll
          for (int q = 0; q < 4; ++q) fa[q] = lds_ld<f32x4>((const lds_u8 *)&sm.v[32 * jb + 8 * q + 4 * L.hh]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int jq = 32 * jb + 8 * q + 4 * L.hh;
            fa[q] = lds_ld<f32x4>((const lds_u8 *)&sm.cs[jq]);
            fb[q] = lds_ld<f32x4>((const lds_u8 *)&sm.dt[jq]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 Mb[2];
        if (jb < W) {
          // all j < i: exp(cs_i - cs_j) = exp(cs_i - cs_r) exp(cs_r - cs_j) with r
          // the last row of block jb; both exponents are <= 0
          const float u = __expf(cs_i - cs_r);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 vj = fa[q];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int r = 4 * q + t;
              Mb[r >> 3][r & 7] = (__bf16)(G[jb][r] * (u * vj[t]));
            }
          }
        } else {
          // diagonal block: d = i - j decides between decay, diagonal and zero
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int jq = 32 * jb + 8 * q + 4 * L.hh;
            const f32x4 cj = fa[q], dj = fb[q];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int r = 4 * q + t;
              const int d = ci - (jq + t);
              // exp(-inf) = 0 above the diagonal
              const float e = __expf(d >= 0 ? cs_i - cj[t] : -INFINITY);
              Mb[r >> 3][r & 7] = (__bf16)(G[jb][r] * e * dj[t]);
            }
          }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int q = 0; q < 2; ++q) yo[q] = mfma32(xf[s2][q], Mb[s2], yo[q]);
      }
      // the skip term D x_i in fp32 (x rows are still this chunk's until
      // barrier A): the lane holds p = 32 q + 8 r4 + 4 hh + 0..3 of row ci
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2 xv = lds_ld<u32x2>(sm.X + off128(ci, 32 * q + 8 * r4 + 4 * L.hh));
          yo[q][4 * r4 + 0] = fmaf(Dh, lo_bf16(xv[0]), yo[q][4 * r4 + 0]);
          yo[q][4 * r4 + 1] = fmaf(Dh, hi_bf16(xv[0]), yo[q][4 * r4 + 1]);
          yo[q][4 * r4 + 2] = fmaf(Dh, lo_bf16(xv[1]), yo[q][4 * r4 + 2]);
          yo[q][4 * r4 + 3] = fmaf(Dh, hi_bf16(xv[1]), yo[q][4 * r4 + 3]);
        }
    }
    if (has_next && __builtin_amdgcn_readfirstlane(done) == 3)
      issue_b(L.lane, c1, nvn, 0, std::integral_constant<int, 32>{});
    // A: every read of this chunk's tiles, H and cs/dt/w/v is done.  LDS only:
    // the next B tile may still be landing (nothing reads it before barrier B).
    lds_barrier();
    // the next chunk's direct loads go first, so that they land while this
    // wave writes H and stages y: LDS writes do not wait for them, the first
    // LDS read behind them (the y read-back) does
    if (has_next) issue_x(L.lane, c1, nvn);
    __builtin_amdgcn_sched_barrier(0);  // keep them first
    if (kFull) {
      write_state_lds(L.lane);  // H_c for the next chunk's state->output product
      // y rows through the staging tile, so each store writes 8 whole
      // 128-byte rows.  The lane holds p = 32q + 8 r4 + 4 hh + 0..3 of chunk row ci.
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          u32x2 v;
          v[0] = pack2_bf16(yo[q][4 * r4], yo[q][4 * r4 + 1]);
          v[1] = pack2_bf16(yo[q][4 * r4 + 2], yo[q][4 * r4 + 3]);
          lds_st<u32x2>(sm.Y + off128(ci, 32 * q + 8 * r4 + 4 * L.hh), v);
        }
    }
    ChunkDt nd;
    if (W == kDtWave && has_next) nd = chunk_dt_wave(raw_next, nvn, bias, Ah);
    if (kFull) {
      const int rr = 32 * W + (L.lane >> 3);  // + 8k: rows this lane stores
      char *yc = reinterpret_cast<char *>(yg + (int64_t)c0 * p.y_st);
      const uint32_t yo0 = (uint32_t)rr * yst * 2 + 16 * (L.lane & 7), ystep = 8 * yst * 2;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 v = lds_ld<u32x4>(sm.Y + off128(rr + 8 * k, 8 * (L.lane & 7)));
        if (rr + 8 * k < nv) *reinterpret_cast<u32x4 *>(yc + yo0 + k * ystep) = v;
      }
    }
    // kConv: the next tile's halo rows and the taps, issued once y is out of
    // the registers; the wait below is for the y stores too, which covers them
    if (kConv && has_next) {
      conv_halo_load(L.lane, c1, nvn);
      conv_taps_load(L.lane);
    }
    // after this wave's y read-back: the arrays overlay its staging rows
    if (W == kDtWave && has_next) nd.store(sm.cs, sm.dt, sm.w, sm.v, sm.misc);
    __builtin_amdgcn_s_waitcnt(0);       // this wave's direct loads of the next chunk have landed
    if (kConv && has_next) conv_in_place(L.lane);  // (this chunk's reads of the tile ended at barrier A)
    __syncthreads();                     // B: ... and every wave's
  }

  // outputs of the segment
  const int l32 = threadIdx.x & 31, hh = (threadIdx.x >> 5) & 1;
  float *out = nullptr;
  if (kFull) {
    if (it.last && p.final_state) out = p.final_state + ((int64_t)it.row * p.H + h) * kPN;
  } else {
    out = ws_f32(plan, ws, plan.ws_local_off) + ((int64_t)item * p.H + h) * kPN;
    if (threadIdx.x == 0) ws_f32(plan, ws, plan.ws_decay_off)[(int64_t)item * p.H + h] = logdecay;
  }
  if (out) {
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(out + (32 * Cf::spb(t) + l32) * kDState + 32 * Cf::nb(t) + 8 * q + 4 * hh) =
            make_float4(hs[t][4 * q], hs[t][4 * q + 1], hs[t][4 * q + 2], hs[t][4 * q + 3]);
  }
}

template <bool kFull, bool kConv>
__global__ __launch_bounds__(kThr, 2) void chunk_scan_bf16_kernel(ScanParams p, ScanPlan plan, char *ws) {
  __shared__ __attribute__((aligned(16))) Smem smem;
  lds_f32 *small = (lds_f32 *)((lds_u8 *)smem.Y + kSmallOff);
  const Lds sm{(lds_u8 *)smem.B, (lds_u8 *)smem.X, (lds_u8 *)smem.H, (lds_u8 *)smem.Y,
               small, small + kChunk, small + 2 * kChunk, small + 3 * kChunk, small + 4 * kChunk};
  int item, h, g;
  if (!map_workgroup(p, plan, ws, item, h, g)) return;
  Item it;
  if (!get_item(p, plan, ws, item, it)) return;
  if (!kFull && it.last) return;  // the pre-pass only needs segments that have a successor
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: run_wave<kFull, kConv, 0>(p, plan, ws, it, item, h, g, sm); break;
    case 1: run_wave<kFull, kConv, 1>(p, plan, ws, it, item, h, g, sm); break;
    case 2: run_wave<kFull, kConv, 2>(p, plan, ws, it, item, h, g, sm); break;
    default: run_wave<kFull, kConv, 3>(p, plan, ws, it, item, h, g, sm); break;
  }
}

}  // namespace

hipError_t launch_chunk_scan_bf16(const ScanParams &p, const ScanPlan &plan, char *ws, unsigned nblk, bool full,
                                  hipStream_t stream) {
  if (p.xconv) {
    if (full) hipLaunchKernelGGL((chunk_scan_bf16_kernel<true, true>), dim3(nblk), dim3(kThr), 0, stream, p, plan, ws);
    else hipLaunchKernelGGL((chunk_scan_bf16_kernel<false, true>), dim3(nblk), dim3(kThr), 0, stream, p, plan, ws);
  } else {
    if (full) hipLaunchKernelGGL((chunk_scan_bf16_kernel<true, false>), dim3(nblk), dim3(kThr), 0, stream, p, plan, ws);
    else hipLaunchKernelGGL((chunk_scan_bf16_kernel<false, false>), dim3(nblk), dim3(kThr), 0, stream, p, plan, ws);
  }
  return hipGetLastError();
}

}  // namespace ssd
