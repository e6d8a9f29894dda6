// The mixer's projections on gfx950: y (M, N) = x (M, K) . w (N, K)^T, bf16
// operands, fp32 accumulation, bf16 result.
//
// in_proj takes each token's d_model features to x|B|C, z and dt, and
// out_proj takes the gated, normalised y back to d_model ("Nemotron-H style
// Hybrid Mamba-Transformer 3B feasibility study", the projection parameters
// of the Mamba-2 block; "Nemotron-Mamba3 architecture" article, sec. 2.2).
// The weight is stored like a torch Linear weight, (out, in): both operands
// are K-contiguous, which is exactly the operand layout of the bf16 matrix
// cores, so no operand is transposed anywhere.
//
// A workgroup computes a BM x BN tile of y over K in 64-wide steps; its
// waves form a kWM x kWN grid, each wave owning (32 kTM) x (32 kTN) of the
// tile as tiles of v_mfma_f32_32x32x16_bf16.  Large products take 256 x 256
// tiles (8 waves of 128 x 64, one workgroup per CU): per flop that is half the
// operand traffic through L2 of 128 x 128 tiles, which small products keep
// (4 waves of 64 x 64, two workgroups per CU).
//  * x and w tiles arrive by global->LDS direct loads (16 bytes per lane, no
//    register staging), double-buffered: the next K step lands while the
//    current one is multiplied.  The 16-byte blocks of a 128-byte row are
//    XOR-swizzled by (row / 2) % 8, so the 16 lanes of one ds_read_b128
//    phase (16 consecutive rows, one block column) hit all 64 banks once.
//  * The product is taken as y^T per tile (w rows as the first operand), so
//    each lane's accumulator holds 4 consecutive output columns of one row:
//    8-byte LDS writes into a padded staging tile (one row of waves at a
//    time), then whole 16-byte row pieces go out to HBM.
//  * Tiles are dealt to the XCDs in contiguous ranges, grouped 16 tile rows
//    deep, so the workgroups sharing an x row block or a w column block run
//    on one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kBK = 64;
constexpr int kGroupM = 16;

#define SSD_LDS __attribute__((address_space(3)))
typedef SSD_LDS void lds_void;
typedef SSD_LDS uint8_t lds_u8;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// byte offset of 16-byte block `blk` of row `row` in a 128-byte-row tile
__device__ __forceinline__ uint32_t blk_off(int row, int blk) { return row * 128 + ((blk ^ swz(row)) << 4); }

// one 16-byte global -> LDS direct load per lane (LDS address: wave-uniform base + 16 lane)
__device__ __forceinline__ void load_lds16(const char *src, lds_u8 *dst_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)dst_base, 16, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int kWM, int kWN, int kTM, int kTN> struct LinCfg {
  static constexpr int kThr = 64 * kWM * kWN;
  static constexpr int BM = 32 * kTM * kWM, BN = 32 * kTN * kWN;
  static constexpr int kStageRowB = BN * 2 + 16;  // staging row: BN bf16 + 16 bytes of padding
  // two K steps of both tiles; the staging rows of one row of waves overlay them
  static constexpr int kLds = 2 * (BM + BN) * kBK * 2;
  static_assert(32 * kTM * kStageRowB <= kLds, "staging rows fit in the operand tiles");
  static_assert(BM % (8 * kWM * kWN) == 0 && BN % (8 * kWM * kWN) == 0, "8-row direct-load groups per wave");
};

template <int kWM, int kWN, int kTM, int kTN>
__global__ __launch_bounds__(64 * kWM * kWN) void linear_bf16_kernel(LinearParams p, int ntm, int ntn) {
  using Cf = LinCfg<kWM, kWN, kTM, kTN>;
  constexpr int BM = Cf::BM, BN = Cf::BN, kThr = Cf::kThr;
  constexpr int kLX = BM / 8 / (kWM * kWN), kLW = BN / 8 / (kWM * kWN);  // direct loads per wave and K step
  // LDS: x tiles of K steps 0 and 1 (BM rows of 128 bytes), then the w tiles
  extern __shared__ __attribute__((aligned(16))) uint8_t lin_smem[];
  constexpr uint32_t kXOff = 0, kWOff = 2 * BM * 128;
  // tile of this workgroup: XCD x gets tiles [x per, (x + 1) per), in order
  const int T = ntm * ntn;
  const int per = (T + kNumXCD - 1) / kNumXCD;
  const int t = (blockIdx.x % kNumXCD) * per + blockIdx.x / kNumXCD;
  if (t >= T) return;
  const int gsz = kGroupM * ntn;
  const int first_m = (t / gsz) * kGroupM;
  const int rows_in_group = min(ntm - first_m, kGroupM);
  const int tm = first_m + (t % gsz) % rows_in_group;
  const int tn = (t % gsz) / rows_in_group;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const char *xb = reinterpret_cast<const char *>(p.x) + (int64_t)m0 * p.x_st * 2;
  const char *wb = reinterpret_cast<const char *>(p.w) + (int64_t)n0 * p.w_st * 2;
  // direct loads: wave w fills rows kL w 8 .. of each tile, 8 rows per
  // instruction; lane -> row 8 i + lane / 8 of its range, LDS block lane % 8,
  // which holds global block (lane % 8) ^ swz(row).  Rows past M / N repeat
  // the last row (their results are not stored).
  uint32_t ox[kLX], ow[kLW];
#pragma unroll
  for (int i = 0; i < kLX; ++i) {
    const int r = 8 * (kLX * wave + i) + (lane >> 3);
    ox[i] = (uint32_t)min(r, p.M - 1 - m0) * (uint32_t)p.x_st * 2 + 16 * ((lane & 7) ^ swz(r));
  }
#pragma unroll
  for (int i = 0; i < kLW; ++i) {
    const int r = 8 * (kLW * wave + i) + (lane >> 3);
    ow[i] = (uint32_t)min(r, p.N - 1 - n0) * (uint32_t)p.w_st * 2 + 16 * ((lane & 7) ^ swz(r));
  }
  auto issue = [&](int buf, int k0) {
    const char *xk = xb + (int64_t)k0 * 2, *wk = wb + (int64_t)k0 * 2;
#pragma unroll
    for (int i = 0; i < kLX; ++i)
      load_lds16(xk + ox[i], (lds_u8 *)lin_smem + kXOff + buf * BM * 128 + 8 * (kLX * wave + i) * 128);
#pragma unroll
    for (int i = 0; i < kLW; ++i)
      load_lds16(wk + ow[i], (lds_u8 *)lin_smem + kWOff + buf * BN * 128 + 8 * (kLW * wave + i) * 128);
  };

  // this wave's block: w rows (y columns) wn .., x rows (y rows) wm ..
  const int wmi = wave / kWN;
  const int wn = 32 * kTN * (wave % kWN), wm = 32 * kTM * wmi;
  const int l32 = lane & 31, hk = lane >> 5;
  f32x16 acc[kTN][kTM];  // [n tile][m tile]: y^T[n][m]
#pragma unroll
  for (int a = 0; a < kTN; ++a)
#pragma unroll
    for (int b = 0; b < kTM; ++b) acc[a][b] = f32x16{};

  const int nk = p.K / kBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(buf ^ 1, (kt + 1) * kBK);
    const lds_u8 *Wt = (const lds_u8 *)lin_smem + kWOff + buf * BN * 128;
    const lds_u8 *Xt = (const lds_u8 *)lin_smem + kXOff + buf * BM * 128;
    // operand fragments: row l32 of the 32-row block, K values 16 s + 8 hk .. + 7.
    // Double-buffered: sub-step s + 1's reads go out before sub-step s's
    // products, so the matrix core never waits for the LDS latency of the
    // step it is about to run (only the first sub-step after the barrier does).
    bf16x8 fw[2][kTN], fx[2][kTM];
    auto read_frags = [&](int s, int slot) {
#pragma unroll
      for (int a = 0; a < kTN; ++a)
        fw[slot][a] = *reinterpret_cast<const SSD_LDS bf16x8 *>(Wt + blk_off(wn + 32 * a + l32, 2 * s + hk));
#pragma unroll
      for (int b = 0; b < kTM; ++b)
        fx[slot][b] = *reinterpret_cast<const SSD_LDS bf16x8 *>(Xt + blk_off(wm + 32 * b + l32, 2 * s + hk));
    };
    read_frags(0, 0);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      if (s + 1 < kBK / 16) read_frags(s + 1, (s + 1) & 1);
      // keeps the next sub-step's reads ahead of this one's products
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < kTN; ++a)
#pragma unroll
        for (int b = 0; b < kTM; ++b) acc[a][b] = mfma32(fw[s & 1][a], fx[s & 1][b], acc[a][b]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next K step has landed (this wave's loads)
    __syncthreads();                // ... every wave's, and this one's reads are done
  }

  // y^T tile [n][m] in the accumulators: lane holds m = wm + 32 b + l32 and
  // n = wn + 32 a + 8 (r / 4) + 4 hk + (r % 4) -> 4 consecutive n per r / 4.
  // One row of waves at a time stages its 32 kTM rows, then all threads store them.
  lds_u8 *st = (lds_u8 *)lin_smem;
  char *yb = reinterpret_cast<char *>(p.y) + (int64_t)m0 * p.y_st * 2 + (int64_t)n0 * 2;
  constexpr int kRows = 32 * kTM;
  constexpr int kPieces = kRows * BN / 8;  // 16-byte pieces of one staged row block
#pragma unroll
  for (int mg = 0; mg < kWM; ++mg) {
    if (wmi == mg) {
#pragma unroll
      for (int a = 0; a < kTN; ++a)
#pragma unroll
        for (int b = 0; b < kTM; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = 32 * b + l32, n = wn + 32 * a + 8 * q + 4 * hk;
            u32x2 v;
            v[0] = pack2_bf16(acc[a][b][4 * q], acc[a][b][4 * q + 1]);
            v[1] = pack2_bf16(acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
            *reinterpret_cast<SSD_LDS u32x2 *>(st + m * Cf::kStageRowB + n * 2) = v;
          }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (kPieces + kThr - 1) / kThr; ++i) {
      const int c = tid + kThr * i;
      const int row = c / (BN / 8), col = 8 * (c % (BN / 8));
      const int m = 32 * kTM * mg + row;
      if (c < kPieces && m0 + m < p.M && n0 + col < p.N) {
        const u32x4 v = *reinterpret_cast<const SSD_LDS u32x4 *>(st + row * Cf::kStageRowB + col * 2);
        *reinterpret_cast<u32x4 *>(yb + (int64_t)m * p.y_st * 2 + col * 2) = v;
      }
    }
    if (mg + 1 < kWM) __syncthreads();  // the staging rows are rewritten by the next row of waves
  }
}

template <int kWM, int kWN, int kTM, int kTN>
hipError_t launch_cfg(const LinearParams &p, hipStream_t stream) {
  using Cf = LinCfg<kWM, kWN, kTM, kTN>;
  const int ntm = (p.M + Cf::BM - 1) / Cf::BM, ntn = (p.N + Cf::BN - 1) / Cf::BN;
  const long long T = (long long)ntm * ntn;
  if (T == 0) return hipSuccess;
  const long long per = (T + kNumXCD - 1) / kNumXCD;
  const size_t lds = Cf::kLds;
  const hipError_t e =
      set_max_dynamic_lds(reinterpret_cast<const void *>(linear_bf16_kernel<kWM, kWN, kTM, kTN>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((linear_bf16_kernel<kWM, kWN, kTM, kTN>), dim3((unsigned)(per * kNumXCD)), dim3(Cf::kThr), lds,
                     stream, p, ntm, ntn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bf16(const LinearParams &p, hipStream_t stream) {
  // 256 x 256 tiles once both sides give at least 8 of them; 128 x 128 below
  if (p.M >= 2048 && p.N >= 2048) return launch_cfg<2, 4, 4, 2>(p, stream);
  return launch_cfg<2, 2, 2, 2>(p, stream);
}

}  // namespace ssd
