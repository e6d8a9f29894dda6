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
// One workgroup (4 waves) computes a 128 x 128 tile of y over K in 64-wide
// steps; each wave owns 64 x 64 (2 x 2 tiles of v_mfma_f32_32x32x16_bf16).
//  * x and w tiles arrive by global->LDS direct loads (16 bytes per lane, no
//    register staging), double-buffered: the next K step lands while the
//    current one is multiplied.  The 16-byte blocks of a 128-byte row are
//    XOR-swizzled by (row / 2) % 8, so the 16 lanes of one ds_read_b128
//    phase (16 consecutive rows, one block column) hit all 64 banks once.
//  * The product is taken as y^T per tile (w rows as the first operand), so
//    each lane's accumulator holds 4 consecutive output columns of one row:
//    8-byte LDS writes into a padded staging tile, then whole 16-byte row
//    pieces go out to HBM.
//  * Tiles are dealt to the XCDs in contiguous ranges, grouped 16 tile rows
//    deep, so the workgroups sharing an x row block or a w column block run
//    on one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace ssd {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kThr = 256;
constexpr int kGroupM = 16;
constexpr int kStageRowB = 136 * 2;  // staging row: 128 bf16 + 8 of padding (16-byte aligned rows)

#define SSD_LDS __attribute__((address_space(3)))
typedef SSD_LDS void lds_void;
typedef SSD_LDS uint8_t lds_u8;

struct LinSmem {
  uint8_t W[2][kBN * kBK * 2];  // w rows n of the tile, K-contiguous, swizzled
  uint8_t X[2][kBM * kBK * 2];  // x rows m
};
static_assert(kBM * kStageRowB <= sizeof(LinSmem), "the output staging tile overlays the operand tiles");

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// byte offset of 16-byte block `blk` of row `row` in a 128-byte-row tile
__device__ __forceinline__ uint32_t blk_off(int row, int blk) { return row * 128 + ((blk ^ swz(row)) << 4); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThr, 2) void linear_bf16_kernel(LinearParams p, int ntm, int ntn) {
  __shared__ __attribute__((aligned(16))) LinSmem sm;
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
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const char *xb = reinterpret_cast<const char *>(p.x) + (int64_t)m0 * p.x_st * 2;
  const char *wb = reinterpret_cast<const char *>(p.w) + (int64_t)n0 * p.w_st * 2;
  // direct loads: wave w fills rows 32 w .. 32 w + 31 of both tiles, 8 rows per
  // instruction; lane -> row 8 i + lane / 8 of that range, LDS block lane % 8,
  // which holds global block (lane % 8) ^ swz(row).  Rows past M / N repeat the
  // last row (their results are not stored).
  uint32_t ox[4], ow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int blk = (lane & 7) ^ swz(r);
    ox[i] = (uint32_t)min(r, p.M - 1 - m0) * (uint32_t)p.x_st * 2 + 16 * blk;
    ow[i] = (uint32_t)min(r, p.N - 1 - n0) * (uint32_t)p.w_st * 2 + 16 * blk;
  }
  auto issue = [&](int buf, int k0) {
    const char *xk = xb + (int64_t)k0 * 2, *wk = wb + (int64_t)k0 * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds(xk + ox[i], (lds_void *)((lds_u8 *)sm.X[buf] + (32 * wave + 8 * i) * 128),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(wk + ow[i], (lds_void *)((lds_u8 *)sm.W[buf] + (32 * wave + 8 * i) * 128),
                                       16, 0, 0);
    }
  };

  // this wave's 64 x 64: columns (w rows) 64 (wave % 2) .., rows (x rows) 64 (wave / 2) ..
  const int wn = 64 * (wave & 1), wm = 64 * (wave >> 1);
  const int l32 = lane & 31, hk = lane >> 5;
  f32x16 acc[2][2];  // [n tile][m tile]: y^T[n][m]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int nk = p.K / kBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(buf ^ 1, (kt + 1) * kBK);
    const lds_u8 *Wt = (const lds_u8 *)sm.W[buf];
    const lds_u8 *Xt = (const lds_u8 *)sm.X[buf];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      // operand fragment: row l32 of the 32-row block, K values 16 s + 8 hk .. + 7
      bf16x8 fw[2], fx[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        fw[a] = *reinterpret_cast<const SSD_LDS bf16x8 *>(Wt + blk_off(wn + 32 * a + l32, 2 * s + hk));
        fx[a] = *reinterpret_cast<const SSD_LDS bf16x8 *>(Xt + blk_off(wm + 32 * a + l32, 2 * s + hk));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(fw[a], fx[b], acc[a][b]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next K step has landed (this wave's loads)
    __syncthreads();                // ... every wave's, and this one's reads are done
  }

  // y^T tile [n][m] in the accumulators: lane holds m = wm + 32 b + l32 and
  // n = wn + 32 a + 8 (r / 4) + 4 hk + (r % 4) -> 4 consecutive n per r / 4
  lds_u8 *st = (lds_u8 *)&sm;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm + 32 * b + l32, n = wn + 32 * a + 8 * q + 4 * hk;
        u32x2 v;
        v[0] = pack2_bf16(acc[a][b][4 * q], acc[a][b][4 * q + 1]);
        v[1] = pack2_bf16(acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
        *reinterpret_cast<SSD_LDS u32x2 *>(st + m * kStageRowB + n * 2) = v;
      }
  __syncthreads();
  char *yb = reinterpret_cast<char *>(p.y) + (int64_t)m0 * p.y_st * 2 + (int64_t)n0 * 2;
#pragma unroll
  for (int i = 0; i < kBM * kBN / 8 / kThr; ++i) {
    const int c = tid + kThr * i;
    const int row = c >> 4, col = 8 * (c & 15);
    if (m0 + row < p.M && n0 + col < p.N) {
      const u32x4 v = *reinterpret_cast<const SSD_LDS u32x4 *>(st + row * kStageRowB + col * 2);
      *reinterpret_cast<u32x4 *>(yb + (int64_t)row * p.y_st * 2 + col * 2) = v;
    }
  }
}

}  // namespace

hipError_t launch_linear_bf16(const LinearParams &p, hipStream_t stream) {
  const int ntm = (p.M + kBM - 1) / kBM, ntn = (p.N + kBN - 1) / kBN;
  const long long T = (long long)ntm * ntn;
  if (T == 0) return hipSuccess;
  const long long per = (T + kNumXCD - 1) / kNumXCD;
  hipLaunchKernelGGL(linear_bf16_kernel, dim3((unsigned)(per * kNumXCD)), dim3(kThr), 0, stream, p, ntm, ntn);
  return hipGetLastError();
}

}  // namespace ssd
