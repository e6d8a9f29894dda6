// Device helpers shared by the gfx950 kernels of libssd.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef uint16_t bf16_t;  // storage of a bfloat16 value
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round to nearest even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats -> one dword of two bf16 (lo in the low half), one instruction.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// softplus(z) = log(1 + e^z); log1pf keeps full precision for very negative z
// (dt_bias pushes z down to about -11 for the smallest time steps).
__device__ __forceinline__ float softplus_f32(float z) {
  return z > 20.f ? z : log1pf(__expf(z));
}

// SiLU(u) = u * sigmoid(u), with the hardware reciprocal (about 1 ulp) in place
// of an IEEE division sequence: the result is rounded to the I/O dtype anyway.
// Very negative u gives exp(-u) = inf, rcp(inf) = 0 and the limit -0.
__device__ __forceinline__ float silu_f32(float u) {
  return u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
}

// The value held by the lane paired with this one across lane bit BIT of a
// 16-lane row, by a DPP move (a VALU operand modifier, no LDS round trip):
// the row mirror pairs across bit 3, the half-row mirror across bit 2 (lane
// i with 7 - i), the quad permutations across bits 1 and 0.  Each pairing
// keeps the lower bits' partition: lanes paired at one step held the same
// column set after the steps over the higher bits.
template <int BIT> __device__ __forceinline__ float row_pair(float v) {
  constexpr int ctrl = BIT == 3 ? 0x140 : BIT == 2 ? 0x141 : BIT == 1 ? 0x4E : 0xB1;
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Reduce-scatter of CNT sums over the 32 lanes of a half-wave: steps over
// lane bits 3, 2, 1, 0 (DPP) split the column set in halves while CNT > 1 and
// add whole sums after; a last step over bit 4 crosses the two rows.  Lane
// bit b's step leaves the upper lane of each pair with the upper half, so the
// column a lane ends with is read off the bits it split on (rsel).
template <int CNT, int BIT> struct RowScatter {
  static __device__ __forceinline__ void run(float *part, int lane32, int &rsel) {
    const bool upper = (lane32 >> BIT) & 1;
    if constexpr (CNT > 1) {
      constexpr int half = CNT / 2;
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const float send = upper ? part[j] : part[j + half];
        const float keep = upper ? part[j + half] : part[j];
        part[j] = keep + row_pair<BIT>(send);
      }
      rsel += upper ? half : 0;
      RowScatter<half, BIT - 1>::run(part, lane32, rsel);
    } else {
      part[0] += row_pair<BIT>(part[0]);
      RowScatter<1, BIT - 1>::run(part, lane32, rsel);
    }
  }
};
// The sum of the two 16-lane rows of each half-wave, in every lane of both:
// v_permlane16_swap with the value as both operands leaves row 0 of each
// half in the first result and row 1 in the second (a VALU op, no LDS).
__device__ __forceinline__ float cross_row_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// ... and of the two half-waves (v_permlane32_swap).
__device__ __forceinline__ float cross_half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CNT> struct RowScatter<CNT, -1> {
  static_assert(CNT == 1, "at most 16 sums per row");
  static __device__ __forceinline__ void run(float *part, int, int &) { part[0] = cross_row_sum(part[0]); }
};
// lanes holding a finished sum with every all-reduced bit zero: one writer per column
template <int R> constexpr int kRowWriterMask = 0x10 | ((16 / R) - 1);

// Sum over the 16 lanes of a row (every lane gets it), by DPP moves.
__device__ __forceinline__ float row_sum16(float v) {
  v += row_pair<3>(v);
  v += row_pair<2>(v);
  v += row_pair<1>(v);
  return v + row_pair<0>(v);
}
// ... over the 32 lanes of a half-wave (the last step crosses the two rows).
__device__ __forceinline__ float half_wave_sum(float v) { return cross_row_sum(row_sum16(v)); }
// ... over the whole wave.
__device__ __forceinline__ float wave_sum(float v) { return cross_half_sum(half_wave_sum(v)); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

}  // namespace ssd
