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

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

}  // namespace ssd
