// Shared device helpers for the gfx950 kernels: storage types, conversions,
// MFMA fragment traits and wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

#define SF_WAVE 64

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
// round to nearest even (inputs are finite)
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// 16-byte vector of T (8 bf16 or 4 fp32) for global/LDS copies.
struct alignas(16) vec16 { uint32_t w[4]; };

// MFMA 16x16 fragment traits. A operand tile is [16 rows][K] and B operand
// tile is [16 cols][K], both K-contiguous in memory; lane l supplies row/col
// l%16. D (f32x4) holds rows 4*(l/16)+i, column l%16. Both operands use the
// same K->lane mapping, so the product does not depend on which K slice the
// hardware assigns to which lane group.
template <typename T> struct MF;
template <> struct MF<float> {
  static constexpr int KI = 4;  // K per instruction
  typedef float frag;
  __device__ __forceinline__ static frag ld(const float* row_k0, int lane) {
    return row_k0[lane >> 4];
  }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <> struct MF<bf16_t> {
  static constexpr int KI = 32;
  typedef bf16x8_t frag;
  __device__ __forceinline__ static frag ld(const bf16_t* row_k0, int lane) {
    return *reinterpret_cast<const bf16x8_t*>(row_k0 + 8 * (lane >> 4));
  }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// reductions over the 16 lanes that share l/16 (one MFMA D row group)
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ __forceinline__ float swishf_(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ float geluf_(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
