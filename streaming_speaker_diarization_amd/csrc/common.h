// Shared device helpers for the gfx950 kernels: storage types, conversions,
// MFMA fragment traits and wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

#define SF_WAVE 64

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
// round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
typedef float f32x8 __attribute__((ext_vector_type(8)));
// eight floats to one bf16 MFMA operand (four packed conversions)
__device__ __forceinline__ bf16x8_t pack_bf16x8(const float* v) {
  const f32x8 f = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return __builtin_convertvector(f, bf16x8_t);
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

// Reductions over the 16 lanes of each row (lanes 16r..16r+15) with DPP, no
// LDS: quad swaps (xor 1, xor 2), then rotations by 4 and 8 within the row;
// every lane ends with its row's result.
#define SF_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false))
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, SF_DPP(v, 0xB1));
  v = fmaxf(v, SF_DPP(v, 0x4E));
  v = fmaxf(v, SF_DPP(v, 0x124));
  v = fmaxf(v, SF_DPP(v, 0x128));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += SF_DPP(v, 0xB1);
  v += SF_DPP(v, 0x4E);
  v += SF_DPP(v, 0x124);
  v += SF_DPP(v, 0x128);
  return v;
}
#undef SF_DPP

// Whole-wave reductions (all 64 lanes active): the four row results are read
// back as scalars, so the result is wave-uniform.
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// exp and reciprocal on the hardware's transcendental unit (relative error a
// few ulp of fp32, far inside every tolerance of the forward)
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float swishf_(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float geluf_(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
