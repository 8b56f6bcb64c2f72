// Shared device helpers for the gfx950 Gated DeltaNet kernels: io-dtype traits,
// bf16 conversion, activations and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.hpp"

namespace gdn {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf2f(u16 h) { return __uint_as_float(((uint32_t)h) << 16); }

// round-to-nearest-even fp32 -> bf16 (inputs are finite)
__device__ __forceinline__ u16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// ---------------------------------------------------------------- io traits
template <int IO> struct Io;

template <> struct Io<IO_F32> {
  typedef float T;
  static constexpr int BYTES = 4;
  __device__ static __forceinline__ float ld(const T* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void st(T* p, int64_t i, float v) { p[i] = v; }
  // 8 consecutive elements (p + i must be 32-byte aligned)
  __device__ static __forceinline__ void ld8(const T* p, int64_t i, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    const float4 b = *reinterpret_cast<const float4*>(p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static __forceinline__ void st8(T* p, int64_t i, const float* v) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  // value as it would be stored (identity for fp32)
  __device__ static __forceinline__ float round(float v) { return v; }
};

template <> struct Io<IO_BF16> {
  typedef u16 T;
  static constexpr int BYTES = 2;
  __device__ static __forceinline__ float ld(const T* p, int64_t i) { return bf2f(p[i]); }
  __device__ static __forceinline__ void st(T* p, int64_t i, float v) { p[i] = f2bf(v); }
  // 8 consecutive elements (p + i must be 16-byte aligned)
  __device__ static __forceinline__ void ld8(const T* p, int64_t i, float* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ void st8(T* p, int64_t i, const float* v) {
    uint4 a;
    a.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    a.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    a.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
    a.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
    *reinterpret_cast<uint4*>(p + i) = a;
  }
  __device__ static __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};

// ---------------------------------------------------------------- activations
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }
// log(1 + e^x); for x > 20 the correction is below fp32 resolution
__device__ __forceinline__ float softplus(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

// gate pair of the gated delta rule: g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b)
__device__ __forceinline__ void gate_pair(float a, float b, float A_log, float dt_bias, float& g,
                                          float& beta) {
  g = -expf(A_log) * softplus(a + dt_bias);
  beta = sigmoid(b);
}

// ---------------------------------------------------------------- reductions
// sum over groups of W consecutive lanes (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace gdn
