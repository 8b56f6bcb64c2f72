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

// round-to-nearest-even fp32 -> bf16 on the hardware converter (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }
// two values packed, a in the low half
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
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
    a.x = f2bf2(v[0], v[1]);
    a.y = f2bf2(v[2], v[3]);
    a.z = f2bf2(v[4], v[5]);
    a.w = f2bf2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p + i) = a;
  }
  __device__ static __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};

// ---------------------------------------------------------------- activations
// x sigmoid(x) on the hardware exp2 and reciprocal (a few ulp of fp32; e^{-x} rounding to
// +inf for very negative x gives the limit 0)
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
// one output of the causal depthwise conv (width 4) + SiLU: taps w.x .. w.w applied to
// the inputs at t-3 .. t, in this order of fp32 operations.  Every kernel that forms
// conv outputs calls this, so that they agree bit for bit.
__device__ __forceinline__ float conv4_silu(float4 w, float x0, float x1, float x2, float x3) {
  float acc = w.x * x0;
  acc = fmaf(w.y, x1, acc);
  acc = fmaf(w.z, x2, acc);
  acc = fmaf(w.w, x3, acc);
  return silu(acc);
}
// 1 / (1 + e^{-x}) on the hardware exp2 and reciprocal (a few ulp)
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
// log(1 + e^x) on the hardware exp2 and log2, a few ulp relative: with u = 1 + e^x rounded,
// log1p(e) = log(u) e / (u - 1) cancels the rounding of u (Goldberg's log1p), and u == 1
// (e below half an ulp of 1) gives e itself; for x > 20 the correction is below fp32
// resolution
__device__ __forceinline__ float softplus(float x) {
  if (x > 20.0f) return x;
  const float e = __expf(x);
  const float u = 1.0f + e;
  return u == 1.0f ? e : __logf(u) * (e * __builtin_amdgcn_rcpf(u - 1.0f));
}

// gate pair of the gated delta rule: g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b)
__device__ __forceinline__ void gate_pair(float a, float b, float A_log, float dt_bias, float& g,
                                          float& beta) {
  g = -__expf(A_log) * softplus(a + dt_bias);
  beta = sigmoid(b);
}

// ---------------------------------------------------------------- DPP cross-lane ops
// (VALU data-parallel primitives: no LDS round trip)
template <int CTRL, int ROW_MASK = 0xf, bool BOUND_ZERO = true>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                    BOUND_ZERO));
}

// sum over each DPP row of 16 lanes; every lane receives its row's total
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: quads
  v += dpp<0x141>(v);   // row_half_mirror: the two quads of each half row
  v += dpp<0x140>(v);   // row_mirror: the two halves of the row
  return v;
}

// inclusive prefix sum over the 64 lanes of a wavefront
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp<0x111>(v);            // row_shr:1  (lanes shifted in from outside the row read 0)
  v += dpp<0x112>(v);            // row_shr:2
  v += dpp<0x114>(v);            // row_shr:4
  v += dpp<0x118>(v);            // row_shr:8   -> inclusive scan inside each row of 16
  v += dpp<0x142, 0xa, false>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xc, false>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// ---------------------------------------------------------------- barriers
// Workgroup barrier that orders LDS accesses only: this wave's LDS reads and writes have
// completed (lgkmcnt 0) when it arrives, while its global loads, stores and LDS DMA
// copies stay in flight (a __syncthreads() also waits for those: vmcnt 0).  For kernels
// whose barriers order no global memory between threads.  The signal fences keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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
