// z-gated RMSNorm over rows of 128 values:  y = w * o / sqrt(mean(o^2) + eps) * silu(z).
//
// Operation: llm-arch-viz Qwen3.5-9B page, module tree (norm Qwen3_5RMSNormGated
// with a 128-wide weight shared by every value head); eps 1e-6 from the
// KerasFormers Qwen3.5 page, "API" table (norm_eps).  The weight multiplies
// directly and the gate silu(z) is applied after normalisation.
//
// Layout: 16 lanes per row, 8 contiguous values per lane (one 16-byte bf16 or
// 32-byte fp32 load of o and of z), row sum of squares reduced with
// cross-lane shuffles inside each 16-lane group; 16 rows per 256-thread block.
// HBM-bound: 3 * 128 * sizeof(io) bytes per row.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int NORM_D = 128;
constexpr int NORM_BLOCK = 256;
constexpr int NORM_ROWS_PER_BLOCK = NORM_BLOCK / 16;

template <int IO>
__global__ void __launch_bounds__(NORM_BLOCK)
gated_rmsnorm_kernel(const typename Io<IO>::T* o, const typename Io<IO>::T* __restrict__ z,
                     const float* __restrict__ w, typename Io<IO>::T* y, int64_t rows,
                     float eps) {
  typedef Io<IO> io;
  const int l16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * NORM_ROWS_PER_BLOCK + (threadIdx.x >> 4);
  if (row >= rows) return;  // whole 16-lane groups leave together
  const int64_t base = row * NORM_D + l16 * 8;
  float ov[8], zv[8], wv[8];
  io::ld8(o, base, ov);
  io::ld8(z, base, zv);
  const float4 w0 = *reinterpret_cast<const float4*>(w + l16 * 8);
  const float4 w1 = *reinterpret_cast<const float4*>(w + l16 * 8 + 4);
  wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
  wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(ov[j], ov[j], ss);
  ss = group_sum<16>(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / NORM_D) + eps);
  float out[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = wv[j] * (ov[j] * inv) * silu(zv[j]);
  io::st8(y, base, out);
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, int io, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int64_t blocks = (a.rows + NORM_ROWS_PER_BLOCK - 1) / NORM_ROWS_PER_BLOCK;
  if (io == IO_BF16) {
    typedef Io<IO_BF16>::T T;
    hipLaunchKernelGGL(gated_rmsnorm_kernel<IO_BF16>, dim3((unsigned)blocks), dim3(NORM_BLOCK), 0,
                       s, (const T*)a.o, (const T*)a.z, a.w, (T*)a.y, a.rows, a.eps);
  } else {
    hipLaunchKernelGGL(gated_rmsnorm_kernel<IO_F32>, dim3((unsigned)blocks), dim3(NORM_BLOCK), 0,
                       s, (const float*)a.o, (const float*)a.z, a.w, (float*)a.y, a.rows, a.eps);
  }
  return hipGetLastError();
}

}  // namespace gdn
