// Causal depthwise conv1d (width 4, no bias) + SiLU over packed sequences.
//
// Operation: llm-arch-viz Qwen3.5-9B page, module tree (conv1d 8192x1x4 inside
// Qwen3_5GatedDeltaNet: one 4-tap filter per channel, no bias); the conv state
// carried between calls is the one of the KerasFormers Qwen page, "Generation".
//
// Layout: x, y [N, Cq] row-major (channels contiguous); each thread owns 8
// consecutive channels and walks a tile of tokens, keeping the 3-row history
// in registers, so every row of x is read with 16-byte (bf16) or 32-byte
// (fp32) coalesced loads and the only re-read is the 3-row halo of each tile.
// The final conv state is written by a second kernel after the main pass has
// consumed conv_state_in, which makes in-place state updates safe.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int CONV_TT = 32;      // tokens per thread
constexpr int CONV_BLOCK = 256;  // threads per block (channel groups)

// largest s with cu[s] <= t: the (non-empty) sequence that holds token t
__device__ __forceinline__ int find_seq(const int32_t* cu, int Ns, int64_t t) {
  int lo = 0, hi = Ns - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int IO>
__global__ void __launch_bounds__(CONV_BLOCK)
conv1d_silu_kernel(const typename Io<IO>::T* __restrict__ x, const float* __restrict__ w,
                   typename Io<IO>::T* __restrict__ y, const int32_t* __restrict__ cu, int Ns,
                   int64_t N, int Cq, const typename Io<IO>::T* __restrict__ state_in) {
  typedef Io<IO> io;
  const int c0 = (blockIdx.y * CONV_BLOCK + threadIdx.x) * 8;
  if (c0 >= Cq) return;
  const int64_t t0 = (int64_t)blockIdx.x * CONV_TT;
  if (t0 >= N) return;
  const int64_t t1 = t0 + CONV_TT < N ? t0 + CONV_TT : N;

  float wt[4][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 ww = *reinterpret_cast<const float4*>(w + (int64_t)(c0 + j) * 4);
    wt[0][j] = ww.x; wt[1][j] = ww.y; wt[2][j] = ww.z; wt[3][j] = ww.w;
  }

  int s = cu ? find_seq(cu, Ns, t0) : 0;
  int64_t sb = cu ? (int64_t)cu[s] : 0;
  int64_t se = cu ? (int64_t)cu[s + 1] : N;

  // h[0] = row t-3, h[1] = row t-2, h[2] = row t-1
  float h[3][8];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int64_t p = t0 - 3 + r;
    if (p >= sb) {
      io::ld8(x, p * Cq + c0, h[r]);
    } else if (state_in) {
      io::ld8(state_in, ((int64_t)s * 3 + (p - sb + 3)) * Cq + c0, h[r]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[r][j] = 0.f;
    }
  }

  for (int64_t t = t0; t < t1; ++t) {
    if (t >= se) {  // a new sequence starts at t (skip empty ones)
      while (t >= se && s < Ns - 1) {
        ++s;
        sb = cu[s];
        se = cu[s + 1];
      }
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        if (state_in) {
          io::ld8(state_in, ((int64_t)s * 3 + r) * Cq + c0, h[r]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) h[r][j] = 0.f;
        }
      }
    }
    float xv[8], out[8];
    io::ld8(x, t * Cq + c0, xv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float acc = wt[0][j] * h[0][j];
      acc = fmaf(wt[1][j], h[1][j], acc);
      acc = fmaf(wt[2][j], h[2][j], acc);
      acc = fmaf(wt[3][j], xv[j], acc);
      out[j] = silu(acc);
      h[0][j] = h[1][j];
      h[1][j] = h[2][j];
      h[2][j] = xv[j];
    }
    io::st8(y, t * Cq + c0, out);
  }
}

// conv_state_out[s] = last 3 rows of [conv_state_in[s]; x rows of s] (raw bits)
template <int IO>
__global__ void __launch_bounds__(CONV_BLOCK)
conv_state_kernel(const typename Io<IO>::T* __restrict__ x, const int32_t* __restrict__ cu,
                  int64_t N, int Cq, const typename Io<IO>::T* state_in,
                  typename Io<IO>::T* state_out) {
  typedef typename Io<IO>::T T;
  constexpr int NV = Io<IO>::BYTES / 2;  // uint4 words per 8 elements
  const int c0 = (blockIdx.y * CONV_BLOCK + threadIdx.x) * 8;
  if (c0 >= Cq) return;
  const int s = blockIdx.x;
  // offsets are clamped to [0, N] so inconsistent cu_seqlens cannot index outside x
  const int64_t se = cu ? min((int64_t)cu[s + 1], N) : N;
  const int64_t sb = cu ? max((int64_t)0, min((int64_t)cu[s], se)) : 0;
  uint4 rows[3][NV];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int64_t p = se - 3 + r;
    const T* src = nullptr;
    if (p >= sb) src = x + p * Cq + c0;
    else if (state_in) src = state_in + ((int64_t)s * 3 + (p - sb + 3)) * Cq + c0;
#pragma unroll
    for (int u = 0; u < NV; ++u)
      rows[r][u] = src ? reinterpret_cast<const uint4*>(src)[u] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    T* dst = state_out + ((int64_t)s * 3 + r) * Cq + c0;
#pragma unroll
    for (int u = 0; u < NV; ++u) reinterpret_cast<uint4*>(dst)[u] = rows[r][u];
  }
}

template <int IO>
static hipError_t conv_impl(const ConvArgs& a, hipStream_t st) {
  typedef typename Io<IO>::T T;
  const int groups = (a.Cq / 8 + CONV_BLOCK - 1) / CONV_BLOCK;
  if (a.N > 0) {
    const int64_t tiles = (a.N + CONV_TT - 1) / CONV_TT;
    dim3 grid((unsigned)tiles, (unsigned)groups);
    hipLaunchKernelGGL(conv1d_silu_kernel<IO>, grid, dim3(CONV_BLOCK), 0, st,
                       (const T*)a.x, a.w, (T*)a.y, a.cu, a.Ns, a.N, a.Cq,
                       (const T*)a.state_in);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.state_out) {
    dim3 grid((unsigned)a.Ns, (unsigned)groups);
    hipLaunchKernelGGL(conv_state_kernel<IO>, grid, dim3(CONV_BLOCK), 0, st, (const T*)a.x, a.cu,
                       a.N, a.Cq, (const T*)a.state_in, (T*)a.state_out);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_conv1d(const ConvArgs& a, int io, hipStream_t s) {
  return io == IO_BF16 ? conv_impl<IO_BF16>(a, s) : conv_impl<IO_F32>(a, s);
}

}  // namespace gdn
