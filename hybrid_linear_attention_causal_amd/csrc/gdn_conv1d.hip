// Causal depthwise conv1d (width 4, no bias) + SiLU over packed sequences.
//
// Operation: llm-arch-viz Qwen3.5-9B page, module tree (conv1d 8192x1x4 inside
// Qwen3_5GatedDeltaNet: one 4-tap filter per channel, no bias); the conv state
// carried between calls is the one of the KerasFormers Qwen page, "Generation".
//
// Layout: x, y [N, Cq] row-major (channels contiguous); each thread owns 8
// consecutive channels of a tile of 32 (bf16) or 16 (fp32) tokens, so every row of x
// is read with 16-byte (bf16) or 32-byte (fp32) coalesced loads and the only re-read
// is the 3-row halo of each tile.  A tile that lies inside one sequence issues all its
// row loads at once (the kernel is bound by HBM, not by one load's latency per token);
// a tile that crosses a sequence end walks its tokens one by one.
// The final conv state is written by a second kernel after the main pass has
// consumed conv_state_in, which makes in-place state updates safe.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// tokens per thread: bf16 rows stay packed (4 VGPRs each), fp32 rows take 8
template <int IO> constexpr int conv_tt() { return IO == IO_BF16 ? 32 : 16; }
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

// 8 consecutive io elements kept as raw words until use
template <int IO> struct Row8;
template <> struct Row8<IO_BF16> {
  uint4 w;
  __device__ __forceinline__ void load(const u16* p) { w = *reinterpret_cast<const uint4*>(p); }
  // nontemporal: x is read once per call (its halo rows come from L2 either way)
  __device__ __forceinline__ void load_nt(const u16* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w = make_uint4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void get(float* v) const {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(u[j] << 16);
      v[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  }
};
template <> struct Row8<IO_F32> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void load_nt(const float* p) { load(p); }   // (fp32: plain)
  __device__ __forceinline__ void get(float* v) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Two workgroups per CU: a 4096-token batch of 8192 bf16 channels is one pass of 512
// workgroups.  Workgroup b takes channel group b % groups of token tile b / groups: the
// groups that share a tile's rows are consecutive in launch order, so each row is
// fetched from HBM by workgroups that run together.
template <int IO>
__global__ void __launch_bounds__(CONV_BLOCK, 2)
conv1d_silu_kernel(const typename Io<IO>::T* __restrict__ x, const float* __restrict__ w,
                   typename Io<IO>::T* __restrict__ y, const int32_t* __restrict__ cu, int Ns,
                   int64_t N, int Cq, const typename Io<IO>::T* __restrict__ state_in,
                   int groups) {
  typedef Io<IO> io;
  const int64_t b = blockIdx.x;
  const int c0 = ((int)(b % groups) * CONV_BLOCK + threadIdx.x) * 8;
  if (c0 >= Cq) return;
  constexpr int CONV_TT = conv_tt<IO>();
  const int64_t t0 = (b / groups) * CONV_TT;
  if (t0 >= N) return;
  const int64_t t1 = t0 + CONV_TT < N ? t0 + CONV_TT : N;

  float4 wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wt[j] = *reinterpret_cast<const float4*>(w + (int64_t)(c0 + j) * 4);

  int s = cu ? find_seq(cu, Ns, t0) : 0;
  int64_t sb = cu ? (int64_t)cu[s] : 0;
  int64_t se = cu ? (int64_t)cu[s + 1] : N;

  if (t0 + CONV_TT <= se) {
    // the whole tile lies in sequence s: rows t0-3 .. t0+CONV_TT-1, the ones before the
    // sequence start from its conv state (or zeros)
    Row8<IO> rows[CONV_TT + 3];
#pragma unroll
    for (int r = 0; r < CONV_TT + 3; ++r) {
      const int64_t p = t0 - 3 + r;
      if (p >= sb)
        rows[r].load_nt(x + p * Cq + c0);
      else if (state_in)
        rows[r].load(state_in + ((int64_t)s * 3 + (p - sb + 3)) * Cq + c0);
      else
        rows[r].zero();
    }
#pragma unroll
    for (int t = 0; t < CONV_TT; ++t) {
      float v0[8], v1[8], v2[8], v3[8], out[8];
      rows[t].get(v0);
      rows[t + 1].get(v1);
      rows[t + 2].get(v2);
      rows[t + 3].get(v3);
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = conv4_silu(wt[j], v0[j], v1[j], v2[j], v3[j]);
      // nontemporal: y is written once here and read by the next call
      if constexpr (IO == IO_BF16) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = {f2bf2(out[0], out[1]), f2bf2(out[2], out[3]), f2bf2(out[4], out[5]),
                         f2bf2(out[6], out[7])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y + (t0 + t) * Cq + c0));
      } else {
        io::st8(y, (t0 + t) * Cq + c0, out);
      }
    }
    return;
  }

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
      out[j] = conv4_silu(wt[j], h[0][j], h[1][j], h[2][j], xv[j]);
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
static hipError_t conv_impl(const ConvArgs& a, bool main_pass, hipStream_t st) {
  typedef typename Io<IO>::T T;
  const int groups = (a.Cq / 8 + CONV_BLOCK - 1) / CONV_BLOCK;
  if (main_pass && a.N > 0) {
    const int64_t tiles = (a.N + conv_tt<IO>() - 1) / conv_tt<IO>();
    if (tiles * groups > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(conv1d_silu_kernel<IO>, dim3((unsigned)(tiles * groups)),
                       dim3(CONV_BLOCK), 0, st, (const T*)a.x, a.w, (T*)a.y, a.cu, a.Ns, a.N,
                       a.Cq, (const T*)a.state_in, groups);
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
  return io == IO_BF16 ? conv_impl<IO_BF16>(a, true, s) : conv_impl<IO_F32>(a, true, s);
}

hipError_t launch_conv_state(const ConvArgs& a, int io, hipStream_t s) {
  return io == IO_BF16 ? conv_impl<IO_BF16>(a, false, s) : conv_impl<IO_F32>(a, false, s);
}

}  // namespace gdn
