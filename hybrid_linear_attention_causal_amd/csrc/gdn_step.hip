// Single-token decode of the Gated DeltaNet mixer: conv window + SiLU, L2 norm,
// gates and one gated delta-rule step per value head, with the conv state and
// the fp32 recurrent state updated in place.
//
// Operation: KerasFormers Qwen page, "Generation" (decode carries the per-layer
// conv state and the delta-rule recurrent state); HF Qwen3.5 docs page,
// "Usage tips" (the single-token recurrence is memory-bandwidth-bound).
//
// Work split: one workgroup per (sequence, key head).  It owns the conv
// channels of that key head's q and k and of its r = Hv/Hk value heads, so
// every conv-state element is read and rewritten by exactly one thread, and it
// runs the r value heads HPP (1 or 2) at a time with 256 threads per head.
//
// Barriers order LDS only (lds_barrier: no wait for global loads or stores), since no
// thread reads global memory another thread of the workgroup writes: each conv-state
// channel is read and rewritten by one thread, and every exchange goes through LDS.  So
// the state stores drain while the output and the norm are formed.
//
// State traffic (the roofline): each head's 128 x 128 state (fp32, or bf16 in the
// bf16-state variant: read, computed in fp32, rounded back) is read once and written
// once, with nontemporal loads and stores (the state is touched once per step, so it
// need not displace anything in the caches).  Thread (rg, cg) of a head holds rows 16*rg .. 16*rg+15 of
// columns 4*cg .. 4*cg+3 in registers (16 float4 loads, each wave covering two
// contiguous 512-byte rows per instruction).  S^T k and S^T q are column sums
// over rows: reduced over the 8 row groups with one cross-lane shuffle and an
// LDS exchange between the 4 waves of the head.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int SD = 128;  // head width (dk = dv)

// Four consecutive state values (columns 4 cg .. 4 cg + 3 of one row) at element offset
// i, as stored: fp32 (f32x4) or bf16 (two packed words, kept packed in registers so the
// bf16 variant holds half the registers).  Nontemporal: the state is touched once per step.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <bool SBF> struct StateQuad;

// An io value's bits in a 32-bit register (bf16: zero-extended, fp32: as is), its value,
// and the io value of such bits
template <int IO>
__device__ __forceinline__ uint32_t raw_bits(const typename Io<IO>::T* p, int64_t i) {
  if constexpr (IO == IO_BF16) return (uint32_t)p[i];
  else return __float_as_uint(p[i]);
}
// the aligned 32-bit word holding element i (bf16: two elements; the row bases are
// 16-byte aligned and the channel counts even), and element i's bits from it
template <int IO>
__device__ __forceinline__ uint32_t raw_word(const typename Io<IO>::T* p, int64_t i) {
  if constexpr (IO == IO_BF16) return *reinterpret_cast<const uint32_t*>(p + (i & ~(int64_t)1));
  else return __float_as_uint(p[i]);
}
template <int IO>
__device__ __forceinline__ uint32_t word_bits(uint32_t w, int64_t i) {
  if constexpr (IO == IO_BF16) return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
  else return w;
}
template <int IO>
__device__ __forceinline__ float from_raw_bits(uint32_t w) {
  if constexpr (IO == IO_BF16) return __uint_as_float(w << 16);
  else return __uint_as_float(w);
}
template <int IO>
__device__ __forceinline__ typename Io<IO>::T raw_to_io(uint32_t w) {
  if constexpr (IO == IO_BF16) return (u16)w;
  else return __uint_as_float(w);
}
template <> struct StateQuad<false> {
  typedef f32x4 Raw;
  static __device__ __forceinline__ Raw ld(const void* base, uint32_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>((const float*)base + i));
  }
  static __device__ __forceinline__ f32x4 f32(Raw w) { return w; }
  static __device__ __forceinline__ void st(void* base, uint32_t i, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>((float*)base + i));
  }
};
template <> struct StateQuad<true> {
  typedef u32x2 Raw;
  static __device__ __forceinline__ Raw ld(const void* base, uint32_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>((const u16*)base + i));
  }
  static __device__ __forceinline__ f32x4 f32(Raw w) {
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
  }
  static __device__ __forceinline__ void st(void* base, uint32_t i, f32x4 v) {
    const u32x2 w = {f2bf2(v[0], v[1]), f2bf2(v[2], v[3])};   // round to nearest even
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>((u16*)base + i));
  }
};

// The bf16-state variant holds its state packed and fits four waves per SIMD (two
// 512-thread workgroups per CU); the fp32 one holds 64 state registers and runs three.
template <int IO, int HPP, bool SBF, bool SLOTS, bool NORM>
__global__ void __launch_bounds__(256 * HPP, 4)
recurrent_step_kernel(StepArgs p) {
  typedef Io<IO> io;
  typedef StateQuad<SBF> SQ;
  typedef typename io::T T;
  extern __shared__ float smem[];
  const int Hk = p.Hk, Hv = p.Hv;
  const int r = Hv / Hk;
  const int Cq = 2 * Hk * SD + Hv * SD;
  const int bseq = blockIdx.x / Hk;
  const int kh = blockIdx.x % Hk;
  const int tid = threadIdx.x;
  const int nthr = 256 * HPP;

  // LDS: conv outputs [q | k | v of r heads], then reduction buffers and gates
  float* yv = smem;                          // 256 + r*128
  float* red1 = yv + 256 + r * SD;           // HPP * 4 waves * 128
  float* red2 = red1 + HPP * 4 * SD;         // HPP * 4 * 128
  float* gsh = red2 + HPP * 4 * SD;          // r: decay e^g
  float* bsh = gsh + r;                      // r: beta
  float* zsh = bsh + r + 2;                  // NORM: r * 128 gate values z (after 2 spare)
  float* wsh = zsh + (NORM ? r * SD : 0);    // NORM: 128 norm weights

  const int hl = __builtin_amdgcn_readfirstlane(tid >> 8);   // head slot inside a pass
  const int t256 = tid & 255;
  const int cg = t256 & 31;       // column group: columns 4cg .. 4cg+3
  const int rg = t256 >> 5;       // row group: rows 16rg .. 16rg+15
  const int wv = (t256 >> 6);     // wave within the head's 256 threads
  const int hi_half = (t256 >> 5) & 1;
  // a head's state base is wave-uniform (scalar); the thread's rows and columns are a
  // 32-bit offset from it, row i of the thread's 16 at a further i * SD
  const uint32_t toff = (uint32_t)(rg * 16 * SD + cg * 4);
  // the state and conv-state row of this sequence: its slot in the pools, or the row itself
  int slot = bseq;
  if constexpr (SLOTS) {
    slot = p.slots[bseq];
    if (slot < 0 || slot >= p.n_slots) {
      // padding row: no state is read or written; the group's o rows are zero
      T* ob = (T*)p.o + ((int64_t)bseq * Hv + kh * r) * SD;
      for (int i = tid; i < r * SD; i += nthr) io::st(ob, i, 0.f);
      return;   // uniform over the workgroup
    }
  }
  // (the byte offset is wave-uniform: kept in scalar registers)
  auto head_state = [&](int h) {
    const uint64_t off = (uint64_t)(((int64_t)slot * Hv + h) * SD) * SD * (SBF ? 2 : 4);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)off);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(off >> 32));
    return (char*)p.state + (((uint64_t)hi << 32) | lo);
  };

  // Loads complete in issue order (one counter per wave), so everything the conv and the
  // gates need is issued first and the first pass's state after it: the conv then waits
  // for its own inputs only, while the state streams in behind them.
  const T* xb = (const T*)p.x + (int64_t)bseq * Cq;
  T* cs = (T*)p.conv_state + (int64_t)slot * 3 * Cq;
  const int nch = 256 + r * SD;
  auto conv_channel = [&](int i) {
    if (i < SD) return kh * SD + i;                                   // q channel
    if (i < 2 * SD) return Hk * SD + kh * SD + (i - SD);              // k channel
    return 2 * Hk * SD + kh * r * SD + (i - 2 * SD);                  // v channels
  };
  // Every load before the state's is held as raw bits and read only after the state's
  // loads are issued (the empty asm statements below): a value widened or used inside
  // its branch would make the wave wait for its load there, one round trip at a time.
  // The loads below that not every thread needs are issued by all threads at a clamped
  // (in-bounds) index: a load under a branch gets its register copied where the branch
  // joins, which waits for it.
  // the conv inputs of this thread's first channel (i = tid: there are at least as many
  // channels as threads)
  float4 cw0;
  uint32_t cv0[4];
  {
    const int c = conv_channel(min(tid, nch - 1));
    cw0 = *reinterpret_cast<const float4*>(p.w + (int64_t)c * 4);
    cv0[0] = raw_word<IO>(cs, c);
    cv0[1] = raw_word<IO>(cs, Cq + c);
    cv0[2] = raw_word<IO>(cs, 2 * Cq + c);
    cv0[3] = raw_word<IO>(xb, c);
  }

  // the gate inputs of the r value heads (threads 64 .. 64 + r - 1)
  uint32_t gr_a = 0u, gr_b = 0u, gr_al = 0u, gr_dt = 0u;
  if (tid >= 64 && tid < 64 + r) {
    const int h = kh * r + (tid - 64);
    if (p.g_opt) {
      gr_a = __float_as_uint(p.g_opt[(int64_t)bseq * Hv + h]);
      gr_b = __float_as_uint(p.beta_opt[(int64_t)bseq * Hv + h]);
    } else {
      gr_a = raw_bits<IO>((const T*)p.a, (int64_t)bseq * Hv + h);
      gr_b = raw_bits<IO>((const T*)p.b, (int64_t)bseq * Hv + h);
      gr_al = __float_as_uint(p.A_log[h]);
      gr_dt = __float_as_uint(p.dt_bias[h]);
    }
  }

  // the fused norm's z rows of the r heads (four values per thread, as raw 8-byte words:
  // the first 256 HPP groups of four) and its weights, parked in LDS after the conv
  constexpr int ZW = IO == IO_BF16 ? 1 : 2;
  uint2 zw[ZW];
  float4 wr;
  if constexpr (NORM) {
    const uint2* zp = reinterpret_cast<const uint2*>(
        (const T*)p.z + ((int64_t)bseq * Hv + kh * r) * SD + min(tid, r * 32 - 1) * 4);
#pragma unroll
    for (int w = 0; w < ZW; ++w) zw[w] = zp[w];
    wr = *reinterpret_cast<const float4*>(p.norm_w + min(tid, 31) * 4);
  }

  // the first pass's state, behind the loads above
  __builtin_amdgcn_sched_barrier(0);
  typename SQ::Raw Sv[16];
  {
    const char* sb = head_state(kh * r + hl);
#pragma unroll
    for (int i = 0; i < 16; ++i) Sv[i] = SQ::ld(sb, toff + i * SD);
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" : "+v"(cw0.x), "+v"(cw0.y), "+v"(cw0.z), "+v"(cw0.w));
  asm volatile("" : "+v"(cv0[0]), "+v"(cv0[1]), "+v"(cv0[2]), "+v"(cv0[3]));
  asm volatile("" : "+v"(gr_a), "+v"(gr_b), "+v"(gr_al), "+v"(gr_dt));
  if constexpr (NORM) {
#pragma unroll
    for (int w = 0; w < ZW; ++w) asm volatile("" : "+v"(zw[w].x), "+v"(zw[w].y));
    asm volatile("" : "+v"(wr.x), "+v"(wr.y), "+v"(wr.z), "+v"(wr.w));
  }
  const float gin_a = p.g_opt ? __uint_as_float(gr_a) : from_raw_bits<IO>(gr_a);
  const float gin_b = p.g_opt ? __uint_as_float(gr_b) : from_raw_bits<IO>(gr_b);
  const float gin_al = __uint_as_float(gr_al), gin_dt = __uint_as_float(gr_dt);

  // ---- conv window + SiLU for this group's channels; shift the conv state
  for (int i = tid; i < nch; i += nthr) {
    const int c = conv_channel(i);
    float4 w4;
    uint32_t c0, c1, c2, xc;
    if (i == tid) {
      w4 = cw0;
      c0 = word_bits<IO>(cv0[0], c);
      c1 = word_bits<IO>(cv0[1], c);
      c2 = word_bits<IO>(cv0[2], c);
      xc = word_bits<IO>(cv0[3], c);
    } else {
      w4 = *reinterpret_cast<const float4*>(p.w + (int64_t)c * 4);
      c0 = raw_bits<IO>(cs, c);
      c1 = raw_bits<IO>(cs, Cq + c);
      c2 = raw_bits<IO>(cs, 2 * Cq + c);
      xc = raw_bits<IO>(xb, c);
    }
    const float f0 = from_raw_bits<IO>(c0), f1 = from_raw_bits<IO>(c1);
    const float f2 = from_raw_bits<IO>(c2), fx = from_raw_bits<IO>(xc);
    float acc = w4.x * f0;
    acc = fmaf(w4.y, f1, acc);
    acc = fmaf(w4.z, f2, acc);
    acc = fmaf(w4.w, fx, acc);
    yv[i] = io::round(silu(acc));  // the conv output crosses the io boundary
    cs[c] = raw_to_io<IO>(c1);
    cs[Cq + c] = raw_to_io<IO>(c2);
    cs[2 * Cq + c] = raw_to_io<IO>(xc);
  }
  if constexpr (NORM) {
    if (tid < r * 32) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t b;
        if constexpr (IO == IO_BF16) {
          const uint32_t w = (c >> 1) ? zw[0].y : zw[0].x;
          b = (c & 1) ? (w >> 16) : (w & 0xFFFFu);
        } else {
          const uint2 w = zw[c >> 1];
          b = (c & 1) ? w.y : w.x;
        }
        zsh[tid * 4 + c] = from_raw_bits<IO>(b);
      }
    }
    // more value heads than one z row per thread (r * 32 > threads): the rest of the
    // rows, strided over the workgroup
    for (int i = tid + nthr; i < r * 32; i += nthr) {
      const T* zp = (const T*)p.z + ((int64_t)bseq * Hv + kh * r) * SD + i * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) zsh[i * 4 + c] = io::ld(zp, c);
    }
    if (tid < 32) *reinterpret_cast<float4*>(&wsh[tid * 4]) = wr;
  }
  lds_barrier();

  // ---- L2 norms of q and k: every wave forms them from the staged conv outputs and keeps
  // them in registers (the same lanes and shuffle order in every wave, so the same values),
  // which saves a barrier; gates of the r value heads, read after the first exchange
  // barrier of the head loop
  float rq, rk;
  {
    const int l = tid & 63;
    const float q0 = yv[l], q1 = yv[l + 64], k0 = yv[SD + l], k1 = yv[SD + l + 64];
    const float sq = group_sum<64>(q0 * q0 + q1 * q1);
    const float sk = group_sum<64>(k0 * k0 + k1 * k1);
    // hardware reciprocal square root (about 1 ulp)
    rq = p.use_l2 ? __builtin_amdgcn_rsqf(sq + 1e-6f) : 1.0f;
    rk = p.use_l2 ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 1.0f;
  }
  if (tid >= 64 && tid < 64 + r) {
    const int j = tid - 64;
    float g, beta;
    if (p.g_opt) {
      g = gin_a;
      beta = gin_b;
    } else {
      gate_pair(gin_a, gin_b, gin_al, gin_dt, g, beta);
    }
    gsh[j] = expf(g);
    bsh[j] = beta;
  }

  for (int h0 = 0; h0 < r; h0 += HPP) {
    const int j = h0 + hl;        // value head inside the group
    const int h = kh * r + j;
    char* sb = head_state(h);
    if (h0 > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Sv[i] = SQ::ld(sb, toff + i * SD);
    }

    // p = S^T k^ (undecayed)
    float pk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float kv = yv[SD + rg * 16 + i] * rk;
      const f32x4 sv = SQ::f32(Sv[i]);
      pk[0] = fmaf(sv[0], kv, pk[0]);
      pk[1] = fmaf(sv[1], kv, pk[1]);
      pk[2] = fmaf(sv[2], kv, pk[2]);
      pk[3] = fmaf(sv[3], kv, pk[3]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) pk[c] += __shfl_xor(pk[c], 32, 64);
    if (!hi_half) {
#pragma unroll
      for (int c = 0; c < 4; ++c) red1[(hl * 4 + wv) * SD + cg * 4 + c] = pk[c];
    }
    lds_barrier();
    if constexpr (SBF) {
      // keep the bf16 state packed across the exchange: without this the compiler keeps
      // the values unpacked for the first product alive for the update (64 more registers)
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(Sv[i]));
    }
    float u[4];
    const float eg = gsh[j], beta = bsh[j];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float tot = 0.f;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) tot += red1[(hl * 4 + w4) * SD + cg * 4 + c];
      const float vj = yv[2 * SD + j * SD + cg * 4 + c];
      u[c] = beta * (vj - eg * tot);
    }
    // S <- e^g S + k^ u^T, and the output partials S^T q^
    float po[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float kv = yv[SD + rg * 16 + i] * rk;
      const float qv = yv[rg * 16 + i] * rq;
      f32x4 sv = SQ::f32(Sv[i]);
      sv[0] = fmaf(eg, sv[0], kv * u[0]);
      sv[1] = fmaf(eg, sv[1], kv * u[1]);
      sv[2] = fmaf(eg, sv[2], kv * u[2]);
      sv[3] = fmaf(eg, sv[3], kv * u[3]);
      po[0] = fmaf(sv[0], qv, po[0]);     // o from the updated state before any rounding
      po[1] = fmaf(sv[1], qv, po[1]);
      po[2] = fmaf(sv[2], qv, po[2]);
      po[3] = fmaf(sv[3], qv, po[3]);
      SQ::st(sb, toff + i * SD, sv);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) po[c] += __shfl_xor(po[c], 32, 64);
    if (!hi_half) {
#pragma unroll
      for (int c = 0; c < 4; ++c) red2[(hl * 4 + wv) * SD + cg * 4 + c] = po[c];
    }
    lds_barrier();
    if (t256 < 32) {
      float ov[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float tot = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) tot += red2[(hl * 4 + w4) * SD + cg * 4 + c];
        ov[c] = io::round(p.scale * tot);      // o as stored
      }
      const int64_t ob = ((int64_t)bseq * Hv + h) * SD + cg * 4;
      if (p.o) {
#pragma unroll
        for (int c = 0; c < 4; ++c) io::st((T*)p.o + ob, c, ov[c]);
      }
      if constexpr (NORM) {
        // z-gated RMSNorm of the head's row: lanes 0 .. 31 hold its 128 values
        float ss = ov[0] * ov[0];
        ss = fmaf(ov[1], ov[1], ss);
        ss = fmaf(ov[2], ov[2], ss);
        ss = fmaf(ov[3], ov[3], ss);
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float inv = 1.0f / sqrtf(ss * (1.0f / SD) + p.eps);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          io::st((T*)p.y + ob, c, wsh[cg * 4 + c] * (ov[c] * inv) * silu(zsh[j * SD + cg * 4 + c]));
      }
    }
    lds_barrier();  // red1/red2 are reused by the next pass
  }
}

template <int IO, int HPP, bool SBF>
static hipError_t step_launch(const StepArgs& a, hipStream_t s) {
  const int r = a.Hv / a.Hk;
  const bool norm = a.y != nullptr;
  const size_t lds = sizeof(float) * (256 + r * SD + 2 * HPP * 4 * SD + 2 * r + 2 +
                                      (norm ? r * SD + SD : 0));
  const dim3 grid((unsigned)(a.B * a.Hk)), block(256 * HPP);
  if (norm)   // (the fused norm takes no slots)
    hipLaunchKernelGGL((recurrent_step_kernel<IO, HPP, SBF, false, true>), grid, block, lds, s, a);
  else if (a.slots)
    hipLaunchKernelGGL((recurrent_step_kernel<IO, HPP, SBF, true, false>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((recurrent_step_kernel<IO, HPP, SBF, false, false>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int IO>
static hipError_t step_impl(const StepArgs& a, hipStream_t s) {
  const int r = a.Hv / a.Hk;
  // two heads per pass at most: 512 threads leave 256 VGPRs per lane (no spills)
  if (r % 2 == 0)
    return a.state_bf16 ? step_launch<IO, 2, true>(a, s) : step_launch<IO, 2, false>(a, s);
  return a.state_bf16 ? step_launch<IO, 1, true>(a, s) : step_launch<IO, 1, false>(a, s);
}

hipError_t launch_recurrent_step(const StepArgs& a, int io, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  return io == IO_BF16 ? step_impl<IO_BF16>(a, s) : step_impl<IO_F32>(a, s);
}

}  // namespace gdn
