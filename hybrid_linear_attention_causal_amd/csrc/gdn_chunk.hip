// Chunked (WY/UT) gated delta rule for prefill over packed sequences, gfx950.
//
// Operation: the gated delta rule of the Qwen3.5 linear-attention layer
// (KerasFormers Qwen page, "Architecture notes": conv1d + delta rule) in its
// chunked form, which the KerasFormers Qwen page ("Verified parity") states to
// be algebraically identical to the token-by-token recurrence; prefill runs
// this chunked core (HF Qwen3.5 docs page, "Usage tips").
//
// Chunk algebra (64 tokens, in-chunk cumulative log decay gamma_i, start state S):
//   A_ij = beta_i e^{gamma_i - gamma_j} (k^_i . k^_j)  (j < i),  T = (I + A)^{-1}
//   R    = V - diag(e^{gamma} / |k|) (K S)        (raw K; 1/|k| folds the L2 norm)
//   U    = T diag(beta) R                          (= the WY/UT pseudo-values)
//   O    = scale (diag(e^{gamma} / |q|) (Q S) + P U),
//          P_ij = e^{gamma_i - gamma_j} (q^_i . k^_j) (j <= i)
//   S'   = e^{gamma_L} S + K^T diag(e^{gamma_L - gamma} / |k|) U
//
// Work split: one 256-thread workgroup per (sequence, value head, 64-column
// block of dv).  Each of its 4 waves keeps a 128 x 16 slice of the fp32 state
// in registers for the whole sequence (MFMA accumulator layout) and walks the
// chunks in order.  Per chunk the workgroup stages raw K and Q rows (bf16, or
// bf16 hi/lo planes for fp32 io) in LDS, forms K K^T and Q K^T on MFMA,
// inverts I + A with a blocked fp32 forward substitution, and then each wave
// runs its column slice of the S-dependent products on MFMA.
//
// MFMA use: v_mfma_f32_16x16x32_bf16.  Operand fragments use a permuted
// contraction index (lane group g, element e -> k = 4g + e for e < 4, 16 + 4g
// + e - 4 otherwise), the same for A and B, so the accumulator of one product
// (lane group g holds rows 4g .. 4g+3) is the B operand of the next without
// any data movement.
//
// Precision (from an emulation of this exact scheme against the fp64
// recurrence): raw bf16 K/Q/V enter MFMA exactly; every fp32 operand that
// feeds the state or the output (S in K S and Q S, R and T in T R, P and U in
// P U, U in the state update) is split into bf16 hi + lo, giving ~1e-5 of
// the output RMS.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int CH = 64;                 // chunk length
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVB = 64;                // dv columns per workgroup
constexpr int NBLK = DV / DVB;
constexpr int NTHR = 256;
constexpr int KS_STRIDE = DK + 8;      // u16 per staged K/Q row
constexpr int T_STRIDE = CH + 8;       // u16 per T'/P row
constexpr int F_STRIDE = CH + 4;       // floats per A/T row

template <int IO>
struct ChunkSmem {
  static constexpr int NLO = (IO == IO_F32) ? 1 : 0;
  u16 kh[CH * KS_STRIDE];
  u16 kl[NLO ? CH * KS_STRIDE : 2];
  u16 qh[CH * KS_STRIDE];
  u16 ql[NLO ? CH * KS_STRIDE : 2];
  u16 th[CH * T_STRIDE];
  u16 tl[CH * T_STRIDE];
  u16 ph[CH * T_STRIDE];
  u16 pl[CH * T_STRIDE];
  float af[CH * F_STRIDE];
  float tf[CH * F_STRIDE];
  float msc[4][16 * 20];
  float gam[CH];
  float beta[CH];
  float rnk[CH];
  float rnq[CH];
};

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(uint2 lo, uint2 hi) {
  const uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(bf16x8, v);
}

// A-operand (or B-operand of a transposed matrix) from a row-major u16 tile:
// lane (g, r) gets M[row0 + r][k0 + perm(g, e)].
__device__ __forceinline__ bf16x8 frag_rows(const u16* m, int stride, int row0, int k0, int lane) {
  const u16* p = m + (row0 + (lane & 15)) * stride + k0 + 4 * (lane >> 4);
  return pack8(*reinterpret_cast<const uint2*>(p), *reinterpret_cast<const uint2*>(p + 16));
}

// A-operand of M^T from a row-major u16 tile: lane (g, r) gets M[k0 + perm(g, e)][col0 + r].
__device__ __forceinline__ bf16x8 frag_cols(const u16* m, int stride, int k0, int col0, int lane) {
  const int g = lane >> 4;
  const u16* p = m + (k0 + 4 * g) * stride + col0 + (lane & 15);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u16* q = p + j * 16 * stride;
    w[2 * j] = (uint32_t)q[0] | ((uint32_t)q[stride] << 16);
    w[2 * j + 1] = (uint32_t)q[2 * stride] | ((uint32_t)q[3 * stride] << 16);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// B-operand from two stacked accumulator tiles (rows 0..15 and 16..31 of a
// 32-row slab), split into bf16 hi and lo parts.
__device__ __forceinline__ void frag_acc_split(f32x4 top, f32x4 bot, bf16x8& hi, bf16x8& lo) {
  u16 h[8], l[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f2bf(top[e]);
    l[e] = f2bf(top[e] - bf2f(h[e]));
    h[e + 4] = f2bf(bot[e]);
    l[e + 4] = f2bf(bot[e] - bf2f(h[e + 4]));
  }
  uint4 vh, vl;
  vh.x = h[0] | ((uint32_t)h[1] << 16); vh.y = h[2] | ((uint32_t)h[3] << 16);
  vh.z = h[4] | ((uint32_t)h[5] << 16); vh.w = h[6] | ((uint32_t)h[7] << 16);
  vl.x = l[0] | ((uint32_t)l[1] << 16); vl.y = l[2] | ((uint32_t)l[3] << 16);
  vl.z = l[4] | ((uint32_t)l[5] << 16); vl.w = l[6] | ((uint32_t)l[7] << 16);
  hi = __builtin_bit_cast(bf16x8, vh);
  lo = __builtin_bit_cast(bf16x8, vl);
}

// lower-triangle tile list of a 4 x 4 grid of 16 x 16 tiles
__device__ __forceinline__ void tri_tile(int n, int& I, int& J) {
  I = (n >= 6) ? 3 : (n >= 3) ? 2 : (n >= 1) ? 1 : 0;
  J = n - I * (I + 1) / 2;
}
// strictly-upper tile list
__device__ __forceinline__ void up_tile(int n, int& I, int& J) {
  const int Is[6] = {0, 0, 0, 1, 1, 2};
  const int Js[6] = {1, 2, 3, 2, 3, 3};
  I = Is[n];
  J = Js[n];
}

template <int IO>
__global__ void __launch_bounds__(NTHR)
chunk_prefill_kernel(ChunkArgs p) {
  typedef Io<IO> io;
  typedef typename io::T T;
  constexpr bool F32 = (IO == IO_F32);
  __shared__ ChunkSmem<IO> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  int bid = blockIdx.x;
  const int blk = bid % NBLK;
  bid /= NBLK;
  const int Hv = p.Hv;
  const int h = bid % Hv;
  const int s = bid / Hv;
  const int kh = h / (Hv / p.Hk);
  // sequence bounds, clamped to [0, N] so inconsistent offsets cannot index outside q/k/v/o
  const int64_t b1 = p.cu ? min((int64_t)p.cu[s + 1], p.N) : p.N;
  const int64_t b0 = p.cu ? max((int64_t)0, min((int64_t)p.cu[s], b1)) : 0;
  const int col = blk * DVB + wave * 16 + c16;      // this lane's dv column

  const T* qg = (const T*)p.q + (int64_t)kh * DK;
  const T* kg = (const T*)p.k + (int64_t)kh * DK;
  const T* vg = (const T*)p.v + (int64_t)h * DV + col;
  T* og = (T*)p.o + (int64_t)h * DV + col;
  const int64_t o_stride = (int64_t)Hv * DV;

  // ---- recurrent state slice: S[i] holds rows 16 i + 4 g4 + e of column col
  f32x4 S[8];
  {
    const float* sp = p.state_in ? p.state_in + ((int64_t)s * Hv + h) * DK * DV + col : nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[i][e] = sp ? sp[(16 * i + 4 * g4 + e) * DV] : 0.f;
  }

  float A_log = 0.f, dt_bias = 0.f;
  if (!p.g_opt) {
    A_log = p.A_log[h];
    dt_bias = p.dt_bias[h];
  }

  for (int64_t t0 = b0; t0 < b1; t0 += CH) {
    const int L = (b1 - t0) < CH ? (int)(b1 - t0) : CH;

    // ---------------- (1) loads: V slice into registers, K/Q rows into LDS, gates
    float vr[4][4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g4 + e;
        vr[I][e] = (t < L) ? io::ld(vg, (t0 + t) * p.stride_v) : 0.f;
      }

    if constexpr (!F32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 4) + 16 * j;
        const int c8 = tid & 15;
        uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
        if (row < L) {
          kv = *reinterpret_cast<const uint4*>(kg + (t0 + row) * p.stride_k + c8 * 8);
          qv = *reinterpret_cast<const uint4*>(qg + (t0 + row) * p.stride_q + c8 * 8);
        }
        *reinterpret_cast<uint4*>(&sm.kh[row * KS_STRIDE + c8 * 8]) = kv;
        *reinterpret_cast<uint4*>(&sm.qh[row * KS_STRIDE + c8 * 8]) = qv;
        float sk = 0.f, sq = 0.f;
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float k0 = __uint_as_float(kw[u] << 16), k1 = __uint_as_float(kw[u] & 0xFFFF0000u);
          const float q0 = __uint_as_float(qw[u] << 16), q1 = __uint_as_float(qw[u] & 0xFFFF0000u);
          sk = fmaf(k0, k0, fmaf(k1, k1, sk));
          sq = fmaf(q0, q0, fmaf(q1, q1, sq));
        }
        sk = group_sum<16>(sk);
        sq = group_sum<16>(sq);
        if (c8 == 0) {
          sm.rnk[row] = p.use_l2 ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
          sm.rnq[row] = p.use_l2 ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = (tid >> 5) + 8 * j;
        const int c4 = tid & 31;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
        if (row < L) {
          kv = *reinterpret_cast<const float4*>((const float*)kg + (t0 + row) * p.stride_k + c4 * 4);
          qv = *reinterpret_cast<const float4*>((const float*)qg + (t0 + row) * p.stride_q + c4 * 4);
        }
        const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
        const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
        u16 khi[4], klo[4], qhi[4], qlo[4];
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          khi[u] = f2bf(kk[u]);
          klo[u] = f2bf(kk[u] - bf2f(khi[u]));
          qhi[u] = f2bf(qq[u]);
          qlo[u] = f2bf(qq[u] - bf2f(qhi[u]));
          sk = fmaf(kk[u], kk[u], sk);
          sq = fmaf(qq[u], qq[u], sq);
        }
        const int off = row * KS_STRIDE + c4 * 4;
        *reinterpret_cast<uint2*>(&sm.kh[off]) =
            make_uint2(khi[0] | ((uint32_t)khi[1] << 16), khi[2] | ((uint32_t)khi[3] << 16));
        *reinterpret_cast<uint2*>(&sm.kl[off]) =
            make_uint2(klo[0] | ((uint32_t)klo[1] << 16), klo[2] | ((uint32_t)klo[3] << 16));
        *reinterpret_cast<uint2*>(&sm.qh[off]) =
            make_uint2(qhi[0] | ((uint32_t)qhi[1] << 16), qhi[2] | ((uint32_t)qhi[3] << 16));
        *reinterpret_cast<uint2*>(&sm.ql[off]) =
            make_uint2(qlo[0] | ((uint32_t)qlo[1] << 16), qlo[2] | ((uint32_t)qlo[3] << 16));
        sk = group_sum<32>(sk);
        sq = group_sum<32>(sq);
        if (c4 == 0) {
          sm.rnk[row] = p.use_l2 ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
          sm.rnq[row] = p.use_l2 ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
        }
      }
    }

    if (wave == 0) {
      const int t = lane;
      float g = 0.f, beta = 0.f;
      if (t < L) {
        const int64_t idx = (t0 + t) * Hv + h;
        if (p.g_opt) {
          g = p.g_opt[idx];
          beta = p.beta_opt[idx];
        } else {
          gate_pair(io::ld((const T*)p.a, idx), io::ld((const T*)p.b, idx), A_log, dt_bias, g,
                    beta);
        }
      }
      // inclusive prefix sum of g over the chunk (padding tokens add 0)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_up(g, off, 64);
        if (lane >= off) g += up;
      }
      sm.gam[t] = g;
      sm.beta[t] = beta;
    }
    __syncthreads();

    // ---------------- (2) Gram tiles: A (strictly lower, fp32) and P (lower, hi/lo)
    for (int n = wave; n < 26; n += 4) {
      int I, J;
      if (n < 20) {
        tri_tile(n < 10 ? n : n - 10, I, J);
        const bool isK = n < 10;
        const u16* ah = isK ? sm.kh : sm.qh;
        const u16* al = isK ? sm.kl : sm.ql;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 a = frag_rows(ah, KS_STRIDE, 16 * I, 32 * m, lane);
          const bf16x8 b = frag_rows(sm.kh, KS_STRIDE, 16 * J, 32 * m, lane);
          acc = mma(a, b, acc);
          if constexpr (F32) {
            acc = mma(frag_rows(al, KS_STRIDE, 16 * I, 32 * m, lane), b, acc);
            acc = mma(a, frag_rows(sm.kl, KS_STRIDE, 16 * J, 32 * m, lane), acc);
          }
        }
        const int j = 16 * J + c16;
        const float gj = sm.gam[j], rkj = sm.rnk[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * I + 4 * g4 + e;
          if (isK) {
            float v = 0.f;
            if (i > j) v = sm.beta[i] * expf(sm.gam[i] - gj) * sm.rnk[i] * rkj * acc[e];
            sm.af[i * F_STRIDE + j] = v;
          } else {
            float v = 0.f;
            if (i >= j) v = expf(sm.gam[i] - gj) * sm.rnq[i] * rkj * acc[e];
            const u16 hv = f2bf(v);
            sm.ph[i * T_STRIDE + j] = hv;
            sm.pl[i * T_STRIDE + j] = f2bf(v - bf2f(hv));
          }
        }
      } else {
        up_tile(n - 20, I, J);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * I + 4 * g4 + e, j = 16 * J + c16;
          sm.ph[i * T_STRIDE + j] = 0;
          sm.pl[i * T_STRIDE + j] = 0;
        }
      }
    }
    __syncthreads();

    // ---------------- (3) T = (I + A)^{-1}: 16 x 16 diagonal blocks by forward
    // substitution (one column per lane), then off-diagonal blocks by levels:
    //   T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ
    if (g4 == 0) {
      const int b = wave;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sacc = (i == c16) ? 1.f : 0.f;
        const float* arow = &sm.af[(16 * b + i) * F_STRIDE + 16 * b];
#pragma unroll
        for (int j = 0; j < i; ++j) sacc = fmaf(-arow[j], x[j], sacc);
        x[i] = sacc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.tf[(16 * b + i) * F_STRIDE + 16 * b + c16] = x[i];
    }
    __syncthreads();
    {
      const int ri = lane >> 2;          // row inside the 16 x 16 block
      const int cj = 4 * (lane & 3);     // 4 columns
      float* msc = sm.msc[wave];
#pragma unroll
      for (int lev = 1; lev <= 3; ++lev) {
        const bool active = wave < 4 - lev;
        const int J = wave, I = wave + lev;
        if (active) {
          float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int K = J; K < I; ++K) {
            const float* arow = &sm.af[(16 * I + ri) * F_STRIDE + 16 * K];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              const float av = arow[k];
              const float4 tv = *reinterpret_cast<const float4*>(&sm.tf[(16 * K + k) * F_STRIDE + 16 * J + cj]);
              m4.x = fmaf(av, tv.x, m4.x);
              m4.y = fmaf(av, tv.y, m4.y);
              m4.z = fmaf(av, tv.z, m4.z);
              m4.w = fmaf(av, tv.w, m4.w);
            }
          }
          *reinterpret_cast<float4*>(&msc[ri * 20 + cj]) = m4;
        }
        __syncthreads();
        if (active) {
          float4 t4 = make_float4(0.f, 0.f, 0.f, 0.f);
          const float* trow = &sm.tf[(16 * I + ri) * F_STRIDE + 16 * I];
#pragma unroll
          for (int k = 0; k <= 15; ++k) {
            const float tv = trow[k];
            const float4 mv = *reinterpret_cast<const float4*>(&msc[k * 20 + cj]);
            t4.x = fmaf(-tv, mv.x, t4.x);
            t4.y = fmaf(-tv, mv.y, t4.y);
            t4.z = fmaf(-tv, mv.z, t4.z);
            t4.w = fmaf(-tv, mv.w, t4.w);
          }
          *reinterpret_cast<float4*>(&sm.tf[(16 * I + ri) * F_STRIDE + 16 * J + cj]) = t4;
        }
        __syncthreads();
      }
    }
    // T' = T diag(beta), lower triangle, split into bf16 hi/lo planes
    for (int idx = tid; idx < CH * CH; idx += NTHR) {
      const int i = idx >> 6, j = idx & 63;
      const float v = (j <= i) ? sm.tf[i * F_STRIDE + j] * sm.beta[j] : 0.f;
      const u16 hv = f2bf(v);
      sm.th[i * T_STRIDE + j] = hv;
      sm.tl[i * T_STRIDE + j] = f2bf(v - bf2f(hv));
    }
    __syncthreads();

    // ---------------- (4) S-dependent products for this wave's 16 columns
    float eg[4][4], rkt[4][4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g4 + e;
        eg[I][e] = expf(sm.gam[t]);
        rkt[I][e] = sm.rnk[t];
      }

    // K S and Q S with S split hi/lo (S rows are the contraction index)
    f32x4 KS[4], QS[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      KS[I] = f32x4{0.f, 0.f, 0.f, 0.f};
      QS[I] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bf16x8 sh, sl;
      frag_acc_split(S[2 * m], S[2 * m + 1], sh, sl);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const bf16x8 ak = frag_rows(sm.kh, KS_STRIDE, 16 * I, 32 * m, lane);
        const bf16x8 aq = frag_rows(sm.qh, KS_STRIDE, 16 * I, 32 * m, lane);
        KS[I] = mma(ak, sh, KS[I]);
        KS[I] = mma(ak, sl, KS[I]);
        QS[I] = mma(aq, sh, QS[I]);
        QS[I] = mma(aq, sl, QS[I]);
        if constexpr (F32) {
          KS[I] = mma(frag_rows(sm.kl, KS_STRIDE, 16 * I, 32 * m, lane), sh, KS[I]);
          QS[I] = mma(frag_rows(sm.ql, KS_STRIDE, 16 * I, 32 * m, lane), sh, QS[I]);
        }
      }
    }

    // R = V - diag(e^gamma / |k|) K S
    f32x4 R[4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) R[I][e] = vr[I][e] - eg[I][e] * rkt[I][e] * KS[I][e];

    // U = T' R   (T' lower triangular: row tile I needs token slabs 0 .. I/2)
    f32x4 U[4];
    {
      bf16x8 rh[2], rl[2];
      frag_acc_split(R[0], R[1], rh[0], rl[0]);
      frag_acc_split(R[2], R[3], rh[1], rl[1]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        U[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m <= I / 2; ++m) {
          const bf16x8 ah = frag_rows(sm.th, T_STRIDE, 16 * I, 32 * m, lane);
          const bf16x8 al = frag_rows(sm.tl, T_STRIDE, 16 * I, 32 * m, lane);
          U[I] = mma(ah, rh[m], U[I]);
          U[I] = mma(al, rh[m], U[I]);
          U[I] = mma(ah, rl[m], U[I]);
        }
      }
    }

    // O = scale (diag(e^gamma / |q|) Q S + P U)
    {
      bf16x8 uh[2], ul[2];
      frag_acc_split(U[0], U[1], uh[0], ul[0]);
      frag_acc_split(U[2], U[3], uh[1], ul[1]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 PU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m <= I / 2; ++m) {
          const bf16x8 ah = frag_rows(sm.ph, T_STRIDE, 16 * I, 32 * m, lane);
          const bf16x8 al = frag_rows(sm.pl, T_STRIDE, 16 * I, 32 * m, lane);
          PU = mma(ah, uh[m], PU);
          PU = mma(al, uh[m], PU);
          PU = mma(ah, ul[m], PU);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * g4 + e;
          if (t < L) {
            const float ov = p.scale * (eg[I][e] * sm.rnq[t] * QS[I][e] + PU[e]);
            io::st(og, (t0 + t) * o_stride, ov);
          }
        }
      }
    }

    // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma} / |k|) U
    {
      const float gl = sm.gam[CH - 1];
      const float egl = expf(gl);
      f32x4 Us[4];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * g4 + e;
          Us[I][e] = expf(gl - sm.gam[t]) * rkt[I][e] * U[I][e];
        }
      bf16x8 uh[2], ul[2];
      frag_acc_split(Us[0], Us[1], uh[0], ul[0]);
      frag_acc_split(Us[2], Us[3], uh[1], ul[1]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] *= egl;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 ak = frag_cols(sm.kh, KS_STRIDE, 32 * m, 16 * i, lane);
          S[i] = mma(ak, uh[m], S[i]);
          S[i] = mma(ak, ul[m], S[i]);
          if constexpr (F32) S[i] = mma(frag_cols(sm.kl, KS_STRIDE, 32 * m, 16 * i, lane), uh[m], S[i]);
        }
      }
    }
    __syncthreads();  // the next chunk overwrites the LDS tiles
  }

  if (p.state_out) {
    float* sp = p.state_out + ((int64_t)s * Hv + h) * DK * DV + col;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[(16 * i + 4 * g4 + e) * DV] = S[i][e];
  }
}

template <int IO>
static hipError_t chunk_impl(const ChunkArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.Ns * a.Hv * NBLK;
  hipLaunchKernelGGL(chunk_prefill_kernel<IO>, dim3((unsigned)blocks), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chunk_prefill(const ChunkArgs& a, int io, hipStream_t s) {
  return io == IO_BF16 ? chunk_impl<IO_BF16>(a, s) : chunk_impl<IO_F32>(a, s);
}

}  // namespace gdn
