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
//   U    = T diag(beta) R                          (the WY/UT pseudo-values)
//   O    = scale (diag(e^{gamma} / |q|) (Q S) + P U),
//          P_ij = e^{gamma_i - gamma_j} (q^_i . k^_j) (j <= i)
//   S'   = e^{gamma_L} S + K^T diag(e^{gamma_L - gamma} / |k|) U
//
// Three launches:
//   1. chunk map: chunk offsets of the packed sequences and a per-chunk table
//      (sequence, valid rows, first token); one small workgroup.
//   2. chunk prep: one workgroup per (chunk, key head), all in parallel.  Stages
//      raw K and Q rows in LDS, forms K K^T and Q K^T on MFMA once for the value
//      heads sharing the key head, then per value head inverts I + A (blocked:
//      fp32 forward substitution on the diagonal blocks, fp32 MFMA products off
//      it) and writes T' = T diag(beta) as bf16 hi/lo parts (MFMA A-operand
//      fragments for bf16 io, row-major planes for fp32 io), P where the sweep
//      reads it, and the per-token factors to the workspace.
//   3. sweep: one workgroup per (sequence, value head, block of dv columns; 4 or 8
//      waves of 16 columns).  Each wave keeps a 128 x 16 slice of the fp32 state in
//      registers for the whole sequence and walks the chunks in order; per chunk
//      the S-dependent products (K S, T' R, Q S + P U, K^T U) and the chunk's P
//      (from the Q and K rows it stages) run on operands staged in LDS by DMA
//      while the other phase's products run.  With few chains (bf16, B = 1) the
//      sweep instead spreads each chain over more compute units: the row-split
//      sweep (16 columns per workgroup, its rows over four chain waves) while those
//      workgroups fit the chip at once, else the column-chain sweep (two 16-column
//      tiles per workgroup, one chain wave each).
//
// MFMA use: v_mfma_f32_16x16x32_bf16.  Operand fragments use a permuted
// contraction index (lane group g, element e -> k = 4g + e for e < 4, 16 + 4g
// + e - 4 otherwise), the same for A and B, so the accumulator of one product
// (lane group g holds rows 4g .. 4g+3) is the B operand of the next without
// any data movement.
//
// Precision (from an emulation of this exact scheme against the fp64
// recurrence): raw bf16 K/Q/V enter MFMA exactly (fp32 io: split into bf16 hi
// + lo); every fp32 operand that feeds the state or the output (S in K S and
// Q S, R and T' in T' R, P and U in P U, U in the state update) is split into
// bf16 hi + lo, which leaves ~1e-5 of the output RMS.
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int CH = 64;                 // chunk length
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NTHR = 256;              // prep workgroup
constexpr int KS_STRIDE = DK + 8;      // u16 per staged K/Q row
constexpr int T_STRIDE = CH + 8;       // u16 per staged T'/P row
constexpr int F_STRIDE = CH + 4;       // floats per A/T row

// Workspace (all LDS-ready, so the sweep stages operands with plain DMA copies):
//   chunk offsets: int32 [Ns + 1], padded to 256 bytes; chunk table: int4 [cmax]
//     {sequence, valid rows, first token lo, hi}, padded to 256 bytes
//     (cmax = ceil(N / 64) + Ns bounds the chunk count);
//   per (global chunk c, value head h): T' hi, T' lo as row-major 64 x 72 (padded) bf16
//     planes, then 8 x 64 fp32 per-token rows e^gamma/|k|, e^gamma/|q|,
//     e^{gamma_L - gamma}/|k|, e^{gamma_L}, gamma, 1/|k|, 1/|q| (and one of padding),
//     then, for the 4-wave sweep, P hi, P lo planes (38912 bytes; 20480 without P:
//     the fp32 8-wave sweep forms P from the Q and K rows it stages anyway); bf16 io
//     writes fragment-native records instead (below: with P for the row-split,
//     column-chain and 4-wave sweeps and the transition launches, T' only for the 8-wave
//     sweep);
//   fp32 io only, per (global chunk c, key head kh): K hi, K lo, Q hi, Q lo rows
//     (64 x 136 bf16 each); bf16 io stages K and Q straight from the input rows.
constexpr int64_t WS_PL_BYTES = (int64_t)CH * T_STRIDE * 2;          // 9216 per plane
constexpr int64_t WS_FAC_OFF = 2 * WS_PL_BYTES;                       // 18432
constexpr int FAC_ROWS = 8;    // factor rows of 64 fp32 (row 7 is padding)
constexpr int64_t WS_P_OFF = WS_FAC_OFF + FAC_ROWS * CH * 4;          // 20480
__host__ __device__ constexpr int64_t ws_rec_bytes(bool with_p) {
  return WS_P_OFF + (with_p ? 2 * WS_PL_BYTES : 0);                   // 38912 / 20480
}
constexpr int64_t WS_ROWS_BYTES = (int64_t)CH * KS_STRIDE * 2;       // 17408 per row plane

// Fragment-native records of the row-split sweep (bf16 io), per (global chunk, value
// head), FR_REC_BYTES: T' fragments [row tile j 4][token slab m 2][plane hi, lo 2] (the A
// operand of T' R; each fragment 1 KB, lane l's 16 bytes at 16 l), P fragments in the same
// order, then the 8 x 64 fp32 factor rows.  The fragments of token slab 1 for row tiles 0
// and 1 are zero; they are neither written nor read.
constexpr int64_t FR_T_OFF = 0;
constexpr int64_t FR_P_OFF = 16 * 1024;
constexpr int64_t FR_FAC_OFF = 32 * 1024;
constexpr int64_t FR_REC_BYTES = FR_FAC_OFF + FAC_ROWS * CH * 4;     // 34816
__host__ __device__ constexpr int fr_tp(int j, int m, int plane) { return ((j * 2 + m) * 2 + plane) * 1024; }
// Fragment-native records without P (the 8-wave sweep of bf16 io, which forms P itself):
// the T' fragments as above, then the factor rows
constexpr int64_t FRT_FAC_OFF = 16 * 1024;
constexpr int64_t FRT_REC_BYTES = FRT_FAC_OFF + FAC_ROWS * CH * 4;   // 18432
// u16 offset of element (i, j) of a 64 x 64 operand held as A-operand fragments in LDS
// (fragment (i / 16, j / 32, plane) of 512 u16 at the fr_tp place; lane (g, r) holds row
// r and the permuted contraction index 4 g + e, e < 4, and 16 + 4 g + e - 4, e >= 4)
__device__ __forceinline__ int frag_off(int i, int j, int plane) {
  const int kk = j & 31;
  const int lane = ((kk & 15) >> 2) * 16 + (i & 15);
  const int e = (kk & 3) + ((kk >> 4) << 2);
  return (((i >> 4) * 2 + (j >> 5)) * 2 + plane) * 512 + lane * 8 + e;
}

static int64_t ws_max_chunks(int64_t N, int Ns) { return (N + CH - 1) / CH + Ns; }
static int64_t ws_cmap_bytes(int Ns) { return (((int64_t)Ns + 1) * 4 + 255) / 256 * 256; }
static int64_t ws_map_bytes(int64_t N, int Ns) {
  return ws_cmap_bytes(Ns) + (ws_max_chunks(N, Ns) * 16 + 255) / 256 * 256;
}
__host__ __device__ constexpr int64_t ws_krec_bytes(bool f32) {
  return f32 ? 4 * WS_ROWS_BYTES : 0;
}

// Intra-sequence scan: at most SEG_MAX segments per sequence, each of at least
// SEG_MIN_CHUNKS chunks on average, for at most SEG_MAX_CHAINS (sequence, head) chains;
// the workspace reserves (SEG_MAX - 1) (A, B) pairs per chain when the scan may run.
// fp32 io: whenever the chain count allows.  bf16 io: only for at most SEG_BF16_MAX_CHAINS
// chains averaging at least SEG_BF16_MIN_CHUNKS chunks, where the row-split sweep would
// leave most compute units idle for a long walk.  A transition pass costs as much as a
// normal one over the same chunks, so the scan pays only there (measured on MI355X, B = 1,
// bf16: 1 to 16 chains at 32768 tokens 16-22% faster than the row-split sweep, 5-11% at
// 16384, 10-45% slower at 8192 and below, and 30% slower with 32 chains, which the
// row-split sweep spreads over every compute unit).
constexpr int SEG_MAX = 8;
constexpr int SEG_MIN_CHUNKS = 4;
constexpr int64_t SEG_MAX_CHAINS = 64;
constexpr int64_t SEG_BF16_MAX_CHAINS = 16;
constexpr int64_t SEG_BF16_MIN_CHUNKS = 256;
constexpr int64_t SEG_PAIR_BYTES = 2LL * DK * DV * 4;   // A then B, fp32

// bf16 io: few, long chains (the shape condition; the launch also needs the compute units)
static bool bf16_seg_shape(int64_t N, int Ns, int Hv) {
  const int64_t chains = (int64_t)Ns * Hv;
  return chains <= SEG_BF16_MAX_CHAINS && Ns > 0 && (N + CH - 1) / CH / Ns >= SEG_BF16_MIN_CHUNKS;
}

static int64_t ws_seg_bytes(int64_t N, int Ns, int Hv, bool f32) {
  const int64_t chains = (int64_t)Ns * Hv;
  const bool may = f32 ? chains <= SEG_MAX_CHAINS : bf16_seg_shape(N, Ns, Hv);
  return may ? (SEG_MAX - 1) * chains * SEG_PAIR_BYTES : 0;
}

// Segments per sequence: enough to fill the compute units with the normal launch's two
// 4-wave workgroups per (chain, segment), at least 3 (two segments take as long as
// one: the transition pass is as long as the normal one), else 1.
static int seg_count(int64_t N, int Ns, int Hv, int64_t cus) {
  const int64_t chains = (int64_t)Ns * Hv;
  if (chains > SEG_MAX_CHAINS || N <= 0) return 1;
  int64_t G = cus / (2 * chains);
  G = min(G, (int64_t)SEG_MAX);
  G = min(G, ((N + CH - 1) / CH) / Ns / SEG_MIN_CHUNKS);
  return G >= 3 ? (int)G : 1;
}

size_t chunk_workspace_bytes(int64_t N, int Ns, int Hk, int Hv, bool f32) {
  const int64_t cmax = ws_max_chunks(N, Ns);
  return (size_t)(ws_map_bytes(N, Ns) + cmax * Hv * ws_rec_bytes(true) + cmax * Hk * ws_krec_bytes(f32) +
                  ws_seg_bytes(N, Ns, Hv, f32));
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 x 16 fp32 tile X Y (X: 16 x K, Y: K x 16, both row-major fp32 in LDS) on the fp32
// MFMA: step s takes lane l's X[l % 16][4 s + l / 16] and Y[4 s + l / 16][l % 16]; the
// result is in accumulator layout (lane l: rows 4 (l / 16) + e, column l % 16).
template <int K>
__device__ __forceinline__ f32x4 tile_mma_f32(const float* x, int sx, const float* y, int sy,
                                              int lane) {
  const int r = lane & 15, g = lane >> 4;
  float xa[K / 4], yb[K / 4];
#pragma unroll
  for (int st = 0; st < K / 4; ++st) {
    xa[st] = x[r * sx + 4 * st + g];
    yb[st] = y[(4 * st + g) * sy + r];
  }
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < K / 4; ++st) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[st], yb[st], c, 0, 0, 0);
  return c;
}

// two fp32 -> packed bf16 pair (hardware round-to-nearest-even)
__device__ __forceinline__ uint32_t cvt2(float a, float b) { return f2bf2(a, b); }
// hi = bf16(x), lo = bf16(x - hi) for a pair of values
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt2(a, b);
  lo = cvt2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ bf16x8 pack8(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// A-operand (or B-operand of a transposed matrix) from a row-major u16 tile:
// lane (g, r) gets M[row0 + r][k0 + perm(g, e)].
__device__ __forceinline__ bf16x8 frag_rows(const u16* m, int stride, int row0, int k0, int lane) {
  const u16* p = m + (row0 + (lane & 15)) * stride + k0 + 4 * (lane >> 4);
  return pack8(*reinterpret_cast<const uint2*>(p), *reinterpret_cast<const uint2*>(p + 16));
}

// A-operand of K^T (rows d0 .. d0+15, tokens k0 + perm(g, e)) read from row-major K rows
// in LDS with two transposing reads.  Within each 16-lane group, ds_read_b64_tr_b16
// hands lane t element e of source lane 4 e + t / 4, at that lane's position t % 4; so
// source lane j of group g points at token k0 + 4 g + j / 4 (16 tokens further for the
// second read), dk columns d0 + 4 (j % 4) .. d0 + 4 (j % 4) + 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x8 frag_kt(const u16* krows, int d0, int k0, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const u16* p = krows + (k0 + 4 * g + (j >> 2)) * KS_STRIDE + d0 + 4 * (j & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * KS_STRIDE));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B-operand from two stacked accumulator tiles (rows 0..15 and 16..31 of a
// 32-row slab), split into bf16 hi and lo parts.
__device__ __forceinline__ void frag_acc_split(f32x4 top, f32x4 bot, bf16x8& hi, bf16x8& lo) {
  uint4 vh, vl;
  split2(top[0], top[1], vh.x, vl.x);
  split2(top[2], top[3], vh.y, vl.y);
  split2(bot[0], bot[1], vh.z, vl.z);
  split2(bot[2], bot[3], vh.w, vl.w);
  hi = __builtin_bit_cast(bf16x8, vh);
  lo = __builtin_bit_cast(bf16x8, vl);
}

// Y = M X for a lower-triangular 64 x 64 M (bf16 hi | lo planes, rows of T_STRIDE, in
// LDS) and a 64 x 16 X given as B-operand fragments (hi, lo) of its two 32-row slabs:
// three passes (Mh Xh, Ml Xh, Mh Xl).  Row tile I needs slabs 0 .. I / 2.  The products
// run slab by slab and pass by pass over the row tiles, so that each accumulator's next
// product is four (slab 0) or two (slab 1) products away; mid() runs between the slabs.
template <typename F>
__device__ __forceinline__ void tri_apply(const u16* mp, const bf16x8 (&xh)[2], const bf16x8 (&xl)[2],
                                          f32x4 (&y)[4], int lane, F mid) {
  const u16* mh = mp;
  const u16* ml = mp + CH * T_STRIDE;
  bf16x8 ah[4], al[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    ah[I] = frag_rows(mh, T_STRIDE, 16 * I, 0, lane);
    al[I] = frag_rows(ml, T_STRIDE, 16 * I, 0, lane);
  }
#pragma unroll
  for (int I = 0; I < 4; ++I) y[I] = mma(ah[I], xh[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int I = 0; I < 4; ++I) y[I] = mma(al[I], xh[0], y[I]);
#pragma unroll
  for (int I = 0; I < 4; ++I) y[I] = mma(ah[I], xl[0], y[I]);
  mid();
  bf16x8 bh[2], bl[2];
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    bh[I] = frag_rows(mh, T_STRIDE, 16 * (I + 2), 32, lane);
    bl[I] = frag_rows(ml, T_STRIDE, 16 * (I + 2), 32, lane);
  }
#pragma unroll
  for (int I = 0; I < 2; ++I) y[I + 2] = mma(bh[I], xh[1], y[I + 2]);
#pragma unroll
  for (int I = 0; I < 2; ++I) y[I + 2] = mma(bl[I], xh[1], y[I + 2]);
#pragma unroll
  for (int I = 0; I < 2; ++I) y[I + 2] = mma(bh[I], xl[1], y[I + 2]);
}
__device__ __forceinline__ void tri_apply(const u16* mp, const bf16x8 (&xh)[2], const bf16x8 (&xl)[2],
                                          f32x4 (&y)[4], int lane) {
  tri_apply(mp, xh, xl, y, lane, []() {});
}

// tri_apply for M held as A-operand fragments in LDS (fr_tp order, 512 u16 each): one
// 16-byte lane-linear read per fragment
template <typename F>
__device__ __forceinline__ void tri_apply_frag(const u16* mp, const bf16x8 (&xh)[2], const bf16x8 (&xl)[2],
                                               f32x4 (&y)[4], int lane, F mid) {
  auto fr = [&](int I, int m, int pl) {
    return *reinterpret_cast<const bf16x8*>(mp + fr_tp(I, m, pl) / 2 + lane * 8);
  };
  bf16x8 ah[4], al[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    ah[I] = fr(I, 0, 0);
    al[I] = fr(I, 0, 1);
  }
#pragma unroll
  for (int I = 0; I < 4; ++I) y[I] = mma(ah[I], xh[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int I = 0; I < 4; ++I) y[I] = mma(al[I], xh[0], y[I]);
#pragma unroll
  for (int I = 0; I < 4; ++I) y[I] = mma(ah[I], xl[0], y[I]);
  mid();
  bf16x8 bh[2], bl[2];
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    bh[I] = fr(I + 2, 1, 0);
    bl[I] = fr(I + 2, 1, 1);
  }
#pragma unroll
  for (int I = 0; I < 2; ++I) y[I + 2] = mma(bh[I], xh[1], y[I + 2]);
#pragma unroll
  for (int I = 0; I < 2; ++I) y[I + 2] = mma(bl[I], xh[1], y[I + 2]);
#pragma unroll
  for (int I = 0; I < 2; ++I) y[I + 2] = mma(bh[I], xl[1], y[I + 2]);
}

// lower-triangle tile list of a 4 x 4 grid of 16 x 16 tiles
__device__ __forceinline__ void tri_tile(int n, int& I, int& J) {
  I = (n >= 6) ? 3 : (n >= 3) ? 2 : (n >= 1) ? 1 : 0;
  J = n - I * (I + 1) / 2;
}

// sequence bounds, clamped to [0, N] so inconsistent offsets cannot index outside
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int64_t N, int s, int64_t& b0,
                                           int64_t& b1) {
  b1 = cu ? min((int64_t)cu[s + 1], N) : N;
  b0 = cu ? max((int64_t)0, min((int64_t)cu[s], b1)) : 0;
}

// Raw K/Q rows of one chunk for one thread: rows 4 rq .. 4 rq + 3, columns
// 8 c8 .. 8 c8 + 7 (c8 = tid & 15 spans one 16-lane DPP row), as 16-byte words.
template <int IO>
struct RowBlock {
  static constexpr int W = (IO == IO_F32) ? 2 : 1;  // uint4 words per 8 values
  uint4 w[4][W];
};

template <int IO>
__device__ __forceinline__ void load_rows(RowBlock<IO>& rb, const typename Io<IO>::T* base,
                                          int64_t stride, int64_t t0, int L, int tid) {
  const int c8 = tid & 15, rq = tid >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 4 * rq + u;
    const int64_t r = t0 + (row < L ? row : L - 1);   // in bounds; masked at use
    const uint4* p = reinterpret_cast<const uint4*>(base + r * stride + c8 * 8);
#pragma unroll
    for (int w = 0; w < RowBlock<IO>::W; ++w) rb.w[u][w] = p[w];
  }
}

// values of row u of a RowBlock as 8 floats (0 for rows past the chunk end)
template <int IO>
__device__ __forceinline__ void row_vals(const RowBlock<IO>& rb, int u, bool ok, float* v) {
  if constexpr (IO == IO_F32) {
    const float4 a = __builtin_bit_cast(float4, rb.w[u][0]);
    const float4 b = __builtin_bit_cast(float4, rb.w[u][1]);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint32_t x[4] = {rb.w[u][0].x, rb.w[u][0].y, rb.w[u][0].z, rb.w[u][0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(x[j] << 16);
      v[2 * j + 1] = __uint_as_float(x[j] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = ok ? v[j] : 0.f;
}

// write 8 values of a staged row as bf16 (hi) and, for fp32 io, the lo residual
template <int IO>
__device__ __forceinline__ void put_row8(u16* hi, u16* lo, int off, const float* v, uint4& hw,
                                         uint4& lw) {
  if constexpr (IO == IO_F32) {
    split2(v[0], v[1], hw.x, lw.x);
    split2(v[2], v[3], hw.y, lw.y);
    split2(v[4], v[5], hw.z, lw.z);
    split2(v[6], v[7], hw.w, lw.w);
    *reinterpret_cast<uint4*>(hi + off) = hw;
    *reinterpret_cast<uint4*>(lo + off) = lw;
  } else {
    // bf16 inputs are exact bf16 values: repack without rounding
    hw.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xFFFF0000u);
    hw.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xFFFF0000u);
    hw.z = (__float_as_uint(v[4]) >> 16) | (__float_as_uint(v[5]) & 0xFFFF0000u);
    hw.w = (__float_as_uint(v[6]) >> 16) | (__float_as_uint(v[7]) & 0xFFFF0000u);
    lw = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(hi + off) = hw;
    (void)lo;
  }
}

// ============================================================================ 1. chunk map
// cmap[s] = number of 64-token chunks before sequence s, cmap[Ns] = total; and for every
// global chunk c < cmax, cinfo[c] = {sequence, valid rows L, first token (lo, hi)},
// L = 0 past the total.  One workgroup; the chunk -> sequence search runs on an LDS copy
// of cmap when it fits.
constexpr int MAP_LDS = 8192;
__global__ void __launch_bounds__(256) chunk_map_kernel(const int32_t* cu, int Ns, int64_t N,
                                                        int64_t cmax, int32_t* cmap,
                                                        int4* cinfo) {
  __shared__ int wtot[4];
  __shared__ int lmap[MAP_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool in_lds = Ns + 1 <= MAP_LDS;
  int carry = 0;
  for (int base = 0; base < Ns; base += 256) {
    const int s = base + tid;
    int n = 0;
    if (s < Ns) {
      int64_t b0, b1;
      seq_bounds(cu, N, s, b0, b1);
      n = (int)((b1 - b0 + CH - 1) / CH);
    }
    // inclusive scan inside the wave (exact in fp32 below 2^24 chunks)
    const float incl = wave_prefix_sum((float)n);
    if (lane == 63) wtot[wave] = (int)incl;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    if (s < Ns) {
      cmap[s] = before + (int)incl - n;
      if (in_lds) lmap[s] = before + (int)incl - n;
    }
    carry += wtot[0] + wtot[1] + wtot[2] + wtot[3];
    __syncthreads();
  }
  if (tid == 0) {
    cmap[Ns] = carry;
    if (in_lds) lmap[Ns] = carry;
  }
  __syncthreads();   // also orders this workgroup's cmap stores before the reads below
  const int* map = in_lds ? lmap : cmap;
  for (int64_t c = tid; c < cmax; c += 256) {
    int4 info = make_int4(0, 0, 0, 0);
    if (c < carry) {
      int lo = 0, hi = Ns - 1;          // the last sequence starting at or before chunk c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (map[mid] <= c) lo = mid; else hi = mid - 1;
      }
      int64_t b0, b1;
      seq_bounds(cu, N, lo, b0, b1);
      const int64_t t0 = b0 + (c - map[lo]) * CH;
      info = make_int4(lo, (int)min((int64_t)CH, b1 - t0), (int)(uint32_t)t0, (int)(t0 >> 32));
    }
    cinfo[c] = info;
  }
}

// ============================================================================ 2. chunk prep
// One workgroup per (global chunk, key head), for the r = Hv / Hk value heads that
// share the key head: the K and Q rows, their norms and the raw Gram tiles
// (K^ K^T and Q^ K^T with the 1/|k|, 1/|q| factors) are formed once; then, per value
// head, its decay and write strength scale the tiles into A and P, I + A is inverted,
// and the head's record is written.
// record layouts the prep kernel writes: rows without P (8-wave sweep) and rows with P
// (4-wave sweep) for fp32 io; for bf16 io fragment-native with P (row-split, column-chain
// and 4-wave sweeps, transition launches) and fragment-native T' without P (8-wave sweep)
enum PrepMode { PREP_ROWS = 0, PREP_ROWS_P = 1, PREP_FRAG = 2, PREP_FRAG_T = 3 };
constexpr int PREP_RB = 4;                // value heads whose gates are staged at once
static_assert(PREP_RB == NTHR / 64, "one wave stages the gates of one value head");

template <int IO>
struct PrepSmem {
  static constexpr bool F32 = (IO == IO_F32);
  // phase 0 holds the K and Q rows; once the Gram tiles are in registers the same
  // bytes hold A and T of the current value head (every member 16-byte aligned)
  struct Rows {
    alignas(16) u16 kh[CH * KS_STRIDE];   // K rows (bf16 / hi part)
    alignas(16) u16 qh[CH * KS_STRIDE];
    alignas(16) u16 kl[F32 ? CH * KS_STRIDE : 8];
    alignas(16) u16 ql[F32 ? CH * KS_STRIDE : 8];
  };
  struct Mats {
    alignas(16) float af[CH * F_STRIDE];  // strictly lower A (fp32); its dead top rows
                                          // serve as scratch of the block products
    alignas(16) float tf[CH * F_STRIDE];  // T (fp32); first holds the staged P planes
  };
  union alignas(16) {
    Rows r;
    Mats m;
  } u;
  alignas(16) float gam[PREP_RB][CH];     // in-chunk cumulative log decay per value head
  alignas(16) float beta[PREP_RB][CH];
  alignas(16) float rnk[CH];              // 1/|k_t| (1 without the L2 norm)
  alignas(16) float rnq[CH];
};

// Fused conv of the prep kernel (bf16 io): the conv window + SiLU of this key head's
// channels over the chunk's rows, rounded to bf16 as the conv call stores them (the
// operation of gdn_conv1d_fwd: llm-arch-viz Qwen3.5-9B page, module tree, conv1d 8192x1x4,
// depthwise, no bias).  The rows go to y, where the sweep reads them; the q and k rows
// also go to LDS for the Gram products, with their row norms.  A lane handles a group of
// 8 channels (q 16 groups, k 16, then 16 per value head) over 8 rows; its window adds the
// 3 rows before them (from x, or before the sequence start from its conv state, or zeros).
// Every global load is unconditional and in bounds (a load under a condition is waited for
// where its branch joins), so a window's rows are waited for one by one as they are used.
// gin (loaded before the call) is marked complete after the first row, whose wait covers
// it (loads complete in order), so no later use of it waits for the y stores.

// the 11 window rows r0 - 3 .. r0 + 7 of channels ch .. ch + 7 (rows at or past the chunk
// end clamped to its last row: they feed only outputs that are not stored); inside:
// the whole window lies inside the sequence
__device__ __forceinline__ void conv_window(const ChunkArgs& p, int s, int64_t sb, int64_t t0,
                                            int L, int r0, int ch, bool inside, uint4 (&raw)[11]) {
  const int Cq = p.Cq;
  const u16* x = (const u16*)p.x;
  const u16* cs = (const u16*)p.conv_state_in;
  if (inside) {
    // one base pointer, row i is i Cq further (no per-row 64-bit offsets to hold)
    const u16* xr = x + (t0 + r0 - 3) * (int64_t)Cq + ch;
#pragma unroll
    for (int i = 0; i < 11; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(xr + (min(r0 - 3 + i, L - 1) - (r0 - 3)) * Cq);
  } else {
    // rows before the sequence come from its conv state, or are zero without one (read
    // from the sequence's first row and cleared)
#pragma unroll
    for (int i = 0; i < 11; ++i) {
      const int64_t tok = t0 + min(r0 - 3 + i, L - 1);
      const bool in_seq = tok >= sb;
      const u16* src = in_seq ? x + tok * Cq + ch
                     : cs    ? cs + ((int64_t)s * 3 + (tok - sb + 3)) * Cq + ch
                             : x + sb * Cq + ch;
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      raw[i] = (in_seq || cs) ? v : make_uint4(0, 0, 0, 0);
    }
  }
}

// output row t (0 .. 7) of a window: 8 channels as packed bf16
__device__ __forceinline__ uint4 conv_row8(const float4 (&wt)[8], const uint4 (&raw)[11], int t) {
  const uint32_t w0[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
  const uint32_t w1[4] = {raw[t + 1].x, raw[t + 1].y, raw[t + 1].z, raw[t + 1].w};
  const uint32_t w2[4] = {raw[t + 2].x, raw[t + 2].y, raw[t + 2].z, raw[t + 2].w};
  const uint32_t w3[4] = {raw[t + 3].x, raw[t + 3].y, raw[t + 3].z, raw[t + 3].w};
  float out[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      auto val = [&](uint32_t wd) { return __uint_as_float(hf ? (wd & 0xFFFF0000u) : (wd << 16)); };
      out[2 * q + hf] = conv4_silu(wt[2 * q + hf], val(w0[q]), val(w1[q]), val(w2[q]), val(w3[q]));
    }
  }
  return make_uint4(f2bf2(out[0], out[1]), f2bf2(out[2], out[3]), f2bf2(out[4], out[5]),
                    f2bf2(out[6], out[7]));
}

// a q (group < 16) or k row of 8 channels to LDS (zero past the chunk end), with the
// squared norm of the row over the 16 lanes of its DPP row
__device__ __forceinline__ void qk_row_to_lds(const ChunkArgs& p, uint4 ow, int row, int L, int cg,
                                              u16* k_rows, u16* q_rows, float* rnk, float* rnq) {
  if (row >= L) ow = make_uint4(0, 0, 0, 0);
  const uint32_t ox[4] = {ow.x, ow.y, ow.z, ow.w};
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float v0 = __uint_as_float(ox[q] << 16), v1 = __uint_as_float(ox[q] & 0xFFFF0000u);
    ss = fmaf(v1, v1, fmaf(v0, v0, ss));
  }
  ss = row16_sum(ss);
  const float rn = p.use_l2 ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.0f;
  if (cg < 16) {
    *reinterpret_cast<uint4*>(q_rows + row * KS_STRIDE + cg * 8) = ow;
    if (cg == 0) rnq[row] = rn;
  } else if (cg < 32) {
    *reinterpret_cast<uint4*>(k_rows + row * KS_STRIDE + (cg - 16) * 8) = ow;
    if (cg == 16) rnk[row] = rn;
  }
}

// channel of group cg of key head kh (q 16 groups, k 16, then 16 per value head)
__device__ __forceinline__ int conv_group_channel(int cg, int kh, int Hk, int r) {
  return cg < 16 ? kh * DK + cg * 8
       : cg < 32 ? Hk * DK + kh * DK + (cg - 16) * 8
                 : 2 * Hk * DK + kh * r * DV + (cg - 32) * 8;
}

// the final conv state of every channel of this key head (the last 3 raw rows of the
// sequence, from x or, for a sequence shorter than 3, from the conv state before it),
// written by wave 0 of the workgroup whose chunk ends the sequence
__device__ __forceinline__ void final_conv_state(const ChunkArgs& p, int s, int64_t sb, int64_t se,
                                                 int kh, int r, int lane) {
  const int Cq = p.Cq, G = 32 + 16 * r;
  const u16* x = (const u16*)p.x;
  const u16* cs = (const u16*)p.conv_state_in;
  u16* cso = (u16*)p.conv_state_out;
  for (int cg = lane; cg < G; cg += 64) {
    const int ch = conv_group_channel(cg, kh, p.Hk, r);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int64_t tok = se - 3 + i;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok >= sb)
        v = *reinterpret_cast<const uint4*>(x + tok * Cq + ch);
      else if (cs)
        v = *reinterpret_cast<const uint4*>(cs + ((int64_t)s * 3 + (tok - sb + 3)) * Cq + ch);
      *reinterpret_cast<uint4*>(cso + ((int64_t)s * 3 + i) * Cq + ch) = v;
    }
  }
}

// one pass over 32 channel groups from group g0: lane l takes group g0 + (l & 31) (lanes
// past the last group repeat it: they compute and store the same bytes) over rows
// 16 w + 8 (l >> 5) .. + 7 of wave w.  The weights are loaded with the window (L1 hits).
// The first row is opaque to the compiler: the rows do not depend on the pass, and their
// 64-bit offsets, hoisted out of the v passes' loop, would stay live across it and spill.
// QK: groups 0 .. 31 (q, then k), whose rows also go to LDS with their norms (each DPP row
// of 16 lanes then holds the 16 groups of one head's q or k for the same rows); gin is
// marked complete after the first row, whose wait covers it (loads complete in order).
template <bool QK>
__device__ __forceinline__ void conv_pass(const ChunkArgs& p, int s, int64_t sb, int64_t t0, int L,
                                          int kh, int r, int wave, int lane, int g0, u16* k_rows,
                                          u16* q_rows, float* rnk, float* rnq, uint4& gin) {
  const int Cq = p.Cq;
  u16* y = (u16*)p.y;
  const int cg = min(g0 + (lane & 31), 32 + 16 * r - 1);
  const int ch = conv_group_channel(cg, kh, p.Hk, r);
  float4 wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wt[j] = *reinterpret_cast<const float4*>(p.conv_w + (int64_t)(ch + j) * 4);
  int r0 = 16 * wave + 8 * (lane >> 5);
  asm volatile("" : "+v"(r0));
  uint4 raw[11];
  conv_window(p, s, sb, t0, L, r0, ch, t0 + r0 - 3 >= sb, raw);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = r0 + t;
    const uint4 ow = conv_row8(wt, raw, t);
    if (QK && t == 0) asm volatile("" : "+v"(gin.x), "+v"(gin.y), "+v"(gin.z), "+v"(gin.w));
    if (row < L) *reinterpret_cast<uint4*>(y + (t0 + row) * Cq + ch) = ow;
    if constexpr (QK) qk_row_to_lds(p, ow, row, L, cg, k_rows, q_rows, rnk, rnq);
  }
}

// the q and k channels of the key head: rows to y, and to LDS for the Gram products
__device__ __forceinline__ void conv_qk(const ChunkArgs& p, int s, int64_t t0, int L, int kh, int r,
                                        int wave, int lane, u16* k_rows, u16* q_rows, float* rnk,
                                        float* rnq, uint4& gin) {
  int64_t sb, se;
  seq_bounds(p.cu, p.N, s, sb, se);
  conv_pass<true>(p, s, sb, t0, L, kh, r, wave, lane, 0, k_rows, q_rows, rnk, rnq, gin);
}

// the v channels of the key head's r value heads (rows to y only, for the sweep), and the
// final conv state of every channel of the key head
__device__ __forceinline__ void conv_v(const ChunkArgs& p, int s, int64_t t0, int L, int kh, int r,
                                       int wave, int lane) {
  int64_t sb, se;
  seq_bounds(p.cu, p.N, s, sb, se);
  uint4 none = make_uint4(0, 0, 0, 0);
#pragma unroll 1
  for (int g0 = 32; g0 < 32 + 16 * r; g0 += 32)
    conv_pass<false>(p, s, sb, t0, L, kh, r, wave, lane, g0, nullptr, nullptr, nullptr, nullptr, none);
  if (p.conv_state_in_prep && wave == 0 && t0 + L == se) final_conv_state(p, s, sb, se, kh, r, lane);
}

// waves per SIMD the prep kernel is built for (its workgroups resident per CU)
constexpr int prep_occupancy(int io, int mode) {
  return io == IO_BF16 ? (mode != PREP_ROWS_P ? 4 : 3) : 2;
}

// fused conv of the prep: none, or every channel of the key head
enum PrepConv { CONV_NONE = 0, CONV_ALL = 1 };
template <int IO, int MODE, int CONV = CONV_NONE>
__global__ void __launch_bounds__(NTHR, prep_occupancy(IO, MODE))
chunk_prep_kernel(ChunkArgs p, const int4* __restrict__ cinfo, uint8_t* __restrict__ recs,
                  uint8_t* __restrict__ krecs) {
  typedef Io<IO> io;
  typedef typename io::T T;
  constexpr bool F32 = (IO == IO_F32);
  constexpr bool WITHP = MODE == PREP_ROWS_P || MODE == PREP_FRAG;
  constexpr bool FRAG = MODE == PREP_FRAG || MODE == PREP_FRAG_T;
  static_assert(!(FRAG && F32), "fragment-native records are for bf16 io");
  static_assert(!(CONV != CONV_NONE && F32), "the fused conv is for bf16 io");
  constexpr int64_t REC = FRAG ? (WITHP ? FR_REC_BYTES : FRT_REC_BYTES) : ws_rec_bytes(WITHP);
  constexpr int64_t FAC_OFF = FRAG ? (WITHP ? FR_FAC_OFF : FRT_FAC_OFF) : WS_FAC_OFF;
  __shared__ PrepSmem<IO> sm;

  const int c = blockIdx.x;               // global chunk
  const int kh_ = blockIdx.y;             // key head
  const int Hv = p.Hv, r = Hv / p.Hk;
  // (one sequence: the chunk map is not built; chunk c is tokens b0 + 64 c .. of it)
  int4 ci;
  if (p.Ns == 1) {
    int64_t sb, se;
    seq_bounds(p.cu, p.N, 0, sb, se);
    const int64_t tc = sb + (int64_t)c * CH;
    ci = make_int4(0, (int)max((int64_t)0, min((int64_t)CH, se - tc)), (int)(uint32_t)tc, (int)(tc >> 32));
  } else {
    ci = cinfo[c];
  }
  const int L = ci.y;
  if (L == 0) return;                     // past the last chunk
  const int64_t t0 = ((int64_t)ci.w << 32) | (uint32_t)ci.z;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, c16 = lane & 15;

  // gate inputs of value head kh_ r + hb + wave for this lane's token: {a or g, b or
  // beta, A_log, dt_bias}, as raw bits (a and b in the io dtype, the rest fp32): widening
  // a loaded value where it is loaded would make the wave wait for it there (returned by
  // value: references into branches would leave the four values in scratch memory)
  auto gate_in = [&](int hb) {
    const int jh = hb + wave;
    uint4 gi = make_uint4(0u, 0u, 0u, 0u);
    if (jh < r) {
      const int h = kh_ * r + jh;
      const int64_t idx = (t0 + (lane < L ? lane : L - 1)) * Hv + h;
      if (p.g_opt) {
        gi.x = __float_as_uint(p.g_opt[idx]);
        gi.y = __float_as_uint(p.beta_opt[idx]);
      } else {
        if constexpr (F32) {
          gi.x = __float_as_uint(((const float*)p.a)[idx]);
          gi.y = __float_as_uint(((const float*)p.b)[idx]);
        } else {
          gi.x = ((const u16*)p.a)[idx];
          gi.y = ((const u16*)p.b)[idx];
        }
        gi.z = __float_as_uint(p.A_log[h]);
        gi.w = __float_as_uint(p.dt_bias[h]);
      }
    }
    return gi;
  };
  // the raw bits as values
  auto gate_vals = [&](uint4 gi) {
    const bool raw_io = !p.g_opt && !F32;   // a and b as bf16 bits
    return make_float4(raw_io ? __uint_as_float(gi.x << 16) : __uint_as_float(gi.x),
                       raw_io ? __uint_as_float(gi.y << 16) : __uint_as_float(gi.y),
                       __uint_as_float(gi.z), __uint_as_float(gi.w));
  };
  // the first batch's gate inputs go out before the rows, so their latency hides there
  uint4 gin0 = gate_in(0);

  // ---- phase 0: K and Q rows to LDS, row norms (16 lanes of a DPP row share a row)
  if constexpr (CONV != CONV_NONE) {
    conv_qk(p, ci.x, t0, L, kh_, r, wave, lane, sm.u.r.kh, sm.u.r.qh, sm.rnk, sm.rnq, gin0);
    conv_v(p, ci.x, t0, L, kh_, r, wave, lane);
  } else {
    RowBlock<IO> kb, qb;
    load_rows<IO>(kb, (const T*)p.k + (int64_t)kh_ * DK, p.stride_k, t0, L, tid);
    load_rows<IO>(qb, (const T*)p.q + (int64_t)kh_ * DK, p.stride_q, t0, L, tid);
    const int c8 = tid & 15, rq = tid >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 4 * rq + u;
      const bool ok = row < L;
      float sk = 0.f, sq = 0.f;
      if constexpr (F32) {
        float kv[8], qv[8];
        row_vals<IO>(kb, u, ok, kv);
        row_vals<IO>(qb, u, ok, qv);
        uint4 hw, lw;
        put_row8<IO>(sm.u.r.kh, sm.u.r.kl, row * KS_STRIDE + c8 * 8, kv, hw, lw);
        put_row8<IO>(sm.u.r.qh, sm.u.r.ql, row * KS_STRIDE + c8 * 8, qv, hw, lw);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sk = fmaf(kv[j], kv[j], sk);
          sq = fmaf(qv[j], qv[j], sq);
        }
      } else {
        // bf16 rows go to LDS as they are (zero past the chunk end); the squares come
        // from the two halves of each word
        const uint4 kw = ok ? kb.w[u][0] : make_uint4(0, 0, 0, 0);
        const uint4 qw = ok ? qb.w[u][0] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(sm.u.r.kh + row * KS_STRIDE + c8 * 8) = kw;
        *reinterpret_cast<uint4*>(sm.u.r.qh + row * KS_STRIDE + c8 * 8) = qw;
        const uint32_t kx[4] = {kw.x, kw.y, kw.z, kw.w}, qx[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float k0 = __uint_as_float(kx[j] << 16), k1 = __uint_as_float(kx[j] & 0xFFFF0000u);
          const float q0 = __uint_as_float(qx[j] << 16), q1 = __uint_as_float(qx[j] & 0xFFFF0000u);
          sk = fmaf(k1, k1, fmaf(k0, k0, sk));
          sq = fmaf(q1, q1, fmaf(q0, q0, sq));
        }
      }
      sk = row16_sum(sk);
      sq = row16_sum(sq);
      if (c8 == 0) {
        // hardware reciprocal square root (about 1 ulp)
        sm.rnk[row] = p.use_l2 ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 1.0f;
        sm.rnq[row] = p.use_l2 ? __builtin_amdgcn_rsqf(sq + 1e-6f) : 1.0f;
      }
    }
  }
  __syncthreads();

  // ---- raw Gram tiles, kept in registers: the 10 lower (I >= J) 16 x 16 tiles of
  // rnk_i rnk_j (k_i . k_j) and, when P goes to the record, rnq_i rnk_j (q_i . k_j).
  // Fragment-native records: wave w holds row tile 3 - w of the K Gram (tiles (3 - w, J),
  // J <= 3 - w, in gk[J]) and the transposed Q Gram tiles (J, w), J <= w (pq[J], below):
  // five tiles per wave, and each K row block's fragments are read once per wave and
  // serve both products.  Otherwise wave w holds K Gram tiles w, w+4, w+8 (tri_tile
  // order) and, for P in rows, the Q Gram tiles at the same places.
  constexpr int NG = FRAG ? 4 : 3;
  f32x4 gk[NG], gq[3];
  f32x4 pq[4];
  const int ia = 3 - wave;          // FRAG: this wave's K Gram row tile
  if constexpr (FRAG) {
    // J runs downwards, so block ia is read (as kj) before the tiles J < ia need it (as ka)
    bf16x8 ka[4], qw[4];
    if constexpr (WITHP) {
#pragma unroll
      for (int m = 0; m < 4; ++m) qw[m] = frag_rows(sm.u.r.qh, KS_STRIDE, 16 * wave, 32 * m, lane);
    }
    const float4 ki4 = *reinterpret_cast<const float4*>(&sm.rnk[16 * ia + 4 * g4]);
    const float qi = sm.rnq[16 * wave + c16];
#pragma unroll
    for (int J = 3; J >= 0; --J) {
      gk[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      pq[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (J <= ia || (WITHP && J <= wave)) {
        bf16x8 kj[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) kj[m] = frag_rows(sm.u.r.kh, KS_STRIDE, 16 * J, 32 * m, lane);
        if (J == ia) {
#pragma unroll
          for (int m = 0; m < 4; ++m) ka[m] = kj[m];
        }
        if (J <= ia) {
#pragma unroll
          for (int m = 0; m < 4; ++m) gk[J] = mma(ka[m], kj[m], gk[J]);
          const float rkj = sm.rnk[16 * J + c16];
          gk[J][0] *= ki4.x * rkj;
          gk[J][1] *= ki4.y * rkj;
          gk[J][2] *= ki4.z * rkj;
          gk[J][3] *= ki4.w * rkj;
        }
        if (WITHP && J <= wave) {
          // (K Q^T) tile (J, w): accumulators hold rnq_i rnk_j (q_i . k_j) at
          // i = 16 w + c16, j = 16 J + 4 g4 + e; tiles J = 2m, 2m+1 together are the
          // layout of P's A-operand fragment [row tile w][token slab m]
#pragma unroll
          for (int m = 0; m < 4; ++m) pq[J] = mma(kj[m], qw[m], pq[J]);
          const float4 kj4 = *reinterpret_cast<const float4*>(&sm.rnk[16 * J + 4 * g4]);
          pq[J][0] *= qi * kj4.x;
          pq[J][1] *= qi * kj4.y;
          pq[J][2] *= qi * kj4.z;
          pq[J][3] *= qi * kj4.w;
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < 3 && !FRAG; ++tt) {
    const int n = wave + 4 * tt;
    gk[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    gq[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (n < 10) {
      int I, J;
      tri_tile(n, I, J);
      bf16x8 bk[4], ak[4], aq[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        bk[m] = frag_rows(sm.u.r.kh, KS_STRIDE, 16 * J, 32 * m, lane);
        ak[m] = frag_rows(sm.u.r.kh, KS_STRIDE, 16 * I, 32 * m, lane);
        if constexpr (WITHP && !FRAG) aq[m] = frag_rows(sm.u.r.qh, KS_STRIDE, 16 * I, 32 * m, lane);
      }
      f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        a1 = mma(ak[m], bk[m], a1);
        if constexpr (WITHP && !FRAG) a2 = mma(aq[m], bk[m], a2);
      }
      if constexpr (F32) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 bl = frag_rows(sm.u.r.kl, KS_STRIDE, 16 * J, 32 * m, lane);
          a1 = mma(frag_rows(sm.u.r.kl, KS_STRIDE, 16 * I, 32 * m, lane), bk[m], a1);
          a1 = mma(ak[m], bl, a1);
          if constexpr (WITHP) {
            a2 = mma(frag_rows(sm.u.r.ql, KS_STRIDE, 16 * I, 32 * m, lane), bk[m], a2);
            a2 = mma(aq[m], bl, a2);
          }
        }
      }
      const int j = 16 * J + c16, i0 = 16 * I + 4 * g4;
      const float rkj = sm.rnk[j];
      const float4 ki4 = *reinterpret_cast<const float4*>(&sm.rnk[i0]);
      const float4 qi4 = *reinterpret_cast<const float4*>(&sm.rnq[i0]);
      const float ki[4] = {ki4.x, ki4.y, ki4.z, ki4.w};
      const float qi[4] = {qi4.x, qi4.y, qi4.z, qi4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gk[tt][e] = ki[e] * rkj * a1[e];
        gq[tt][e] = qi[e] * rkj * a2[e];
      }
    }
  }
  // fp32 io: the hi/lo K and Q rows of this (chunk, key head) for the sweep
  if constexpr (F32) {
    uint8_t* krec = krecs + ((int64_t)c * p.Hk + kh_) * ws_krec_bytes(F32);
    const u16* planes[4] = {sm.u.r.kh, sm.u.r.kl, sm.u.r.qh, sm.u.r.ql};
#pragma unroll
    for (int pl = 0; pl < 4; ++pl) {
      const uint4* src = reinterpret_cast<const uint4*>(planes[pl]);
      uint4* dst = reinterpret_cast<uint4*>(krec + pl * WS_ROWS_BYTES);
      for (int i = tid; i < (int)(WS_ROWS_BYTES / 16); i += NTHR) dst[i] = src[i];
    }
  }

  float* const af = sm.u.m.af;
  float* const tf = sm.u.m.tf;
  for (int hb = 0; hb < r; hb += PREP_RB) {
    // ---- gates of value heads hb .. hb+3 (wave w: head hb + w, lane: token)
    __syncthreads();     // K/Q rows (phase 0) or the previous heads' T are no longer read
    {
      // (a later batch's inputs are waited for in their own branch: merged with gin0
      // while still in flight, they would be waited for after the join, behind every
      // store issued since the conv)
      uint4 graw = gin0;
      if (hb > 0) {
        graw = gate_in(hb);
        asm volatile("" : "+v"(graw.x), "+v"(graw.y), "+v"(graw.z), "+v"(graw.w));
      }
      const float4 gin = gate_vals(graw);
      float g = 0.f, beta = 0.f;
      if (hb + wave < r && lane < L) {
        if (p.g_opt) {
          g = gin.x;
          beta = gin.y;
        } else {
          gate_pair(gin.x, gin.y, gin.z, gin.w, g, beta);
        }
      }
      g = wave_prefix_sum(g);       // in-chunk cumulative log decay (padding adds 0)
      sm.gam[wave][lane] = g;
      sm.beta[wave][lane] = beta;
    }
    for (int jb = 0; jb < PREP_RB && hb + jb < r; ++jb) {
      const int h = kh_ * r + hb + jb;
      const float* gam = sm.gam[jb];
      const float* bet = sm.beta[jb];
      uint8_t* rec = recs + ((int64_t)c * Hv + h) * REC;
      __syncthreads();   // gates staged; the previous head's T is no longer read

      // ---- per-token factors for the sweep
      if (tid < 64) {
        const float gl = gam[CH - 1];
        const float gt = gam[tid];
        const float eg = __expf(gt);
        float* fac = reinterpret_cast<float*>(rec + FAC_OFF);
        fac[tid] = eg * sm.rnk[tid];
        fac[CH + tid] = eg * sm.rnq[tid];
        fac[2 * CH + tid] = __expf(gl - gt) * sm.rnk[tid];
        fac[3 * CH + tid] = __expf(gl);
        fac[4 * CH + tid] = gt;
        fac[5 * CH + tid] = sm.rnk[tid];
        fac[6 * CH + tid] = sm.rnq[tid];
        fac[7 * CH + tid] = 0.f;
      }

      // ---- A (fp32) and, for the 4-wave sweep, P (bf16 hi/lo planes staged in the T
      // buffer, strictly-upper tiles zero) of this head
      u16* pst = reinterpret_cast<u16*>(tf);
      if constexpr (FRAG) {
        // A row tile ia = 3 - w: tiles (ia, J), J <= ia
        const int i0 = 16 * ia + 4 * g4;
        const float4 gi4 = *reinterpret_cast<const float4*>(&gam[i0]);
        const float4 bi4 = *reinterpret_cast<const float4*>(&bet[i0]);
        const float gi[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
        const float bi[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          if (J <= ia) {
            const int j = 16 * J + c16;
            const float gj = gam[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = i0 + e;
              af[i * F_STRIDE + j] = (i > j) ? bi[e] * __expf(gi[e] - gj) * gk[J][e] : 0.f;
            }
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4 && !FRAG; ++tt) {
        const int n = wave + 4 * tt;
        if (n < 10) {
          int I, J;
          tri_tile(n, I, J);
          const int j = 16 * J + c16, i0 = 16 * I + 4 * g4;
          const float gj = gam[j];
          const float4 gi4 = *reinterpret_cast<const float4*>(&gam[i0]);
          const float4 bi4 = *reinterpret_cast<const float4*>(&bet[i0]);
          const float gi[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
          const float bi[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float d = (i >= j) ? __expf(gi[e] - gj) : 0.f;   // exponent <= 0
            af[i * F_STRIDE + j] = (i > j) ? bi[e] * d * gk[tt < 3 ? tt : 0][e] : 0.f;
            if constexpr (WITHP && !FRAG) {
              uint32_t ph, pl;
              split2(d * gq[tt < 3 ? tt : 0][e], 0.f, ph, pl);
              pst[i * CH + j] = (u16)ph;
              pst[CH * CH + i * CH + j] = (u16)pl;
            }
          }
        } else if (WITHP && !FRAG && n < 16) {
          // strictly-upper tiles (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
          const int m = n - 10;
          const int I = (m >= 5) ? 2 : (m >= 3) ? 1 : 0;
          const int J = m - (I == 0 ? 0 : I == 1 ? 3 : 5) + I + 1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g4 + e, j = 16 * J + c16;
            pst[i * CH + j] = 0;
            pst[CH * CH + i * CH + j] = 0;
          }
        }
      }
      if constexpr (FRAG && WITHP) {
        // P fragments of row tile w straight from the transposed tiles:
        // P_ij = e^{gamma_i - gamma_j} rnq_i rnk_j (q_i . k_j) for j <= i < L
        const int i = 16 * wave + c16;
        const float gi = gam[i];
        f32x4 pv[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          pv[J] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (J <= wave) {       // tiles right of the diagonal tile are zero
            const float4 gj4 = *reinterpret_cast<const float4*>(&gam[16 * J + 4 * g4]);
            const float gj[4] = {gj4.x, gj4.y, gj4.z, gj4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int jj = 16 * J + 4 * g4 + e;
              pv[J][e] = (jj <= i) ? __expf(gi - gj[e]) * pq[J][e] : 0.f;   // exponent <= 0
            }
          }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m == 1 && wave < 2) continue;   // zero: tokens 32.. lie right of row tiles 0, 1
          bf16x8 hi, lo;
          frag_acc_split(pv[2 * m], pv[2 * m + 1], hi, lo);
          *reinterpret_cast<uint4*>(rec + FR_P_OFF + fr_tp(wave, m, 0) + lane * 16) = __builtin_bit_cast(uint4, hi);
          *reinterpret_cast<uint4*>(rec + FR_P_OFF + fr_tp(wave, m, 1) + lane * 16) = __builtin_bit_cast(uint4, lo);
        }
      }
      __syncthreads();
      if constexpr (WITHP && !FRAG) {
        // P planes to the record, rows padded to 72 (four 16-byte words per thread)
        const uint4* src = reinterpret_cast<const uint4*>(pst);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int i = tid + NTHR * it;        // plane i >> 9, row (i & 511) >> 3, word i & 7
          const int plane = i >> 9, row = (i & 511) >> 3, w = i & 7;
          *reinterpret_cast<uint4*>(rec + WS_P_OFF + plane * WS_PL_BYTES + row * (T_STRIDE * 2) +
                                    w * 16) = src[i];
        }
        __syncthreads();   // the T buffer is reused below
      }

      // ---- T = (I + A)^{-1}, blocked: 16 x 16 diagonal blocks by forward substitution
      // (one column per lane); then T_10, T_32 = -T_ii A_ij T_jj; then the lower
      // 32 x 32 block T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32]
      // (wave 0 solves all four diagonal blocks, block g4 in lane group g4: the same
      // latency as one block per wave, a quarter of the VALU instructions)
      if (wave == 0) {
        const int b = g4;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float* arow = &af[(16 * b + i) * F_STRIDE + 16 * b];
          float a[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 t4 = *reinterpret_cast<const float4*>(arow + 4 * q4);
            a[4 * q4] = t4.x; a[4 * q4 + 1] = t4.y; a[4 * q4 + 2] = t4.z; a[4 * q4 + 3] = t4.w;
          }
          float sacc = (i == c16) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < i; ++j) sacc = fmaf(-a[j], x[j], sacc);
          x[i] = sacc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tf[(16 * b + i) * F_STRIDE + 16 * b + c16] = x[i];
      } else if (wave == 1 && g4 < 2) {
        // the strictly-upper blocks T_01 and T_23 enter the 32 x 32 products below: zero
        const int bb = 2 * g4;
#pragma unroll
        for (int i = 0; i < 16; ++i) tf[(16 * bb + i) * F_STRIDE + 16 * bb + 16 + c16] = 0.f;
      }
      __syncthreads();
      // blocks (1,0) (wave 0) and (3,2) (wave 1): T_IJ = -T_II (A_IJ T_JJ), 16 x 16 fp32
      // MFMA products; the intermediate goes through a wave-private LDS tile
      if (wave < 2) {
        const int I = 2 * wave + 1, J = 2 * wave;
        float* mt = af + wave * (16 * 20);   // rows 0..9 of A: dead by now
        f32x4 m = tile_mma_f32<16>(&af[16 * I * F_STRIDE + 16 * J], F_STRIDE,
                                   &tf[16 * J * F_STRIDE + 16 * J], F_STRIDE, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) mt[(4 * g4 + e) * 20 + c16] = m[e];
        const f32x4 t = tile_mma_f32<16>(&tf[16 * I * F_STRIDE + 16 * I], F_STRIDE, mt, 20, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) tf[(16 * I + 4 * g4 + e) * F_STRIDE + 16 * J + c16] = -t[e];
      }
      __syncthreads();
      // lower 32 x 32 block: T[32:64, 0:32] = -T[32:64, 32:64] (A[32:64, 0:32] T[0:32, 0:32]),
      // one 16 x 16 output tile per wave
      {
        const int ti = wave >> 1, tj = wave & 1;
        const f32x4 m = tile_mma_f32<32>(&af[(32 + 16 * ti) * F_STRIDE], F_STRIDE,
                                         &tf[16 * tj], F_STRIDE, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) af[(16 * ti + 4 * g4 + e) * 36 + 16 * tj + c16] = m[e];
        __syncthreads();
        const f32x4 t = tile_mma_f32<32>(&tf[(32 + 16 * ti) * F_STRIDE + 32], F_STRIDE,
                                         &af[16 * tj], 36, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tf[(32 + 16 * ti + 4 * g4 + e) * F_STRIDE + 16 * tj + c16] = -t[e];
        __syncthreads();
      }
      // ---- T' = T diag(beta), lower triangle, as bf16 hi/lo planes straight to the
      // workspace (4 consecutive columns per thread per step: 8-byte stores)
      if constexpr (FRAG) {
        // fragment order: unit (j, m, lane) splits the lane's 8 values of row 16 j + (lane &
        // 15), columns 32 m + 4 (lane >> 4) .. + 3 and 32 m + 16 + 4 (lane >> 4) .. + 3
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int u = tid + NTHR * it;          // j u >> 7, m (u >> 6) & 1, lane u & 63
          const int jj = u >> 7, m = (u >> 6) & 1, l = u & 63;
          if (m == 1 && jj < 2) continue;    // zero fragments, never read
          const int i = 16 * jj + (l & 15);
          float v[8];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int j0 = 32 * m + 16 * half + 4 * (l >> 4);
            const float4 t4 = *reinterpret_cast<const float4*>(&tf[i * F_STRIDE + j0]);
            const float4 b4 = *reinterpret_cast<const float4*>(&bet[j0]);
            v[4 * half + 0] = (j0 <= i) ? t4.x * b4.x : 0.f;
            v[4 * half + 1] = (j0 + 1 <= i) ? t4.y * b4.y : 0.f;
            v[4 * half + 2] = (j0 + 2 <= i) ? t4.z * b4.z : 0.f;
            v[4 * half + 3] = (j0 + 3 <= i) ? t4.w * b4.w : 0.f;
          }
          uint4 hw, lw;
          split2(v[0], v[1], hw.x, lw.x);
          split2(v[2], v[3], hw.y, lw.y);
          split2(v[4], v[5], hw.z, lw.z);
          split2(v[6], v[7], hw.w, lw.w);
          *reinterpret_cast<uint4*>(rec + FR_T_OFF + fr_tp(jj, m, 0) + l * 16) = hw;
          *reinterpret_cast<uint4*>(rec + FR_T_OFF + fr_tp(jj, m, 1) + l * 16) = lw;
        }
      } else {
        u16* tph = reinterpret_cast<u16*>(rec);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int idx = tid + NTHR * it;          // row i, column group j0
          const int i = idx >> 4, j0 = (idx & 15) * 4;
          const float4 t4 = *reinterpret_cast<const float4*>(&tf[i * F_STRIDE + j0]);
          const float4 b4 = *reinterpret_cast<const float4*>(&bet[j0]);
          const float v0 = (j0 <= i) ? t4.x * b4.x : 0.f;
          const float v1 = (j0 + 1 <= i) ? t4.y * b4.y : 0.f;
          const float v2 = (j0 + 2 <= i) ? t4.z * b4.z : 0.f;
          const float v3 = (j0 + 3 <= i) ? t4.w * b4.w : 0.f;
          uint32_t h0, l0, h1, l1;
          split2(v0, v1, h0, l0);
          split2(v2, v3, h1, l1);
          *reinterpret_cast<uint2*>(tph + i * T_STRIDE + j0) = make_uint2(h0, h1);
          *reinterpret_cast<uint2*>(tph + CH * T_STRIDE + i * T_STRIDE + j0) = make_uint2(l0, l1);
        }
      }
    }
  }
}

// ============================================================================ 3. sweep
typedef __attribute__((address_space(3))) void lds_void;

// Copy nslots 16-byte words from a linear global source into linear LDS with the
// LDS DMA path (global_load_lds_dwordx4: lane l's word lands at dst + 16 l).  Sources
// are a wave-uniform base plus a 32-bit per-lane offset, the LDS destination (M0) is
// scalar, and the sweep workgroup's waves take turns by instruction.  Every wave issues
// the same number of copies (a wave past the last instruction repeats it, writing the
// same bytes again), so a piece is straight-line code that stays where it is placed.
// One LDS DMA copy (lane l's 16 bytes at src land at dst + 16 l).  OPAQUE = false uses
// the compiler builtin, which makes later LDS reads wait for the copy unless the compiler
// can prove them disjoint; OPAQUE = true issues it as inline assembly the compiler does not
// track, for kernels that order every read of a copied buffer after an explicit
// vmcnt(0) wait and a barrier themselves.
template <bool OPAQUE>
__device__ __forceinline__ void lds_dma16(const uint8_t* src, void* dst) {
  if constexpr (OPAQUE) {
    const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)dst;
    // M0 carries the LDS destination; the kernels using this write M0 nowhere else
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m)
                 : "memory", "m0");
#pragma clang diagnostic pop
  } else {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
  }
}

// the same as lds_dma16<true> with the source as a wave-uniform base plus a 32-bit
// per-lane byte offset (the scalar-base form: no 64-bit address arithmetic per copy)
__device__ __forceinline__ void lds_dma16_sbase(const uint8_t* base, uint32_t off, void* dst) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)dst;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(m)
               : "memory", "m0");
#pragma clang diagnostic pop
}

template <int NS, int NW, bool OPAQUE = false>   // 16-byte slots (a multiple of 64), waves taking turns
__device__ __forceinline__ void dma_linear(const uint8_t* src, void* dst, int wave, int lane) {
  static_assert(NS % 64 == 0, "whole instructions only");
  constexpr int INS = NS / 64;
#pragma unroll
  for (int j = 0; j < (INS + NW - 1) / NW; ++j) {
    const int ins = min(wave + NW * j, INS - 1);
    lds_dma16<OPAQUE>(src + ins * 1024 + lane * 16, (char*)dst + ins * 1024);
  }
}

// Staged-row DMA: a chunk's 64 rows of DW 16-byte words each land in LDS rows of
// DW + 1 words (the extra word pads the row against bank conflicts and re-reads the
// last data word); slot = 64 ins + lane with ins = min(wave + NW j, INS - 1).  The table
// packs each slot's row (bits 0..7) and the source byte offset of its word (bits 8..).
template <int DW, int NW>
struct RowDma {
  static constexpr int INS = CH * (DW + 1) / 64;   // instructions per block
  static constexpr int J = (INS + NW - 1) / NW;    // per wave, rounded up
};

template <int DW, int NW>
__device__ __forceinline__ void rows_table(int wave, int lane, uint32_t (&tab)[RowDma<DW, NW>::J]) {
  typedef RowDma<DW, NW> R;
#pragma unroll
  for (int j = 0; j < R::J; ++j) {
    const int sl = min(wave + NW * j, R::INS - 1) * 64 + lane;
    const int row = sl / (DW + 1), w = sl - row * (DW + 1);
    tab[j] = (uint32_t)row | ((uint32_t)((w < DW ? w : DW - 1) * 16) << 8);
  }
}

// rows t0 .. t0+63 of one chunk into LDS; rows past the chunk end (L valid rows) repeat
// the last valid row, which the chunk algebra multiplies by zero.  base = the chunk's
// first row (wave-uniform), row_bytes < 2^24.
template <int DW, int NW, bool OPAQUE = false>
__device__ __forceinline__ void dma_rows(const uint8_t* base, uint32_t row_bytes, int L,
                                         const uint32_t (&tab)[RowDma<DW, NW>::J], void* dst,
                                         int wave) {
  typedef RowDma<DW, NW> R;
#pragma unroll
  for (int j = 0; j < R::J; ++j) {
    const int ins = min(wave + NW * j, R::INS - 1);
    const uint32_t row = min(tab[j] & 0xFFu, (uint32_t)(L - 1));
    const uint32_t off = __umul24(row, row_bytes) + (tab[j] >> 8);
    lds_dma16<OPAQUE>(base + off, (char*)dst + ins * 1024);
  }
}

// wait for all of this wave's outstanding vector-memory operations (incl. LDS DMA)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS buffers of the sweep, one __shared__ object each so that the compiler can tell
// the DMA destinations of one phase from the buffers the other phase reads.
template <int IO, int NW>
struct SweepSizes {
  static constexpr bool F32 = (IO == IO_F32);
  static constexpr int THR = 64 * NW;
  static constexpr int DVB = 16 * NW;                  // dv columns per workgroup
  static constexpr int NBLK = DV / DVB;
  static constexpr int O_STRIDE = DVB + 8;             // u16 per staged output row
  static constexpr int V_STRIDE = DVB + 8;             // u16 per staged V row
  static constexpr int ROWS = CH * KS_STRIDE;          // K or Q rows (u16)
  static constexpr int ROWS_LO = F32 ? ROWS : 8;
  static constexpr int PL2 = 2 * CH * T_STRIDE;        // a hi|lo plane pair (u16)
  static constexpr int OST = F32 ? 8 : CH * O_STRIDE;
  static constexpr int VST = F32 ? 8 : CH * V_STRIDE;
  static constexpr int VW = DVB * 2 / 16;              // 16-byte words per bf16 V row slice
  static constexpr int OW = DVB / 8;                   // 16-byte words per bf16 output row
};

// Segments of a sequence (the intra-sequence scan).  A sequence's nch chunks split into
// G segments, segment g = chunks [g nch / G, (g+1) nch / G).  The transition launch
// (TRANS) runs segments 0 .. G-2 from the augmented start state [0 | I] with no output:
// columns driven by V from zero give B_g, columns started at the identity with V = 0 give
// the segment's transition A_g, so that S(end of g) = A_g S(start of g) + B_g.  The normal
// launch then starts segment g from S = A_{g-1}(... (A_0 S_in + B_0) ...) + B_{g-1}.
struct SegArgs {
  int G;          // segments per sequence (1: none)
  int seg_base;   // first segment of this launch (normal launch)
  int seg_count;  // segments covered by this launch
  float* scratch; // per (sequence, head, segment < G-1): A (dk x dk), then B (dk x dv), fp32
  int64_t rec_bytes;  // stride of the (chunk, head) records: with or without P
};

template <int IO, int NW, bool TRANS>
__global__ void __launch_bounds__(64 * NW)
chunk_sweep_kernel(ChunkArgs p, const int32_t* __restrict__ cmap, const uint8_t* __restrict__ recs,
                   const uint8_t* __restrict__ krecs, SegArgs sg) {
  typedef Io<IO> io;
  typedef typename io::T T;
  constexpr bool F32 = (IO == IO_F32);
  // P: copied from the record by the 4-wave (latency-bound) shape, formed in the sweep
  // from the staged Q and K rows by the 8-wave (throughput-bound) shape
  constexpr bool PREC = (NW == 4);
  // bf16 io: T' (and, for the 4-wave shape, P) comes as fragment-native records, and the
  // 8-wave shape forms P in fragment order, so every T' and P fragment is one 16-byte
  // lane-linear read (records with P for the 4-wave and transition launches, which share
  // them, without P for the 8-wave normal launch)
  constexpr bool FT = !F32;
  constexpr int64_t TFAC_OFF = (TRANS || PREC) ? FR_FAC_OFF : FRT_FAC_OFF;
  typedef SweepSizes<IO, NW> Z;
  constexpr int DVB = Z::DVB, NBLK = Z::NBLK, O_STRIDE = Z::O_STRIDE, V_STRIDE = Z::V_STRIDE;
  // K rows are double-buffered by chunk parity: chunk n's rows serve its K S products
  // and, read transposed, its state update, while chunk n+1's rows land
  __shared__ __attribute__((aligned(16))) u16 s_k0[Z::ROWS];    // K rows (bf16 / hi), even chunks
  __shared__ __attribute__((aligned(16))) u16 s_k1[Z::ROWS];    // K rows (bf16 / hi), odd chunks
  __shared__ __attribute__((aligned(16))) u16 s_kl0[Z::ROWS_LO];
  __shared__ __attribute__((aligned(16))) u16 s_kl1[Z::ROWS_LO];
  __shared__ __attribute__((aligned(16))) u16 s_qh[Z::ROWS];    // Q rows              phase A
  __shared__ __attribute__((aligned(16))) u16 s_ql[Z::ROWS_LO];
  __shared__ __attribute__((aligned(16))) u16 s_tp[Z::PL2];     // T' hi | lo          phase A
  __shared__ __attribute__((aligned(16))) u16 s_pp[Z::PL2];     // P hi | lo (formed in phase A)
  __shared__ __attribute__((aligned(16))) float s_fac[FAC_ROWS * CH];  // per-token factors  phase A
  __shared__ __attribute__((aligned(16))) u16 s_ost[Z::OST];    // output tile (bf16 io)
  __shared__ __attribute__((aligned(16))) u16 s_v[Z::VST];      // V slice (bf16 io)   phase A

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  // Workgroups come in groups (sequence, key head, segment of this launch); a group's
  // members are its value heads times its column blocks (a transition launch has twice
  // the column blocks: half 0 the V-driven columns, half 1 the transition).  The device
  // deals consecutive workgroups to its 8 XCDs in turn, so a group's members get ids
  // congruent mod 8 and share one XCD's L2 (the K/Q rows, and each head's records across
  // its column blocks); the last octet of groups is padded.
  constexpr int NB = TRANS ? 2 * NBLK : NBLK;
  const int Hv = p.Hv, r = Hv / p.Hk;
  const int GS = r * NB;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int member = slot % GS;
  const int group = (slot / GS) * 8 + xcd;
  if (group >= p.Ns * p.Hk * sg.seg_count) return;
  const int blk_all = member % NB;
  const int half = blk_all / NBLK;                   // transition launch: 1 = the A columns
  const int blk = blk_all % NBLK;
  const int gi = group % sg.seg_count;
  const int kh = (group / sg.seg_count) % p.Hk;
  const int s = group / sg.seg_count / p.Hk;
  const int h = kh * r + member / NB;
  const int g = sg.seg_base + gi;                    // this workgroup's segment
  int64_t b0, b1;
  seq_bounds(p.cu, p.N, s, b0, b1);
  const int c0 = p.Ns == 1 ? 0 : cmap[s];   // (one sequence: no chunk map)
  const int nch = (int)((b1 - b0 + CH - 1) / CH);
  const int nb = (int)((int64_t)g * nch / sg.G);        // chunks [nb, ne) of the segment
  const int ne = (int)((int64_t)(g + 1) * nch / sg.G);
  const int col = blk * DVB + wave * 16 + c16;      // this lane's dv column
  float* const seg_rec = sg.scratch + (((int64_t)s * Hv + h) * (sg.G - 1)) * (2 * DK * DV);

  const T* qg = (const T*)p.q + (int64_t)kh * DK;
  const T* kg = (const T*)p.k + (int64_t)kh * DK;
  T* og = (T*)p.o + (int64_t)h * DV + col;
  T* og0 = (T*)p.o + (int64_t)h * DV + blk * DVB;   // this workgroup's output columns
  const int64_t o_stride = (int64_t)Hv * DV;
  const int64_t krec_bytes = ws_krec_bytes(F32);

  // ---- recurrent state slice: S[i] holds rows 16 i + 4 g4 + e of column col
  f32x4 S[8];
  if (TRANS) {
    // zero for the V-driven part, the identity's column col for the transition part
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[i][e] = (half == 1 && 16 * i + 4 * g4 + e == col) ? 1.f : 0.f;
  } else if (p.state_in) {
    const float* sp = p.state_in + ((int64_t)s * Hv + h) * DK * DV + col;
    float tmp[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) tmp[k] = sp[(16 * (k >> 2) + 4 * g4 + (k & 3)) * DV];
#pragma unroll
    for (int k = 0; k < 32; ++k) S[k >> 2][k & 3] = tmp[k];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (!TRANS) {
    // segment g > 0 starts from A_{g-1}(... (A_0 S_in + B_0) ...) + B_{g-1}: MFMA products
    // with A split into bf16 hi/lo and S split into hi/lo (three passes)
    for (int j = 0; j < g; ++j) {
      const float* Aj = seg_rec + (int64_t)j * (2 * DK * DV);
      const float* Bj = Aj + DK * DV;
      bf16x8 sh[4], sl[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) frag_acc_split(S[2 * m], S[2 * m + 1], sh[m], sl[m]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // all of row tile i's loads first, so that they are in flight together
        f32x4 acc;
        float4 xa[4][2];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float* ar = Aj + (16 * i + c16) * DK + 32 * m + 4 * g4;
          xa[m][0] = *reinterpret_cast<const float4*>(ar);
          xa[m][1] = *reinterpret_cast<const float4*>(ar + 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = Bj[(16 * i + 4 * g4 + e) * DV + col];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 x0 = xa[m][0], x1 = xa[m][1];
          uint4 vh, vl;
          split2(x0.x, x0.y, vh.x, vl.x);
          split2(x0.z, x0.w, vh.y, vl.y);
          split2(x1.x, x1.y, vh.z, vl.z);
          split2(x1.z, x1.w, vh.w, vl.w);
          const bf16x8 ah = __builtin_bit_cast(bf16x8, vh), al = __builtin_bit_cast(bf16x8, vl);
          acc = mma(ah, sh[m], acc);
          acc = mma(al, sh[m], acc);
          acc = mma(ah, sl[m], acc);
        }
        S[i] = acc;
      }
    }
  }

  // Operands of chunk n, copied in pieces so that the copies issue between the
  // matrix products of the other phase.  Phase A (K, Q rows, T' planes, factors, the
  // V slice) lands while the previous chunk's phase B runs, phase B (P planes) while
  // chunk n's phase A runs.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  constexpr int VW = Z::VW;
  uint32_t ktab[RowDma<16, NW>::J], vtab[RowDma<VW, NW>::J];
  rows_table<16, NW>(wave_u, lane, ktab);
  rows_table<VW, NW>(wave_u, lane, vtab);
  const uint32_t qrow_bytes = (uint32_t)(p.stride_q * (int64_t)sizeof(T));
  const uint32_t krow_bytes = (uint32_t)(p.stride_k * (int64_t)sizeof(T));
  const uint32_t vrow_bytes = (uint32_t)(p.stride_v * (int64_t)sizeof(T));
  const uint8_t* vg0 = (const uint8_t*)p.v + ((int64_t)h * DV + blk * DVB) * sizeof(T);
  const uint32_t vcol = (uint32_t)((wave * 16 + c16) * sizeof(T));
  T vraw[4][4];   // fp32 io: the V slice goes through registers
  // (sched_barrier keeps the instruction scheduler from sinking a piece past the
  // products it is meant to overlap)
  // the 12 non-zero fragments of a fragment-native T' or P (row tiles 0 and 1 have no
  // token slab 1), one 1 KB copy each, the waves taking turns
  auto frag_copy = [&](const uint8_t* src, u16* dst) {
#pragma unroll
    for (int jj = 0; jj < (12 + NW - 1) / NW; ++jj) {
      const int ins = min(wave_u + NW * jj, 11);
      const int f = ins < 2 ? ins : ins < 4 ? ins + 2 : ins + 4;
      lds_dma16<false>(src + f * 1024 + lane * 16, (char*)dst + f * 1024);
    }
  };
  auto stage_a = [&](int n, int part, u16* kdst, u16* kldst) {
    __builtin_amdgcn_sched_barrier(0);
    const int64_t t0 = b0 + (int64_t)n * CH;
    const int L = (int)min((int64_t)CH, b1 - t0);
    const uint8_t* rec = recs + ((int64_t)(c0 + n) * Hv + h) * sg.rec_bytes;
    const uint8_t* krec = krecs + ((int64_t)(c0 + n) * p.Hk + kh) * krec_bytes;
    if (part == 0) {
      if constexpr (F32) {
        dma_linear<(WS_ROWS_BYTES) / 16, NW>(krec, kdst, wave_u, lane);
        dma_linear<(WS_ROWS_BYTES) / 16, NW>(krec + WS_ROWS_BYTES, kldst, wave_u, lane);
      } else {
        (void)kldst;
        dma_rows<16, NW>((const uint8_t*)kg + t0 * krow_bytes, krow_bytes, L, ktab, kdst, wave_u);
      }
    } else if (part == 1) {
      if constexpr (TRANS) {
      } else if constexpr (F32) {
        dma_linear<(WS_ROWS_BYTES) / 16, NW>(krec + 2 * WS_ROWS_BYTES, s_qh, wave_u, lane);
        dma_linear<(WS_ROWS_BYTES) / 16, NW>(krec + 3 * WS_ROWS_BYTES, s_ql, wave_u, lane);
      } else {
        dma_rows<16, NW>((const uint8_t*)qg + t0 * qrow_bytes, qrow_bytes, L, ktab, s_qh, wave_u);
      }
    } else if (part == 2) {
      if constexpr (FT) {
        // the 12 non-zero T' fragments (row tiles 0 and 1 have no token slab 1), one
        // 1 KB copy each, then the factor rows
        frag_copy(rec + FR_T_OFF, s_tp);
        dma_linear<FAC_ROWS * CH * 4 / 16, NW>(rec + TFAC_OFF, s_fac, wave_u, lane);
      } else {
        dma_linear<(2 * WS_PL_BYTES) / 16, NW>(rec, s_tp, wave_u, lane);
        dma_linear<FAC_ROWS * CH * 4 / 16, NW>(rec + WS_FAC_OFF, s_fac, wave_u, lane);
      }
    } else if (!TRANS || half == 0) {
      const uint8_t* vb = vg0 + t0 * vrow_bytes;
      if constexpr (F32) {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t t = (uint32_t)min(16 * I + 4 * g4 + e, L - 1);
            vraw[I][e] = *(const T*)(vb + (__umul24(t, vrow_bytes) + vcol));
          }
      } else {
        dma_rows<VW, NW>(vb, vrow_bytes, L, vtab, s_v, wave_u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // bf16 io: a chunk's output stays in registers (packed pairs of rows) through the
  // next chunk boundary, is written to the LDS tile there while no DMA is in flight
  // (the compiler makes LDS stores wait for every pending DMA), and leaves as
  // coalesced 16-byte rows after the next barrier.
  uint32_t opk[4][2];
  auto write_ost = [&]() {
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g4 + e;
        const uint32_t w = opk[I][e >> 1];
        s_ost[t * O_STRIDE + wave * 16 + c16] = (u16)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
      }
  };
  auto store_o = [&](int n) {
    const int64_t t0 = b0 + (int64_t)n * CH;
    const int L = (int)min((int64_t)CH, b1 - t0);
    const u16* ot = s_ost;
    constexpr int WPR = Z::OW;
    static_assert((CH * WPR) % Z::THR == 0, "whole output tile per pass");
    // (all LDS reads first, kept out of the conditional stores so that they share one wait)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int NIT = CH * WPR / Z::THR;
    u32x4 w[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + Z::THR * it;
      w[it] = *reinterpret_cast<const u32x4*>(&ot[(idx / WPR) * O_STRIDE + (idx % WPR) * 8]);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) asm volatile("" : "+v"(w[it]));
    // (a wave-uniform base and a 32-bit element offset: no 64-bit addresses per lane)
    T* const ob = og0 + t0 * o_stride;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + Z::THR * it;
      const int row = idx / WPR, c8 = idx % WPR;
      if (row < L)
        *reinterpret_cast<u32x4*>(ob + (uint32_t)(row * (uint32_t)o_stride + c8 * 8)) = w[it];
    }
  };

  auto stage_p = [&](int n) {     // phase-B operand of chunk n: the P planes of its record
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* rec = recs + ((int64_t)(c0 + n) * Hv + h) * sg.rec_bytes;
    if constexpr (FT)
      frag_copy(rec + FR_P_OFF, s_pp);
    else
      dma_linear<(2 * WS_PL_BYTES) / 16, NW>(rec + WS_P_OFF, s_pp, wave_u, lane);
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (!TRANS && !PREC) {
    // P U reads the strictly-upper tiles (0,1) and (2,3) of P's planes: zero them once
    for (int idx = tid; idx < 1024; idx += Z::THR) {
      const int t = (idx >> 8) & 1, e = idx & 255;
      const int i = 32 * t + (e >> 4), j = 32 * t + 16 + (e & 15);
      if constexpr (FT)
        s_pp[frag_off(i, j, idx >> 9)] = 0;
      else
        s_pp[(idx >> 9) * CH * T_STRIDE + i * T_STRIDE + j] = 0;
    }
  }
  if (ne > nb) {
#pragma unroll
    for (int part = 0; part < 4; ++part) stage_a(nb, part, s_k0, s_kl0);
  }

  // one chunk; PAR = n & 1 picks the K buffers at compile time
  auto chunk = [&](int n, auto par) {
    constexpr int PAR = decltype(par)::value;
    u16* const kcur = PAR ? s_k1 : s_k0;
    u16* const kcl = PAR ? s_kl1 : s_kl0;
    u16* const knext = PAR ? s_k0 : s_k1;
    u16* const knl = PAR ? s_kl0 : s_kl1;
    const int64_t t0 = b0 + (int64_t)n * CH;
    const int L = (b1 - t0) < CH ? (int)(b1 - t0) : CH;

    wait_vmem();
    __syncthreads();       // phase-A operands of chunk n are in LDS; phase B of n-1 is done
    if constexpr (!F32 && !TRANS) {
      if (n > nb) write_ost();
    }
    if constexpr (!TRANS && PREC) stage_p(n);

    // ================= phase A: K S and Q S (S hi/lo), R, U = T' R
    float vr[4][4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g4 + e;
        // rows past the chunk end hold copies of its last row: read, then zero (and
        // V = 0 for the transition columns of a transition launch)
        const float x = F32 ? (float)vraw[I][e] : bf2f(s_v[t * V_STRIDE + wave * 16 + c16]);
        vr[I][e] = (t < L && !(TRANS && half == 1)) ? x : 0.f;
      }

    f32x4 R[4], QS[4];
    {
      // contraction slab outermost: the eight accumulators (K S and Q S for four row
      // tiles) are independent, so consecutive products never wait on each other
      f32x4 ks[4], qs[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        ks[I] = f32x4{0.f, 0.f, 0.f, 0.f};
        qs[I] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        bf16x8 sh, sl;
        frag_acc_split(S[2 * m], S[2 * m + 1], sh, sl);
        bf16x8 ak[4], aq[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          ak[I] = frag_rows(kcur, KS_STRIDE, 16 * I, 32 * m, lane);
          if constexpr (!TRANS) aq[I] = frag_rows(s_qh, KS_STRIDE, 16 * I, 32 * m, lane);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          ks[I] = mma(ak[I], sh, ks[I]);
          if constexpr (!TRANS) qs[I] = mma(aq[I], sh, qs[I]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          ks[I] = mma(ak[I], sl, ks[I]);
          if constexpr (!TRANS) qs[I] = mma(aq[I], sl, qs[I]);
        }
        if constexpr (F32) {
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            ks[I] = mma(frag_rows(kcl, KS_STRIDE, 16 * I, 32 * m, lane), sh, ks[I]);
            if constexpr (!TRANS) qs[I] = mma(frag_rows(s_ql, KS_STRIDE, 16 * I, 32 * m, lane), sh, qs[I]);
          }
        }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if constexpr (!TRANS) {
          const float4 cq = *reinterpret_cast<const float4*>(&s_fac[CH + 16 * I + 4 * g4]);
          QS[I][0] = cq.x * qs[I][0];
          QS[I][1] = cq.y * qs[I][1];
          QS[I][2] = cq.z * qs[I][2];
          QS[I][3] = cq.w * qs[I][3];
        }
        const float4 c4 = *reinterpret_cast<const float4*>(&s_fac[16 * I + 4 * g4]);
        R[I][0] = vr[I][0] - c4.x * ks[I][0];
        R[I][1] = vr[I][1] - c4.y * ks[I][1];
        R[I][2] = vr[I][2] - c4.z * ks[I][2];
        R[I][3] = vr[I][3] - c4.w * ks[I][3];
      }
    }
    if constexpr (!TRANS && !PREC) {
      // P of this chunk from its staged Q and K rows: the lower 16 x 16 tiles of
      // e^{gamma_i - gamma_j} (q_i . k_j) / (|q_i| |k_j|) for j <= i < L, as bf16 hi/lo
      // planes, spread over the waves; P U reads them after the phase barrier
      const float* gam = s_fac + 4 * CH;
      const float* rnk = s_fac + 5 * CH;
      const float* rnq = s_fac + 6 * CH;
      for (int tn = wave_u; tn < 10; tn += NW) {
        int I, J;
        tri_tile(tn, I, J);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 aq = frag_rows(s_qh, KS_STRIDE, 16 * I, 32 * m, lane);
          const bf16x8 bk = frag_rows(kcur, KS_STRIDE, 16 * J, 32 * m, lane);
          acc = mma(aq, bk, acc);
          if constexpr (F32) {
            acc = mma(frag_rows(s_ql, KS_STRIDE, 16 * I, 32 * m, lane), bk, acc);
            acc = mma(aq, frag_rows(kcl, KS_STRIDE, 16 * J, 32 * m, lane), acc);
          }
        }
        const int j = 16 * J + c16, i0 = 16 * I + 4 * g4;
        const float gj = gam[j], rkj = rnk[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          const float v = (i >= j && i < L) ? __expf(gam[i] - gj) * rnq[i] * rkj * acc[e] : 0.f;
          uint32_t ph, pl;
          split2(v, 0.f, ph, pl);
          if constexpr (FT) {
            s_pp[frag_off(i, j, 0)] = (u16)ph;
            s_pp[frag_off(i, j, 1)] = (u16)pl;
          } else {
            s_pp[i * T_STRIDE + j] = (u16)ph;
            s_pp[CH * T_STRIDE + i * T_STRIDE + j] = (u16)pl;
          }
        }
      }
    }
    // U = T' R   (T' lower triangular: row tile I needs token slabs 0 .. I/2); the
    // products are ordered so that each accumulator's next product is four (slab 0) or
    // two (slab 1) products away
    f32x4 U[4];
    {
      bf16x8 rh[2], rl[2];
      frag_acc_split(R[0], R[1], rh[0], rl[0]);
      frag_acc_split(R[2], R[3], rh[1], rl[1]);
      if constexpr (FT)
        tri_apply_frag(s_tp, rh, rl, U, lane, []() {});
      else
        tri_apply(s_tp, rh, rl, U, lane);
    }
    // the state update's right operand diag(e^{gamma_L - gamma} / |k|) U, and e^{gamma_L}:
    // every factor is read in phase A, since the next chunk's factors land in phase B
    bf16x8 wh[2], wl[2];
    const float egl = s_fac[3 * CH];
    {
      f32x4 Us[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const float4 c4 = *reinterpret_cast<const float4*>(&s_fac[2 * CH + 16 * I + 4 * g4]);
        Us[I][0] = c4.x * U[I][0];
        Us[I][1] = c4.y * U[I][1];
        Us[I][2] = c4.z * U[I][2];
        Us[I][3] = c4.w * U[I][3];
      }
      frag_acc_split(Us[0], Us[1], wh[0], wl[0]);
      frag_acc_split(Us[2], Us[3], wh[1], wl[1]);
    }

    wait_vmem();
    __syncthreads();       // phase-B operands of chunk n are in LDS; phase A of n is done
    // the last chunk reloads its own phase-A operands (unread in phase B) so that the
    // copies stay unconditional and keep their places between the products
    const int na = n + 1 < ne ? n + 1 : n;
    stage_a(na, 0, knext, knl);
    if constexpr (!F32 && !TRANS) {
      if (n > nb) store_o(n - 1);
    }

    // ================= phase B: O = scale (diag(e^g/|q|) Q S + P U); state update
    if constexpr (!TRANS) {
      bf16x8 uh[2], ul[2];
      frag_acc_split(U[0], U[1], uh[0], ul[0]);
      frag_acc_split(U[2], U[3], uh[1], ul[1]);
      f32x4 pu[4];
      if constexpr (FT)
        tri_apply_frag(s_pp, uh, ul, pu, lane, [&]() { stage_a(na, 1, knext, knl); });
      else
        tri_apply(s_pp, uh, ul, pu, lane, [&]() { stage_a(na, 1, knext, knl); });
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = p.scale * (QS[I][e] + pu[I][e]);
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * I + 4 * g4 + e;
            if (t < L) io::st(og, (t0 + t) * o_stride, ov[e]);
          }
        } else {
          opk[I][0] = cvt2(ov[0], ov[1]);
          opk[I][1] = cvt2(ov[2], ov[3]);
        }
      }
    }
    stage_a(na, 2, knext, knl);
    // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma} / |k|) U, K^T read transposed
    // from this chunk's K rows; token slab outermost, so the eight row tiles' products
    // are independent
    {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] *= egl;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 ak[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ak[i] = frag_kt(kcur, 16 * i, 32 * m, lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = mma(ak[i], wh[m], S[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = mma(ak[i], wl[m], S[i]);
        if constexpr (F32) {
#pragma unroll
          for (int i = 0; i < 8; ++i) S[i] = mma(frag_kt(kcl, 16 * i, 32 * m, lane), wh[m], S[i]);
        }
        if (m == 0) stage_a(na, 3, knext, knl);
      }
    }
  };
  for (int n = nb; n < ne; n += 2) {
    chunk(n, std::integral_constant<int, 0>());
    if (n + 1 < ne) chunk(n + 1, std::integral_constant<int, 1>());
  }
  if constexpr (!F32 && !TRANS) {
    if (ne > nb) {
      __syncthreads();     // every wave has read the tile of chunk ne-2
      write_ost();
      __syncthreads();
      store_o(ne - 1);
    }
  }

  if constexpr (TRANS) {
    // A_g (transition columns) or B_g (V-driven columns) of this segment
    float* sp = seg_rec + (int64_t)g * (2 * DK * DV) + (half == 1 ? 0 : DK * DV) + col;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[(16 * i + 4 * g4 + e) * DV] = S[i][e];
    return;
  }

  if (p.state_out && g == sg.G - 1) {
    float* sp = p.state_out + ((int64_t)s * Hv + h) * DK * DV + col;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[(16 * i + 4 * g4 + e) * DV] = S[i][e];
  }
}

// ============================================================================ 3b. row-split sweep
// For few (sequence, head) chains (bf16 io): one workgroup per (sequence, value head, 16 dv
// columns) with four row groups j.  Row group j keeps state rows 32 j .. 32 j + 31 of the
// 16 columns (two accumulator tiles) and owns token row tile j (tokens 16 j .. 16 j + 15)
// of the chunk's R, U and O, so it does a quarter of the column's products and hi/lo
// splits.  Per chunk, three barriers separate:
//   A  (after barrier 1): K S and Q S for row tile j from the four state slabs (exchanged
//      as ready bf16 hi/lo fragments), R = V - diag(e^g/|k|) K S;  K S takes both parts of
//      the state, and Q S too (o is small where Q S and P U cancel);
//   A2 (after barrier 2): U = T' R for row tile j from the exchanged R tiles;
//   B  (after barrier 3): O = scale (diag(e^g/|q|) Q S + P U) for row tile j and the
//      update of the row group's state slab from the exchanged U tiles.
// Operands: the K rows (double-buffered by chunk parity: they serve K S and, read
// transposed, the state update), the Q rows, the factor rows and the V slice are copied
// to LDS by DMA; T' and P fragments load from the fragment-native records straight into
// registers, one chunk ahead.  Outputs leave through an LDS tile as 16-byte rows after the
// next chunk's first barrier.  It runs where its workgroups fit the compute units once (one
// per CU); more chains, up to a second round, go to the column-chain sweep below.
// the row-split family (this sweep, or the column-chain sweep past one round) is used while
// its one-tile workgroups would fill the compute units at most this many times over
constexpr int ROWSPLIT_CU_ROUNDS = 2;
namespace rs {
constexpr int NW = 4;
constexpr int THR = 64 * NW;
constexpr int NBLK = DV / 16;            // workgroups per chain with one column tile
constexpr int ROWS = CH * KS_STRIDE;
constexpr int KJ = RowDma<16, NW>::J;    // K or Q row copies per wave
// CT 16-column tiles of dv per workgroup.  One tile is what runs: where one tile's
// workgroups would need two per CU, two tiles per workgroup run on the column-chain sweep
// instead (a CT = 2 instance of this kernel, which reads each K, Q, T' and P fragment once
// for both tiles, measured 1-4% slower than that)
template <int CT>
struct Cols {
  static constexpr int DVB = 16 * CT;           // dv columns per workgroup
  static constexpr int NBLK = DV / DVB;         // workgroups per chain
  static constexpr int VW = DVB * 2 / 16;       // 16-byte words per V row slice
  static constexpr int V_STRIDE = DVB + 8;      // u16 per staged V row
  static constexpr int O_STRIDE = DVB + 8;      // u16 per staged output row
};
}  // namespace rs

// one chunk's register operands of wave j: T' and P of row tile j, token slabs 0, 1
struct RsOps {
  bf16x8 th[2], tl[2];
  bf16x8 ph[2], pl[2];
};

// the jp-th row copy of this wave (see dma_rows), issued as OPAQUE inline assembly
template <int DW, int NW>
__device__ __forceinline__ void dma_row_piece(const uint8_t* base, uint32_t row_bytes, int L,
                                              uint32_t tab, void* dst, int wave, int jp) {
  typedef RowDma<DW, NW> R;
  const int ins = wave + NW * jp;
  if (ins >= R::INS) return;   // (wave-uniform) no copy left for this wave
  const uint32_t row = min(tab & 0xFFu, (uint32_t)(L - 1));
  lds_dma16_sbase(base, __umul24(row, row_bytes) + (tab >> 8), (char*)dst + ins * 1024);
}

// Each row group is two waves by role.  Chain waves j = 0..3 carry the recurrence: K S
// for row tile j, R, U = T' R and the update of state rows 32 j .. 32 j + 31, at a raised
// issue priority.  Output waves j = 0..3 form the chunk's output off that path: Q S for
// row tile j in phase A and P U in phase B; they also issue every LDS copy (the next
// chunk's K rows before their own LDS reads, so the chain waves' reads are served first)
// and store the output tiles.  The two roles of a row group share a SIMD, so each fills
// the other's waits.  (Measured at 9B T=4096: 130 us against 138 us with one wave per row
// group; 397B T=32768, when it still ran there at two workgroups per CU: 1.68 against
// 1.70 ms.)
namespace rs2 {
constexpr int THR = 2 * rs::THR;
}

// (CT = 1 is built for four waves per SIMD, which would let two workgroups share a CU; CT = 2
// would run one workgroup per CU, so two waves per SIMD and their registers)
template <int CT>
__global__ void __launch_bounds__(rs2::THR, CT == 1 ? 4 : 2)
chunk_rowsplit2_kernel(ChunkArgs p, const int32_t* __restrict__ cmap, const uint8_t* __restrict__ recs) {
  typedef Io<IO_BF16> io;
  typedef io::T T;
  using namespace rs;
  typedef Cols<CT> C;
  constexpr int DVB = C::DVB, NBLK = C::NBLK, VW = C::VW, V_STRIDE = C::V_STRIDE, O_STRIDE = C::O_STRIDE;
  __shared__ __attribute__((aligned(16))) u16 s_k0[ROWS];     // K rows, even chunks
  __shared__ __attribute__((aligned(16))) u16 s_k1[ROWS];     // K rows, odd chunks
  __shared__ __attribute__((aligned(16))) u16 s_q[ROWS];      // Q rows
  __shared__ __attribute__((aligned(16))) float s_f[4 * CH];    // factor rows 0 .. 3 (c_k, c_q, c_2, e^{gamma_L})
  __shared__ __attribute__((aligned(16))) u16 s_v[CH * V_STRIDE];      // V slice
  __shared__ __attribute__((aligned(16))) uint4 s_sx[CT][4][2][64];    // state slabs: hi, lo fragments
  __shared__ __attribute__((aligned(16))) uint2 s_rx[CT][4][2][64];    // R tiles: hi, lo
  __shared__ __attribute__((aligned(16))) uint2 s_ux[CT][4][4][64];    // U tiles: U hi, U lo, Us hi, Us lo
  __shared__ __attribute__((aligned(16))) u16 s_ost[CH * O_STRIDE];    // output tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wv < NW;        // wave-uniform role
  if (chain) __builtin_amdgcn_s_setprio(2);
  const int j = wv & (NW - 1);       // the wave's row group
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  // workgroup -> (sequence, value head, column block) as in the row-split sweep
  const int Hv = p.Hv, r = Hv / p.Hk;
  const int GS = r * NBLK;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int member = slot % GS;
  const int group = (slot / GS) * 8 + xcd;
  if (group >= p.Ns * p.Hk) return;
  const int blk = member % NBLK;
  const int kh = group % p.Hk;
  const int s = group / p.Hk;
  const int h = kh * r + member / NBLK;
  int64_t b0, b1;
  seq_bounds(p.cu, p.N, s, b0, b1);
  const int c0 = p.Ns == 1 ? 0 : cmap[s];
  const int ne = (int)((b1 - b0 + CH - 1) / CH);
  const int col = blk * DVB + c16;   // column tile ct: col + 16 ct

  const uint8_t* qg = (const uint8_t*)((const T*)p.q + (int64_t)kh * DK);
  const uint8_t* kg = (const uint8_t*)((const T*)p.k + (int64_t)kh * DK);
  const uint8_t* vg = (const uint8_t*)((const T*)p.v + (int64_t)h * DV + blk * DVB);
  const uint32_t qrow_bytes = (uint32_t)(p.stride_q * (int64_t)sizeof(T));
  const uint32_t krow_bytes = (uint32_t)(p.stride_k * (int64_t)sizeof(T));
  const uint32_t vrow_bytes = (uint32_t)(p.stride_v * (int64_t)sizeof(T));
  T* og0 = (T*)p.o + (int64_t)h * DV + blk * DVB;
  const int64_t o_stride = (int64_t)Hv * DV;
  uint32_t ktab[KJ], vtab[RowDma<VW, NW>::J];
  rows_table<16, NW>(j, lane, ktab);
  rows_table<VW, NW>(j, lane, vtab);

  // ---- state slab (chain waves): St[ct][t] holds rows 32 j + 16 t + 4 g4 + e of column
  // col + 16 ct
  f32x4 St[CT][2];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    St[ct][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    St[ct][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (chain && p.state_in) {
    const float* sp = p.state_in + ((int64_t)s * Hv + h) * DK * DV + col;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) St[ct][t][e] = sp[(32 * j + 16 * t + 4 * g4 + e) * DV + 16 * ct];
  }
  auto put_slab = [&]() {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      bf16x8 hi, lo;
      frag_acc_split(St[ct][0], St[ct][1], hi, lo);
      s_sx[ct][j][0][lane] = __builtin_bit_cast(uint4, hi);
      s_sx[ct][j][1][lane] = __builtin_bit_cast(uint4, lo);
    }
  };
  auto chunk_rows = [&](int n, int64_t& t0, int& L) {
    t0 = b0 + (int64_t)n * CH;
    L = (int)min((int64_t)CH, b1 - t0);
  };
  auto rec_of = [&](int n) { return recs + ((int64_t)(c0 + n) * Hv + h) * FR_REC_BYTES; };

  // chunk n's fragments of row tile j: T' for a chain wave, P for an output wave (token
  // slab 1 is zero for row tiles 0 and 1; it is loaded first, see the row-split sweep)
  auto load_ops = [&](int n, RsOps& o) {
    const uint8_t* rec = rec_of(n) + (chain ? FR_T_OFF : FR_P_OFF);
    if (j >= 2) {
      o.th[1] = *reinterpret_cast<const bf16x8*>(rec + fr_tp(j, 1, 0) + lane * 16);
      o.tl[1] = *reinterpret_cast<const bf16x8*>(rec + fr_tp(j, 1, 1) + lane * 16);
    }
    o.th[0] = *reinterpret_cast<const bf16x8*>(rec + fr_tp(j, 0, 0) + lane * 16);
    o.tl[0] = *reinterpret_cast<const bf16x8*>(rec + fr_tp(j, 0, 1) + lane * 16);
  };
  // (output waves) copies of chunk n's Q rows, factor rows and V slice
  auto stage_qfv = [&](int n) {
    int64_t t0;
    int L;
    chunk_rows(n, t0, L);
#pragma unroll
    for (int jp = 0; jp < KJ; ++jp)
      dma_row_piece<16, NW>(qg + t0 * qrow_bytes, qrow_bytes, L, ktab[jp], s_q, j, jp);
    if (j == 0)   // factor rows 0 .. 3 (the rest serve the other sweeps)
      lds_dma16_sbase(rec_of(n) + FR_FAC_OFF, lane * 16, (char*)s_f);
#pragma unroll
    for (int jp = 0; jp < RowDma<VW, NW>::J; ++jp)
      dma_row_piece<VW, NW>(vg + t0 * vrow_bytes, vrow_bytes, L, vtab[jp], s_v, j, jp);
  };
  // (output waves) rows of the output tile of chunk n to global memory
  auto store_o = [&](int n) {
    int64_t t0;
    int L;
    chunk_rows(n, t0, L);
    constexpr int WPR = DVB / 8;
    const int ot = tid - THR;
    if (ot < CH * WPR) {
      const int row = ot / WPR, w = ot % WPR;
      if (row < L)
        *reinterpret_cast<uint4*>(og0 + (t0 + row) * o_stride + w * 8) =
            *reinterpret_cast<const uint4*>(&s_ost[row * O_STRIDE + w * 8]);
    }
  };

  // RsOps th/tl hold T' (chain waves) or P (output waves)
  RsOps oa, ob;
  if (ne > 0) {
    if (!chain) {
      int64_t t0;
      int L;
      chunk_rows(0, t0, L);
#pragma unroll
      for (int jp = 0; jp < KJ; ++jp)
        dma_row_piece<16, NW>(kg + t0 * krow_bytes, krow_bytes, L, ktab[jp], s_k0, j, jp);
      stage_qfv(0);
    }
    load_ops(0, oa);
  }
  if (chain) put_slab();

  auto chunk = [&](int n, const RsOps& cur, RsOps& nxt, auto par) {
    constexpr int PAR = decltype(par)::value;
    const u16* const kcur = PAR ? s_k1 : s_k0;
    u16* const knext = PAR ? s_k0 : s_k1;
    const int na = n + 1 < ne ? n + 1 : n;   // the last chunk reloads its own (unused)

    wait_vmem();
    lds_barrier();     // (1) chunk n's copies and the state slabs are in LDS
    // chunk n+1's fragments of this wave's role, a whole chunk ahead of the wait at the next
    // barrier (1): the previous contents of nxt were last read in chunk n-1
    load_ops(na, nxt);
    if (!chain && n > 0) store_o(n - 1);

    f32x4 QS[CT];      // output waves: Q S of row tile j
    float4 c2;         // chain waves: the update factors of row tile j
    float egl;
    if (chain) {
      // ---- A (chain): K S for row tile j, R = V - diag(e^g/|k|) K S
      const float4 ck = *reinterpret_cast<const float4*>(&s_f[16 * j + 4 * g4]);
      c2 = *reinterpret_cast<const float4*>(&s_f[2 * CH + 16 * j + 4 * g4]);
      egl = s_f[3 * CH];
      u16 vraw[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) vraw[ct][e] = s_v[(16 * j + 4 * g4 + e) * V_STRIDE + 16 * ct + c16];
      f32x4 ka[CT], kb[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        ka[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        kb[ct] = ka[ct];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 ak = frag_rows(kcur, KS_STRIDE, 16 * j, 32 * m, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const bf16x8 sh = __builtin_bit_cast(bf16x8, s_sx[ct][m][0][lane]);
          const bf16x8 sl = __builtin_bit_cast(bf16x8, s_sx[ct][m][1][lane]);
          ka[ct] = mma(ak, sh, ka[ct]);
          kb[ct] = mma(ak, sl, kb[ct]);
        }
      }
      const float ckv[4] = {ck.x, ck.y, ck.z, ck.w};
      int64_t t0;
      int L;
      chunk_rows(n, t0, L);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 R;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * j + 4 * g4 + e;
          const float vv = t < L ? bf2f(vraw[ct][e]) : 0.f;
          R[e] = vv - ckv[e] * (ka[ct][e] + kb[ct][e]);
        }
        uint32_t rh0, rl0, rh1, rl1;
        split2(R[0], R[1], rh0, rl0);
        split2(R[2], R[3], rh1, rl1);
        s_rx[ct][j][0][lane] = make_uint2(rh0, rh1);
        s_rx[ct][j][1][lane] = make_uint2(rl0, rl1);
      }
    } else {
      // ---- A (output): Q S for row tile j; chunk n+1's K rows copied between the products
      int64_t ta;
      int La;
      chunk_rows(na, ta, La);
      const uint8_t* kga = kg + ta * krow_bytes;
      const float4 cq = *reinterpret_cast<const float4*>(&s_f[CH + 16 * j + 4 * g4]);
      // the copies go out first, so that the chain waves' LDS reads are served alone
#pragma unroll
      for (int jp = 0; jp < KJ; ++jp) dma_row_piece<16, NW>(kga, krow_bytes, La, ktab[jp], knext, j, jp);
      f32x4 qa[CT], qb[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        qa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        qb[ct] = qa[ct];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 aq = frag_rows(s_q, KS_STRIDE, 16 * j, 32 * m, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const bf16x8 sh = __builtin_bit_cast(bf16x8, s_sx[ct][m][0][lane]);
          const bf16x8 sl = __builtin_bit_cast(bf16x8, s_sx[ct][m][1][lane]);
          qa[ct] = mma(aq, sh, qa[ct]);
          qb[ct] = mma(aq, sl, qb[ct]);
        }
      }
      const float cqv[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) QS[ct][e] = cqv[e] * (qa[ct][e] + qb[ct][e]);
    }
    lds_barrier();     // (2) R tiles exchanged; every wave has read the slabs, Q, factors, V
    if (chain) {
      // ---- A2 (chain): U = T' R for row tile j
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x8 rh = pack8(s_rx[ct][0][0][lane], s_rx[ct][1][0][lane]);
        const bf16x8 rl = pack8(s_rx[ct][0][1][lane], s_rx[ct][1][1][lane]);
        bf16x8 rh1 = pack8(s_rx[ct][2][0][lane], s_rx[ct][3][0][lane]);
        bf16x8 rl1 = pack8(s_rx[ct][2][1][lane], s_rx[ct][3][1][lane]);
        asm volatile("" : "+v"(rh1), "+v"(rl1));   // keeps the reads out of the branch below
        f32x4 ua = mma(cur.th[0], rh, f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 ub = mma(cur.tl[0], rh, f32x4{0.f, 0.f, 0.f, 0.f});
        ua = mma(cur.th[0], rl, ua);
        if (j >= 2) {
          ub = mma(cur.th[1], rh1, ub);
          ua = mma(cur.tl[1], rh1, ua);
          ub = mma(cur.th[1], rl1, ub);
        }
        const f32x4 U = ua + ub;
        uint32_t uh0, ul0, uh1, ul1, wh0, wl0, wh1, wl1;
        split2(U[0], U[1], uh0, ul0);
        split2(U[2], U[3], uh1, ul1);
        split2(c2.x * U[0], c2.y * U[1], wh0, wl0);
        split2(c2.z * U[2], c2.w * U[3], wh1, wl1);
        s_ux[ct][j][0][lane] = make_uint2(uh0, uh1);
        s_ux[ct][j][1][lane] = make_uint2(ul0, ul1);
        s_ux[ct][j][2][lane] = make_uint2(wh0, wh1);
        s_ux[ct][j][3][lane] = make_uint2(wl0, wl1);
      }
    } else {
      stage_qfv(na);
    }
    lds_barrier();     // (3) U tiles exchanged; every wave has read the R tiles

    if (chain) {
      // ---- B (chain): S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma} / |k|) U for
      // state rows 32 j .. 32 j + 31, K^T read transposed from this chunk's K rows
      bf16x8 ak[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m) ak[t][m] = frag_kt(kcur, 32 * j + 16 * t, 32 * m, lane);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        bf16x8 wh[2], wl[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          wh[m] = pack8(s_ux[ct][2 * m][2][lane], s_ux[ct][2 * m + 1][2][lane]);
          wl[m] = pack8(s_ux[ct][2 * m][3][lane], s_ux[ct][2 * m + 1][3][lane]);
        }
        f32x4 sb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int e = 0; e < 4; ++e) St[ct][t][e] *= egl;
          sb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            St[ct][t] = mma(ak[t][m], wh[m], St[ct][t]);
            sb[t] = mma(ak[t][m], wl[m], sb[t]);
          }
        St[ct][0] += sb[0];
        St[ct][1] += sb[1];
      }
      put_slab();
    } else {
      // ---- B (output): O = scale (Q S + P U) for row tile j, to the LDS output tile
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x8 uh = pack8(s_ux[ct][0][0][lane], s_ux[ct][1][0][lane]);
        const bf16x8 ul = pack8(s_ux[ct][0][1][lane], s_ux[ct][1][1][lane]);
        bf16x8 uh1 = pack8(s_ux[ct][2][0][lane], s_ux[ct][3][0][lane]);
        bf16x8 ul1 = pack8(s_ux[ct][2][1][lane], s_ux[ct][3][1][lane]);
        asm volatile("" : "+v"(uh1), "+v"(ul1));   // keeps the reads out of the branch below
        f32x4 pa = mma(cur.th[0], uh, f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 pb = mma(cur.tl[0], uh, f32x4{0.f, 0.f, 0.f, 0.f});
        pa = mma(cur.th[0], ul, pa);
        if (j >= 2) {
          pb = mma(cur.th[1], uh1, pb);
          pa = mma(cur.tl[1], uh1, pa);
          pb = mma(cur.th[1], ul1, pb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s_ost[(16 * j + 4 * g4 + e) * O_STRIDE + 16 * ct + c16] =
              f2bf(p.scale * (QS[ct][e] + pa[e] + pb[e]));
      }
    }
  };
  for (int n = 0; n < ne; n += 2) {
    chunk(n, oa, ob, std::integral_constant<int, 0>());
    if (n + 1 < ne) chunk(n + 1, ob, oa, std::integral_constant<int, 1>());
  }
  wait_vmem();         // no copy is in flight when the workgroup ends
  if (ne > 0) {
    lds_barrier();     // the last chunk's output tile is complete
    if (!chain) store_o(ne - 1);
  }
  if (chain && p.state_out) {
    float* sp = p.state_out + ((int64_t)s * Hv + h) * DK * DV + col;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[(32 * j + 16 * t + 4 * g4 + e) * DV + 16 * ct] = St[ct][t][e];
  }
}

// ============================================================================ 3c. column-chain sweep
// bf16 io, one sequence-head chain's 128 dv columns over 128 / (16 CT) workgroups, one
// workgroup per CU.  Each 16-column tile has two waves:
//   chain wave: keeps the tile's whole 128 x 16 state slice in registers (eight accumulator
//     tiles, tile t = state rows 16 t .. 16 t + 15) and walks the chunks: K S for the four
//     token tiles, R = V - diag(c_k) K S, U = T' R, S <- e^{gamma_L} S + K^T diag(c_2) U.
//     Every product's accumulator is the next one's B operand, so nothing is exchanged
//     inside a chunk; the chunk's start state (as bf16 hi/lo fragments) and U (fp32) are
//     left in LDS.
//   output wave: forms chunk n-1's output O = scale (diag(c_q) Q S + P U) from what the
//     chain wave left while that wave walks chunk n, storing it through an LDS tile as
//     16-byte rows; the output waves also copy chunk n+1's K, V, factor and Q rows into LDS
//     (the first one K, V and the factors, the last one Q).
// The waves of a workgroup each run on their own SIMD, and the tiles of a workgroup share
// the staged rows.  One barrier per chunk, where the chain waves end it.  K and V rows are
// double-buffered by chunk parity; Q and factor rows, read one chunk later by the output
// waves, by chunk mod 3; the handed-over state and U by parity.  T' (chain) and P (output)
// fragments go straight from the fragment-native records to registers, a chunk ahead.
namespace cc {
constexpr int ROWS = CH * KS_STRIDE;      // u16 per staged K or Q chunk
constexpr int KJ = RowDma<16, 1>::J;      // K or Q row copies per chunk
constexpr int O_STRIDE = 16 + 8;          // u16 per staged output row of a tile
// fragment index of (row tile j, token slab m) in the lower-triangular T' / P operands
__device__ __forceinline__ constexpr int fi(int j, int m) { return j < 2 ? j : 2 * j - 2 + m; }
template <int CT>
struct Cfg {
  static constexpr int THR = 128 * CT;          // CT chain waves, then CT output waves
  static constexpr int DVB = 16 * CT;           // dv columns per workgroup
  static constexpr int NBLK = DV / DVB;         // workgroups per chain
  static constexpr int VW = DVB * 2 / 16;       // 16-byte words per V row slice
  static constexpr int V_STRIDE = DVB + 8;      // u16 per staged V row (pad: one more word)
  static constexpr int VJ = RowDma<VW, 1>::J;   // V row copies per chunk
};
}  // namespace cc

template <int CT>
__global__ void __launch_bounds__(cc::Cfg<CT>::THR, 1)
chunk_colchain_kernel(ChunkArgs p, const int32_t* __restrict__ cmap, const uint8_t* __restrict__ recs) {
  typedef Io<IO_BF16>::T T;
  using namespace cc;
  typedef Cfg<CT> C;
  constexpr int DVB = C::DVB, NBLK = C::NBLK, VW = C::VW, V_STRIDE = C::V_STRIDE, VJ = C::VJ;
  __shared__ __attribute__((aligned(16))) u16 s_k[2][ROWS];             // K rows, by chunk parity
  __shared__ __attribute__((aligned(16))) u16 s_q[3][ROWS];             // Q rows, by chunk mod 3
  __shared__ __attribute__((aligned(16))) u16 s_v[2][CH * V_STRIDE];    // V slice, by parity
  __shared__ __attribute__((aligned(16))) float s_f[3][4 * CH];         // c_k, c_q, c_2, e^{gamma_L}
  __shared__ __attribute__((aligned(16))) uint4 s_sx[2][CT][4][2][64];  // start state: slab, hi/lo
  __shared__ __attribute__((aligned(16))) float4 s_u[2][CT][4][64];     // U tiles (fp32)
  __shared__ __attribute__((aligned(16))) u16 s_ost[CT][CH * O_STRIDE]; // output tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wv < CT;          // wave-uniform role
  const int ct = chain ? wv : wv - CT; // the wave's column tile
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  // workgroup -> (sequence, value head, column block): the r * NBLK workgroups of a key
  // head are consecutive in blockIdx / 8 (they read the same K and Q rows)
  const int Hv = p.Hv, r = Hv / p.Hk;
  const int GS = r * NBLK;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int member = slot % GS;
  const int group = (slot / GS) * 8 + xcd;
  if (group >= p.Ns * p.Hk) return;
  const int blk = member % NBLK;
  const int kh = group % p.Hk;
  const int s = group / p.Hk;
  const int h = kh * r + member / NBLK;
  int64_t b0, b1;
  seq_bounds(p.cu, p.N, s, b0, b1);
  const int c0 = p.Ns == 1 ? 0 : cmap[s];
  const int ne = (int)((b1 - b0 + CH - 1) / CH);
  const int col = blk * DVB + 16 * ct + c16;

  auto chunk_rows = [&](int n, int64_t& t0, int& L) {
    t0 = b0 + (int64_t)n * CH;
    L = (int)min((int64_t)CH, b1 - t0);
  };
  auto rec_of = [&](int n) { return recs + ((int64_t)(c0 + n) * Hv + h) * FR_REC_BYTES; };
  // chunk n's six lower-triangular fragments (hi, lo) of T' (chain wave) or P (output wave)
  auto load_frags = [&](int n, bf16x8 (&fh)[6], bf16x8 (&fl)[6]) {
    const uint8_t* rec = rec_of(n) + (chain ? FR_T_OFF : FR_P_OFF) + lane * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int m = 0; m < (j < 2 ? 1 : 2); ++m) {
        fh[fi(j, m)] = *reinterpret_cast<const bf16x8*>(rec + fr_tp(j, m, 0));
        fl[fi(j, m)] = *reinterpret_cast<const bf16x8*>(rec + fr_tp(j, m, 1));
      }
  };
  // Y = M X for a lower-triangular M given by its fragments and X by the B operands of its
  // two token slabs (hi, lo): three passes (Mh Xh, Ml Xh, Mh Xl)
  auto tri = [&](const bf16x8 (&mh)[6], const bf16x8 (&ml)[6], const bf16x8 (&xh)[2],
                 const bf16x8 (&xl)[2], f32x4 (&y)[4]) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 y2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = mma(mh[fi(j, 0)], xh[0], z);
#pragma unroll
    for (int j = 2; j < 4; ++j) y2[j - 2] = mma(mh[fi(j, 1)], xh[1], z);
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = mma(ml[fi(j, 0)], xh[0], y[j]);
#pragma unroll
    for (int j = 2; j < 4; ++j) y2[j - 2] = mma(ml[fi(j, 1)], xh[1], y2[j - 2]);
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = mma(mh[fi(j, 0)], xl[0], y[j]);
#pragma unroll
    for (int j = 2; j < 4; ++j) y2[j - 2] = mma(mh[fi(j, 1)], xl[1], y2[j - 2]);
    y[2] += y2[0];
    y[3] += y2[1];
  };

  if (chain) {
    // ------------------------------------------------------------------ chain wave
    f32x4 St[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) St[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.state_in) {
      const float* sp = p.state_in + ((int64_t)s * Hv + h) * DK * DV + col;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) St[t][e] = sp[(16 * t + 4 * g4 + e) * DV];
    }
    bf16x8 th[6], tl[6];
    if (ne > 0) load_frags(0, th, tl);
    bf16x8 sh[4], sl[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) frag_acc_split(St[2 * m], St[2 * m + 1], sh[m], sl[m]);
    lds_barrier();   // chunk 0's rows are in LDS

    auto chunk = [&](int n, auto par) {
      constexpr int PAR = decltype(par)::value;
      const u16* kc = s_k[PAR];
      const float* f = s_f[n % 3];
      // K S for token tiles 0 .. 3; every K fragment, the V slice and the factors are read
      // up front (no read sits under a condition, which would wait for it in place)
      bf16x8 ak[4][4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) ak[m][i] = frag_rows(kc, KS_STRIDE, 16 * i, 32 * m, lane);
      u16 vraw[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vraw[i][e] = s_v[PAR][(16 * i + 4 * g4 + e) * V_STRIDE + 16 * ct + c16];
      float4 ck[4], c2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ck[i] = *reinterpret_cast<const float4*>(&f[16 * i + 4 * g4]);
        c2[i] = *reinterpret_cast<const float4*>(&f[2 * CH + 16 * i + 4 * g4]);
      }
      const float egl = f[3 * CH];
      f32x4 ks[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ks[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ks[i] = mma(ak[m][i], sh[m], ks[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) ks[i] = mma(ak[m][i], sl[m], ks[i]);
      }
      // the chunk's start state for the output wave, written once the K S reads are out
      // (the output wave reads it after this chunk's barrier)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        s_sx[PAR][ct][m][0][lane] = __builtin_bit_cast(uint4, sh[m]);
        s_sx[PAR][ct][m][1][lane] = __builtin_bit_cast(uint4, sl[m]);
      }
      // the update's K^T fragments, read while R and U are formed
      bf16x8 kt[2][8];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 8; ++t) kt[m][t] = frag_kt(kc, 16 * t, 32 * m, lane);
      // R = V - diag(e^gamma / |k|) K S (rows past the chunk end are zero)
      int64_t t0;
      int L;
      chunk_rows(n, t0, L);
      f32x4 R[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ckv[4] = {ck[i].x, ck[i].y, ck[i].z, ck[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * i + 4 * g4 + e;
          const float vv = t < L ? bf2f(vraw[i][e]) : 0.f;
          R[i][e] = vv - ckv[e] * ks[i][e];
        }
      }
      bf16x8 rh[2], rl[2];
      frag_acc_split(R[0], R[1], rh[0], rl[0]);
      frag_acc_split(R[2], R[3], rh[1], rl[1]);
      // U = T' R
      f32x4 U[4];
      tri(th, tl, rh, rl, U);
      // the next chunk's T' (this chunk's is dead), a chunk ahead of its use; the last
      // chunk reloads its own
      load_frags(n + 1 < ne ? n + 1 : n, th, tl);
#pragma unroll
      for (int i = 0; i < 4; ++i) s_u[PAR][ct][i][lane] = __builtin_bit_cast(float4, U[i]);
      // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma} / |k|) U
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        U[i][0] *= c2[i].x;
        U[i][1] *= c2[i].y;
        U[i][2] *= c2[i].z;
        U[i][3] *= c2[i].w;
      }
      bf16x8 wh[2], wl[2];
      frag_acc_split(U[0], U[1], wh[0], wl[0]);
      frag_acc_split(U[2], U[3], wh[1], wl[1]);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) St[t][e] *= egl;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int t = 0; t < 8; ++t) St[t] = mma(kt[m][t], wh[m], St[t]);
#pragma unroll
        for (int t = 0; t < 8; ++t) St[t] = mma(kt[m][t], wl[m], St[t]);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) frag_acc_split(St[2 * m], St[2 * m + 1], sh[m], sl[m]);
      lds_barrier();   // this chunk's hand-over is in LDS; the next chunk's rows are too
    };
    for (int n = 0; n < ne; n += 2) {
      chunk(n, std::integral_constant<int, 0>());
      if (n + 1 < ne) chunk(n + 1, std::integral_constant<int, 1>());
    }
    if (p.state_out) {
      float* sp = p.state_out + ((int64_t)s * Hv + h) * DK * DV + col;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[(16 * t + 4 * g4 + e) * DV] = St[t][e];
    }
    return;
  }

  // -------------------------------------------------------------------- output wave
  const uint8_t* qg = (const uint8_t*)((const T*)p.q + (int64_t)kh * DK);
  const uint8_t* kg = (const uint8_t*)((const T*)p.k + (int64_t)kh * DK);
  const uint8_t* vg = (const uint8_t*)((const T*)p.v + (int64_t)h * DV + blk * DVB);
  const uint32_t qrow_bytes = (uint32_t)(p.stride_q * (int64_t)sizeof(T));
  const uint32_t krow_bytes = (uint32_t)(p.stride_k * (int64_t)sizeof(T));
  const uint32_t vrow_bytes = (uint32_t)(p.stride_v * (int64_t)sizeof(T));
  T* og0 = (T*)p.o + (int64_t)h * DV + blk * DVB + 16 * ct;
  const int64_t o_stride = (int64_t)Hv * DV;
  uint32_t ktab[KJ], vtab[VJ];
  rows_table<16, 1>(0, lane, ktab);
  rows_table<VW, 1>(0, lane, vtab);

  // chunk n's rows into LDS (PAR = n & 1): K, V and the factors by the first output wave,
  // Q by the last
  auto stage = [&](int n, auto par) {
    constexpr int PAR = decltype(par)::value;
    int64_t t0;
    int L;
    chunk_rows(n, t0, L);
    if (ct == 0) {
#pragma unroll
      for (int jp = 0; jp < KJ; ++jp)
        dma_row_piece<16, 1>(kg + t0 * krow_bytes, krow_bytes, L, ktab[jp], s_k[PAR], 0, jp);
#pragma unroll
      for (int jp = 0; jp < VJ; ++jp)
        dma_row_piece<VW, 1>(vg + t0 * vrow_bytes, vrow_bytes, L, vtab[jp], s_v[PAR], 0, jp);
      lds_dma16_sbase(rec_of(n) + FR_FAC_OFF, lane * 16, (char*)s_f[n % 3]);
    }
    if (ct == CT - 1) {
#pragma unroll
      for (int jp = 0; jp < KJ; ++jp)
        dma_row_piece<16, 1>(qg + t0 * qrow_bytes, qrow_bytes, L, ktab[jp], s_q[n % 3], 0, jp);
    }
  };
  // chunk n's output from the chain wave's hand-over (PAR = n & 1) and P
  auto output = [&](int n, auto par, const bf16x8 (&ph)[6], const bf16x8 (&pl)[6]) {
    constexpr int PAR = decltype(par)::value;
    const u16* qc = s_q[n % 3];
    const float* f = s_f[n % 3];
    u16* ost = s_ost[ct];
    bf16x8 sh[4], sl[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      sh[m] = __builtin_bit_cast(bf16x8, s_sx[PAR][ct][m][0][lane]);
      sl[m] = __builtin_bit_cast(bf16x8, s_sx[PAR][ct][m][1][lane]);
    }
    f32x4 qs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bf16x8 aq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) aq[i] = frag_rows(qc, KS_STRIDE, 16 * i, 32 * m, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[i] = mma(aq[i], sh[m], qs[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[i] = mma(aq[i], sl[m], qs[i]);
    }
    f32x4 U[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) U[i] = __builtin_bit_cast(f32x4, s_u[PAR][ct][i][lane]);
    bf16x8 uh[2], ul[2];
    frag_acc_split(U[0], U[1], uh[0], ul[0]);
    frag_acc_split(U[2], U[3], uh[1], ul[1]);
    f32x4 pu[4];
    tri(ph, pl, uh, ul, pu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 cq = *reinterpret_cast<const float4*>(&f[CH + 16 * i + 4 * g4]);
      const float cqv[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ost[(16 * i + 4 * g4 + e) * O_STRIDE + c16] = f2bf(p.scale * (cqv[e] * qs[i][e] + pu[i][e]));
    }
    int64_t t0;
    int L;
    chunk_rows(n, t0, L);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int sl2 = lane + 64 * k, row = sl2 >> 1, w = sl2 & 1;
      const uint4 ov = *reinterpret_cast<const uint4*>(&ost[row * O_STRIDE + 8 * w]);
      if (row < L) *reinterpret_cast<uint4*>(og0 + (t0 + row) * o_stride + 8 * w) = ov;
    }
  };

  bf16x8 pah[6], pal[6], pbh[6], pbl[6];   // P of even and odd chunks
  if (ne > 0) {
    stage(0, std::integral_constant<int, 0>());
    load_frags(0, pah, pal);
  }
  wait_vmem();
  lds_barrier();
  // interval n (between the chain waves' barriers n-1 and n): stage chunk n+1, load P of
  // chunk n, form chunk n-1's output
  auto interval = [&](int n, auto par) {
    constexpr int PAR = decltype(par)::value;
    if (n + 1 < ne) stage(n + 1, std::integral_constant<int, 1 - PAR>());
    if constexpr (PAR == 0) {
      if (n > 0) load_frags(n, pah, pal);
      if (n > 0) output(n - 1, std::integral_constant<int, 1>(), pbh, pbl);
    } else {
      load_frags(n, pbh, pbl);
      output(n - 1, std::integral_constant<int, 0>(), pah, pal);
    }
    wait_vmem();
    // every P load is complete here; redefining the registers tells the compiler so (it
    // does not count the copies above, and would otherwise wait for them when P is used)
#pragma unroll
    for (int i = 0; i < 6; ++i) asm volatile("" : "+v"(pah[i]), "+v"(pal[i]), "+v"(pbh[i]), "+v"(pbl[i]));
    lds_barrier();
  };
  for (int n = 0; n < ne; n += 2) {
    interval(n, std::integral_constant<int, 0>());
    if (n + 1 < ne) interval(n + 1, std::integral_constant<int, 1>());
  }
  if (ne > 0) {
    if ((ne - 1) & 1)
      output(ne - 1, std::integral_constant<int, 1>(), pbh, pbl);
    else
      output(ne - 1, std::integral_constant<int, 0>(), pah, pal);
  }
}

template <int IO>
static hipError_t chunk_impl(const ChunkArgs& a, void* ws, hipStream_t st) {
  const int64_t cmax = ws_max_chunks(a.N, a.Ns);
  int32_t* cmap = reinterpret_cast<int32_t*>(ws);
  int4* cinfo = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(ws) + ws_cmap_bytes(a.Ns));
  uint8_t* recs = reinterpret_cast<uint8_t*>(ws) + ws_map_bytes(a.N, a.Ns);
  uint8_t* krecs = recs + cmax * a.Hv * ws_rec_bytes(true);
  float* segs = reinterpret_cast<float*>(krecs + cmax * a.Hk * ws_krec_bytes(IO == IO_F32));
  // launch shapes (see below): the normal sweep runs 4-wave workgroups, with P in the
  // records, or 8-wave ones, which form P themselves
  const int64_t pairs = (int64_t)a.Ns * a.Hv;
  const int64_t cus = a.cu_count > 0 ? a.cu_count : 256;
  // bf16 io with few, long chains whose row-split launch would fill at most half the
  // compute units: the intra-sequence scan (see SEG_BF16_MAX_CHAINS)
  const bool bf16_seg = IO == IO_BF16 && bf16_seg_shape(a.N, a.Ns, a.Hv) &&
                        2 * pairs * rs::NBLK <= cus && seg_count(a.N, a.Ns, a.Hv, cus) >= 3;
  // bf16 io with few chains otherwise: the row-split sweep (eight 8-wave workgroups per chain)
  const bool rowsplit = IO == IO_BF16 && !bf16_seg && pairs * rs::NBLK <= ROWSPLIT_CU_ROUNDS * cus;
  // (segment scratch is in the workspace for fp32 io with few chains and for the bf16 scan)
  const int G = (IO == IO_F32 || bf16_seg) ? seg_count(a.N, a.Ns, a.Hv, cus) : 1;
  const bool four = rowsplit || pairs * G * SweepSizes<IO, 4>::NBLK <= cus;
  // the chunk map of packed sequences (one sequence needs none: its chunks are in order)
  hipError_t e = hipSuccess;
  if (a.Ns > 1) {
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, st, a.cu, a.Ns, a.N, cmax, cmap,
                       cinfo);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // fused conv: bf16 io forms it inside the prep kernel while the prep's workgroups fit
  // on the chip at once.  Then the conv's HBM traffic is spread over one round with
  // nothing else to wait for; over several rounds the conv rows lengthen every
  // workgroup's critical path and the conv kernel ahead of the prep is faster (measured:
  // 9B T=4096, 1024 workgroups in one round, 56 us fused against 64 us as two kernels;
  // 397B T=32768, eight rounds, 658 us against 587 us).  fp32 io always runs the conv
  // kernel first.
  // (the prep's working workgroups: at most one chunk more per sequence boundary than
  // the tokens fill; the grid's spare rows return at once)
  // (bf16 io: fragment-native records, with P where the sweep reads P from them)
  const int prep_mode = IO == IO_BF16 ? ((rowsplit || four) ? PREP_FRAG : PREP_FRAG_T)
                                      : (four ? PREP_ROWS_P : PREP_ROWS);
  const int64_t chunks = (a.N + CH - 1) / CH + a.Ns - 1;
  // the call includes the conv: x given, or (no tokens, x may then be NULL) a final conv
  // state to write, which is then the initial one
  const bool conv = a.x != nullptr || a.conv_state_out != nullptr;
  const bool conv_in_prep = conv && IO == IO_BF16 &&
                            chunks * a.Hk <= (int64_t)prep_occupancy(IO, prep_mode) * cus;
  if (conv && !conv_in_prep) {
    const ConvArgs ca{a.x, a.conv_w, a.y, a.cu, a.Ns, a.N, a.Cq, a.conv_state_in, a.conv_state_out};
    e = launch_conv1d(ca, IO, st);
    if (e != hipSuccess) return e;
  }
  if (a.N > 0) {
    const dim3 pgrid((unsigned)cmax, (unsigned)a.Hk);
    if constexpr (IO == IO_BF16) {
      if (conv_in_prep && prep_mode == PREP_FRAG)
        hipLaunchKernelGGL((chunk_prep_kernel<IO, PREP_FRAG, CONV_ALL>), pgrid, dim3(NTHR), 0, st,
                           a, (const int4*)cinfo, recs, krecs);
      else if (conv_in_prep)
        hipLaunchKernelGGL((chunk_prep_kernel<IO, PREP_FRAG_T, CONV_ALL>), pgrid, dim3(NTHR), 0, st,
                           a, (const int4*)cinfo, recs, krecs);
      else if (prep_mode == PREP_FRAG)
        hipLaunchKernelGGL((chunk_prep_kernel<IO, PREP_FRAG>), pgrid, dim3(NTHR), 0, st, a,
                           (const int4*)cinfo, recs, krecs);
      else
        hipLaunchKernelGGL((chunk_prep_kernel<IO, PREP_FRAG_T>), pgrid, dim3(NTHR), 0, st, a,
                           (const int4*)cinfo, recs, krecs);
    } else if (four) {
      hipLaunchKernelGGL((chunk_prep_kernel<IO, PREP_ROWS_P>), pgrid, dim3(NTHR), 0, st, a,
                         (const int4*)cinfo, recs, krecs);
    } else {
      hipLaunchKernelGGL((chunk_prep_kernel<IO, PREP_ROWS>), pgrid, dim3(NTHR), 0, st, a,
                         (const int4*)cinfo, recs, krecs);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (conv_in_prep && a.conv_state_out && !a.conv_state_in_prep) {
    // the final conv state, after every prep workgroup has read conv_state_in (the two
    // may alias)
    const ConvArgs ca{a.x, a.conv_w, a.y, a.cu, a.Ns, a.N, a.Cq, a.conv_state_in, a.conv_state_out};
    e = launch_conv_state(ca, IO, st);
    if (e != hipSuccess) return e;
  }
  // Each (sequence, head) chain is sequential over its chunks.  While two 4-wave
  // workgroups per chain (64 dv columns each, one wave per SIMD) fit on the chip
  // at once, they give the shortest chain; beyond that one 8-wave workgroup per
  // chain (two waves per SIMD, operands staged once for all 128 columns) gives
  // the higher throughput.  With few chains and long sequences, each chain also
  // splits into G segments (the intra-sequence scan): a transition launch and a
  // normal launch, each filling the compute units.
  // grid of a sweep launch: groups (sequence, key head, segment) padded to a multiple of 8,
  // times the members of a group (value heads of the key head x column blocks)
  auto grid = [&](int segs_in_launch, int nb) {
    const int64_t groups = (int64_t)a.Ns * a.Hk * segs_in_launch;
    return dim3((unsigned)((groups + 7) / 8 * 8 * (a.Hv / a.Hk) * nb));
  };
  // record stride of the sweep launches: bf16 io fragment-native with P (4-wave and
  // transition launches) or without (8-wave), fp32 rows with P (4-wave) or without
  const int64_t rb = IO == IO_BF16 ? (four ? FR_REC_BYTES : FRT_REC_BYTES) : ws_rec_bytes(four);
  if (rowsplit) {
    const int64_t groups = (int64_t)a.Ns * a.Hk;
    // two column tiles per workgroup (the column-chain sweep) where one tile's row-split
    // workgroups would need two per CU
    const bool ct2 = pairs * rs::NBLK > cus;
    const int nblk = ct2 ? cc::Cfg<2>::NBLK : rs::NBLK;
    const dim3 grid((unsigned)((groups + 7) / 8 * 8 * (a.Hv / a.Hk) * nblk));
    if (ct2)
      hipLaunchKernelGGL(chunk_colchain_kernel<2>, grid, dim3(cc::Cfg<2>::THR), 0, st, a,
                         (const int32_t*)cmap, (const uint8_t*)recs);
    else
      hipLaunchKernelGGL(chunk_rowsplit2_kernel<1>, grid, dim3(rs2::THR), 0, st, a,
                         (const int32_t*)cmap, (const uint8_t*)recs);
    return hipGetLastError();
  }
  SegArgs sg{G, 0, G, segs, rb};
  if (G > 1) {
    SegArgs tr{G, 0, G - 1, segs, rb};
    hipLaunchKernelGGL((chunk_sweep_kernel<IO, 8, true>), grid(G - 1, 2 * SweepSizes<IO, 8>::NBLK),
                       dim3(SweepSizes<IO, 8>::THR), 0, st, a, (const int32_t*)cmap,
                       (const uint8_t*)recs, (const uint8_t*)krecs, tr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (four)
    hipLaunchKernelGGL((chunk_sweep_kernel<IO, 4, false>), grid(G, SweepSizes<IO, 4>::NBLK),
                       dim3(SweepSizes<IO, 4>::THR), 0, st, a, (const int32_t*)cmap,
                       (const uint8_t*)recs, (const uint8_t*)krecs, sg);
  else
    hipLaunchKernelGGL((chunk_sweep_kernel<IO, 8, false>), grid(G, SweepSizes<IO, 8>::NBLK),
                       dim3(SweepSizes<IO, 8>::THR), 0, st, a, (const int32_t*)cmap,
                       (const uint8_t*)recs, (const uint8_t*)krecs, sg);
  return hipGetLastError();
}

hipError_t launch_chunk_prefill(const ChunkArgs& a, void* ws, int io, hipStream_t s) {
  hipError_t e = io == IO_BF16 ? chunk_impl<IO_BF16>(a, ws, s) : chunk_impl<IO_F32>(a, ws, s);
  if (e != hipSuccess || a.yn == nullptr) return e;
  // the gated norm of the stored core output, as its own kernel: fused into the output
  // stores of the sweep it measured slower than this separate pass over o and z
  const NormArgs na{a.o, a.z, a.norm_w, a.yn, a.N * a.Hv, a.eps};
  return launch_gated_rmsnorm(na, io, s);
}

}  // namespace gdn
