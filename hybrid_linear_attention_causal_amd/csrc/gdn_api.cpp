// C ABI of libgdn (declared in include/gdn.h): argument checks on the host,
// a one-time gfx950 check per device, then kernel launches on the caller's
// stream.  Nothing here allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

thread_local char g_err[512] = "";

gdn_status_t fail(gdn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status_t hip_fail(hipError_t e, const char* what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDev = 64;
std::mutex g_arch_mu;
int g_arch_ok[kMaxDev];  // 0 unknown, 1 gfx950, -1 other
int g_cus[kMaxDev];      // compute units of each checked device

// The kernels are written for gfx950 only: refuse any other device.  cus (optional)
// receives the current device's compute-unit count.
gdn_status_t check_device(int* cus = nullptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(GDN_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    g_arch_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_cus[dev] = prop.multiProcessorCount;
    if (g_arch_ok[dev] < 0) {
      return fail(GDN_ERR_UNSUPPORTED, "device %d is %s; libgdn is built for gfx950 only", dev,
                  prop.gcnArchName);
    }
  }
  if (g_arch_ok[dev] < 0) return fail(GDN_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  if (cus) *cus = g_cus[dev];
  return GDN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool io_ok(gdn_dtype_t io) { return io == GDN_F32 || io == GDN_BF16; }

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_err; }

const char* gdn_version(void) { return "0.1.0"; }

gdn_status_t gdn_conv1d_fwd(const void* x, const float* w, void* y, const int32_t* cu_seqlens,
                            int Ns, int64_t N, int Cq, int K, const void* conv_state_in,
                            void* conv_state_out, gdn_dtype_t io, void* stream) {
  g_err[0] = 0;
  if (!io_ok(io)) return fail(GDN_ERR_INVALID_ARG, "conv1d: unknown io dtype %d", (int)io);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "conv1d: kernel width %d (only 4)", K);
  if (N < 0 || Ns < 1 || Cq < 1 || Cq % 8 != 0)
    return fail(GDN_ERR_INVALID_ARG, "conv1d: bad sizes N=%lld Ns=%d Cq=%d (Cq %% 8 == 0)",
                (long long)N, Ns, Cq);
  if (!cu_seqlens && Ns != 1)
    return fail(GDN_ERR_INVALID_ARG, "conv1d: cu_seqlens is NULL but Ns=%d", Ns);
  if (N > 0 && (!x || !w || !y)) return fail(GDN_ERR_INVALID_ARG, "conv1d: NULL x, w or y");
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)) || (w && !aligned(w, 16)) ||
      (conv_state_in && !aligned(conv_state_in, 16)) ||
      (conv_state_out && !aligned(conv_state_out, 16)))
    return fail(GDN_ERR_INVALID_ARG, "conv1d: pointers must be 16-byte aligned");
  if (x && y && x == y) return fail(GDN_ERR_INVALID_ARG, "conv1d: y must not alias x");
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  gdn::ConvArgs a{x, w, y, cu_seqlens, Ns, N, Cq, conv_state_in, conv_state_out};
  hipError_t e = gdn::launch_conv1d(a, io == GDN_BF16 ? gdn::IO_BF16 : gdn::IO_F32,
                                    (hipStream_t)stream);
  return e == hipSuccess ? GDN_OK : hip_fail(e, "conv1d launch");
}

size_t gdn_chunk_prefill_workspace_size(int64_t N, int Ns, int Hk, int Hv, int d, gdn_dtype_t io) {
  if (N < 0 || Ns < 1 || Hk < 1 || Hv < 1 || Hv % Hk != 0 || d != 128 || !io_ok(io)) return 0;
  // the chunk and (sequence, head) counts the prefill calls accept
  if ((N + 63) / 64 + Ns > 0x7fffffffLL || ((int64_t)Ns * Hk + 8) * (Hv / Hk) * 2 > 0x7fffffffLL)
    return 0;
  // an upper bound of the byte count, in 128-bit arithmetic: at most 128 KiB per chunk and
  // head (record, K/Q rows, map entry) and 2 MiB per (sequence, value head) of segment
  // scratch.  Below 2^62 the size's own 64-bit arithmetic cannot overflow.
  const __int128 chunks = (__int128)((N + 63) / 64 + Ns);
  const __int128 bound = chunks * (Hv + Hk) * (128 << 10) + (__int128)Ns * Hv * (2 << 20);
  if (bound > ((__int128)1 << 62)) return 0;
  return gdn::chunk_workspace_bytes(N, Ns, Hk, Hv, io == GDN_F32);
}

}  // extern "C"

namespace {

// validation and launch shared by gdn_chunk_prefill and gdn_conv_chunk_prefill
gdn_status_t chunk_prefill_impl(const char* name, gdn::ChunkArgs args, int dk, int dv,
                                void* workspace, size_t ws_bytes, gdn_dtype_t io, void* stream) {
  const int64_t N = args.N;
  const int Ns = args.Ns, Hk = args.Hk, Hv = args.Hv;
  if (!io_ok(io)) return fail(GDN_ERR_INVALID_ARG, "%s: unknown io dtype %d", name, (int)io);
  if (dk != 128 || dv != 128)
    return fail(GDN_ERR_UNSUPPORTED, "%s: head widths %d/%d (only 128/128)", name, dk, dv);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0)
    return fail(GDN_ERR_INVALID_ARG, "%s: Hv=%d must be a positive multiple of Hk=%d", name, Hv,
                Hk);
  if (Ns < 1 || N < 0) return fail(GDN_ERR_INVALID_ARG, "%s: Ns=%d N=%lld", name, Ns, (long long)N);
  if (!args.cu && Ns != 1)
    return fail(GDN_ERR_INVALID_ARG, "%s: cu_seqlens is NULL but Ns=%d", name, Ns);
  if (((int64_t)Ns * Hk + 8) * (Hv / Hk) * 2 > 0x7fffffffLL)
    return fail(GDN_ERR_INVALID_ARG, "%s: too many (sequence, head) pairs", name);
  const int64_t sq = args.stride_q, sk = args.stride_k, sv = args.stride_v;
  if (sq < (int64_t)Hk * dk || sk < (int64_t)Hk * dk || sv < (int64_t)Hv * dv || sq % 8 ||
      sk % 8 || sv % 8 || sq > GDN_MAX_ROW_STRIDE || sk > GDN_MAX_ROW_STRIDE ||
      sv > GDN_MAX_ROW_STRIDE)
    return fail(GDN_ERR_INVALID_ARG,
                "%s: strides must cover a row, be multiples of 8 and at most 2^20 "
                "(q %lld k %lld v %lld)",
                name, (long long)sq, (long long)sk, (long long)sv);
  const bool have_g = args.g_opt != nullptr, have_b = args.beta_opt != nullptr;
  if (have_g != have_b)
    return fail(GDN_ERR_INVALID_ARG, "%s: give both g_opt and beta_opt or neither", name);
  if (N > 0) {
    if (!args.q || !args.k || !args.v || !args.o)
      return fail(GDN_ERR_INVALID_ARG, "%s: NULL q, k, v or o", name);
    if (!have_g && (!args.a || !args.b || !args.A_log || !args.dt_bias))
      return fail(GDN_ERR_INVALID_ARG, "%s: NULL a, b, A_log or dt_bias", name);
    if (!aligned(args.q, 16) || !aligned(args.k, 16) || !aligned(args.v, 16) ||
        !aligned(args.o, 16))
      return fail(GDN_ERR_INVALID_ARG, "%s: q, k, v, o must be 16-byte aligned", name);
  }
  if ((N + 63) / 64 + Ns > 0x7fffffffLL) return fail(GDN_ERR_INVALID_ARG, "%s: too many chunks", name);
  const size_t need = gdn_chunk_prefill_workspace_size(N, Ns, Hk, Hv, dk, io);
  if (need == 0) return fail(GDN_ERR_INVALID_ARG, "%s: sizes beyond the workspace bound", name);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(GDN_ERR_INVALID_ARG,
                "%s: workspace must be a 256-byte aligned buffer of >= %zu bytes", name, need);
  if (args.scale <= 0.f) args.scale = 1.0f / sqrtf((float)dk);
  int cus = 0;
  gdn_status_t st = check_device(&cus);
  if (st != GDN_OK) return st;
  args.cu_count = cus;
  hipError_t e = gdn::launch_chunk_prefill(args, workspace,
                                           io == GDN_BF16 ? gdn::IO_BF16 : gdn::IO_F32,
                                           (hipStream_t)stream);
  return e == hipSuccess ? GDN_OK : hip_fail(e, "chunk_prefill launch");
}

}  // namespace

extern "C" {

gdn_status_t gdn_chunk_prefill(const void* q, const void* k, const void* v, int64_t stride_q,
                               int64_t stride_k, int64_t stride_v, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const float* g_opt,
                               const float* beta_opt, const float* state_in, float* state_out,
                               void* o, const int32_t* cu_seqlens, int Ns, int64_t N, int Hk,
                               int Hv, int dk, int dv, float scale, int use_qk_l2norm,
                               void* workspace, size_t ws_bytes, gdn_dtype_t io, void* stream) {
  g_err[0] = 0;
  gdn::ChunkArgs args{q, k, v, stride_q, stride_k, stride_v, a, b, A_log, dt_bias, g_opt,
                      beta_opt, state_in, state_out, o, cu_seqlens, Ns, N, Hk, Hv, scale,
                      use_qk_l2norm ? 1 : 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
  return chunk_prefill_impl("chunk_prefill", args, dk, dv, workspace, ws_bytes, io, stream);
}

static_assert(GDN_NOALLOC_SCRATCH_BYTES == gdn::NOALLOC_SCRATCH_BYTES, "one scratch size");

gdn_status_t gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                                       int64_t stride_q, int64_t stride_k, int64_t stride_v,
                                       const void* a, const void* b, const float* A_log,
                                       const float* dt_bias, const float* g_opt,
                                       const float* beta_opt, const float* state_in,
                                       float* state_out, void* o, const int32_t* cu_seqlens,
                                       int Ns, int64_t N, int Hk, int Hv, int dk, int dv,
                                       float scale, int use_qk_l2norm, gdn_dtype_t io,
                                       void* stream) {
  g_err[0] = 0;
  const size_t need = gdn_chunk_prefill_workspace_size(N, Ns, Hk, Hv, dk, io);
  if (need > GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_INVALID_ARG,
                "chunk_prefill_noalloc: these sizes need a %zu-byte workspace, above the "
                "fixed %zu bytes; use gdn_chunk_prefill with a caller workspace",
                need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  void* ws = nullptr;
  const hipError_t e = gdn::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "chunk_prefill_noalloc: scratch address");
  gdn::ChunkArgs args{q, k, v, stride_q, stride_k, stride_v, a, b, A_log, dt_bias, g_opt,
                      beta_opt, state_in, state_out, o, cu_seqlens, Ns, N, Hk, Hv, scale,
                      use_qk_l2norm ? 1 : 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
  return chunk_prefill_impl("chunk_prefill_noalloc", args, dk, dv, ws, GDN_NOALLOC_SCRATCH_BYTES,
                            io, stream);
}

}  // extern "C"

namespace {

// validation and launch shared by gdn_conv_chunk_prefill and gdn_prefill_layer (z, norm_w,
// y: the gated norm of the core output, or all NULL)
gdn_status_t conv_chunk_impl(const char* name, const void* x, const float* conv_w,
                             const void* conv_state_in, void* conv_state_out, void* y,
                             const void* a, const void* b, const float* A_log,
                             const float* dt_bias, const float* g_opt, const float* beta_opt,
                             const float* state_in, float* state_out, void* o, const void* z,
                             const float* norm_w, float eps, void* yn,
                             const int32_t* cu_seqlens, int Ns, int64_t N, int Hk, int Hv, int dk,
                             int dv, int K, float scale, int use_qk_l2norm, void* workspace,
                             size_t ws_bytes, gdn_dtype_t io, void* stream) {
  g_err[0] = 0;
  if (!io_ok(io)) return fail(GDN_ERR_INVALID_ARG, "%s: unknown io dtype %d", name, (int)io);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "%s: kernel width %d (only 4)", name, K);
  if (Hk < 1 || Hv < 1 || dk != 128 || dv != 128)
    return fail(dk != 128 || dv != 128 ? GDN_ERR_UNSUPPORTED : GDN_ERR_INVALID_ARG,
                "%s: Hk=%d Hv=%d dk=%d dv=%d", name, Hk, Hv, dk, dv);
  const int64_t cq = 2LL * Hk * dk + (int64_t)Hv * dv;
  if (cq > GDN_MAX_ROW_STRIDE)
    return fail(GDN_ERR_INVALID_ARG, "%s: %lld conv channels", name, (long long)cq);
  if (N > 0 && (!x || !conv_w || !y))
    return fail(GDN_ERR_INVALID_ARG, "%s: NULL x, conv_w or y", name);
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)) || (conv_w && !aligned(conv_w, 16)) ||
      (conv_state_in && !aligned(conv_state_in, 16)) ||
      (conv_state_out && !aligned(conv_state_out, 16)))
    return fail(GDN_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", name);
  if (x && y && x == y) return fail(GDN_ERR_INVALID_ARG, "%s: y must not alias x", name);
  if (yn) {
    if (!(eps >= 0.f)) return fail(GDN_ERR_INVALID_ARG, "%s: eps=%g", name, (double)eps);
    if (N > 0 && (!z || !norm_w))
      return fail(GDN_ERR_INVALID_ARG, "%s: NULL z or norm_w", name);
    if ((z && !aligned(z, 16)) || (norm_w && !aligned(norm_w, 16)) || !aligned(yn, 16))
      return fail(GDN_ERR_INVALID_ARG, "%s: z, norm_w and the norm output must be 16-byte aligned",
                  name);
  }
  const size_t esz = io == GDN_BF16 ? 2 : 4;
  const char* yb = static_cast<const char*>(y);
  gdn::ChunkArgs args{yb, yb ? yb + (size_t)Hk * dk * esz : nullptr,
                      yb ? yb + (size_t)2 * Hk * dk * esz : nullptr, cq, cq, cq, a, b, A_log,
                      dt_bias, g_opt, beta_opt, state_in, state_out, o, cu_seqlens, Ns, N, Hk,
                      Hv, scale, use_qk_l2norm ? 1 : 0, 0, x, conv_w, conv_state_in,
                      conv_state_out, y, (int)cq,
                      // one sequence of all N > 0 tokens (no cu_seqlens, so no empty or
                      // chunk-less sequence to cover) and no in-place state: the prep
                      // writes the final conv state itself
                      (io == GDN_BF16 && conv_state_out && Ns == 1 && N > 0 && !cu_seqlens &&
                       conv_state_out != conv_state_in) ? 1 : 0,
                      z, norm_w, yn, eps};
  return chunk_prefill_impl(name, args, dk, dv, workspace, ws_bytes, io, stream);
}

}  // namespace

extern "C" {

gdn_status_t gdn_conv_chunk_prefill(const void* x, const float* conv_w, const void* conv_state_in,
                                    void* conv_state_out, void* y, const void* a, const void* b,
                                    const float* A_log, const float* dt_bias, const float* g_opt,
                                    const float* beta_opt, const float* state_in,
                                    float* state_out, void* o, const int32_t* cu_seqlens, int Ns,
                                    int64_t N, int Hk, int Hv, int dk, int dv, int K, float scale,
                                    int use_qk_l2norm, void* workspace, size_t ws_bytes,
                                    gdn_dtype_t io, void* stream) {
  return conv_chunk_impl("conv_chunk_prefill", x, conv_w, conv_state_in, conv_state_out, y, a, b,
                         A_log, dt_bias, g_opt, beta_opt, state_in, state_out, o, nullptr,
                         nullptr, 0.f, nullptr, cu_seqlens, Ns, N, Hk, Hv, dk, dv, K, scale,
                         use_qk_l2norm, workspace, ws_bytes, io, stream);
}

gdn_status_t gdn_prefill_layer(const void* x, const float* conv_w, const void* conv_state_in,
                               void* conv_state_out, void* y_conv, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const float* g_opt,
                               const float* beta_opt, const float* state_in, float* state_out,
                               void* o, const void* z, const float* norm_w, float eps, void* y,
                               const int32_t* cu_seqlens, int Ns, int64_t N, int Hk, int Hv,
                               int dk, int dv, int K, float scale, int use_qk_l2norm,
                               void* workspace, size_t ws_bytes, gdn_dtype_t io, void* stream) {
  if (N > 0 && !y) {
    g_err[0] = 0;
    return fail(GDN_ERR_INVALID_ARG, "prefill_layer: NULL norm output y");
  }
  return conv_chunk_impl("prefill_layer", x, conv_w, conv_state_in, conv_state_out, y_conv, a, b,
                         A_log, dt_bias, g_opt, beta_opt, state_in, state_out, o, z, norm_w, eps,
                         y, cu_seqlens, Ns, N, Hk, Hv, dk, dv, K,
                         scale, use_qk_l2norm, workspace, ws_bytes, io, stream);
}

namespace {

gdn_status_t recurrent_step_impl(const char* name, const void* x, const float* w, void* conv_state,
                                 const void* a, const void* b, const float* A_log,
                                 const float* dt_bias, const float* g_opt, const float* beta_opt,
                                 void* state, int state_bf16, void* o, int B, int Hk, int Hv,
                                 int dk, int dv, int K, float scale, int use_qk_l2norm,
                                 gdn_dtype_t io, void* stream, const int32_t* slots = nullptr,
                                 int n_slots = 0, const void* z = nullptr,
                                 const float* norm_w = nullptr, void* y = nullptr,
                                 float eps = 0.f) {
  g_err[0] = 0;
  if (!io_ok(io)) return fail(GDN_ERR_INVALID_ARG, "%s: unknown io dtype %d", name, (int)io);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "%s: kernel width %d (only 4)", name, K);
  if (dk != 128 || dv != 128)
    return fail(GDN_ERR_UNSUPPORTED, "%s: head widths %d/%d (only 128/128)", name, dk, dv);
  if (B < 0 || Hk < 1 || Hv < 1 || Hv % Hk != 0 || Hv / Hk > 128)
    return fail(GDN_ERR_INVALID_ARG, "%s: B=%d Hk=%d Hv=%d", name, B, Hk, Hv);
  if ((int64_t)B * Hk > 0x7fffffffLL)
    return fail(GDN_ERR_INVALID_ARG, "%s: too many (sequence, key head) pairs", name);
  const bool have_g = g_opt != nullptr, have_b = beta_opt != nullptr;
  if (have_g != have_b)
    return fail(GDN_ERR_INVALID_ARG, "%s: give both g_opt and beta_opt or neither", name);
  if (B > 0) {
    if (!x || !w || !conv_state || !state || (!o && !y))
      return fail(GDN_ERR_INVALID_ARG, "%s: NULL x, w, conv_state, state or o", name);
    if (y && (!z || !norm_w))
      return fail(GDN_ERR_INVALID_ARG, "%s: NULL z or norm_w", name);
    if (y && (!aligned(norm_w, 16) || !aligned(z, 8) || !aligned(y, 8) || (o && !aligned(o, 8))))
      return fail(GDN_ERR_INVALID_ARG, "%s: z, y, o must be 8-byte and norm_w 16-byte aligned",
                  name);
    if (!have_g && (!a || !b || !A_log || !dt_bias))
      return fail(GDN_ERR_INVALID_ARG, "%s: NULL a, b, A_log or dt_bias", name);
    if (!aligned(state, 16) || !aligned(w, 16))
      return fail(GDN_ERR_INVALID_ARG, "%s: state and w must be 16-byte aligned", name);
    if (slots && !aligned(slots, 4))
      return fail(GDN_ERR_INVALID_ARG, "%s: slots must be 4-byte aligned", name);
  }
  if (scale <= 0.f) scale = 1.0f / sqrtf((float)dk);
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  gdn::StepArgs args{x, w, conv_state, a, b, A_log, dt_bias, g_opt, beta_opt, state, o, B, Hk, Hv,
                     scale, use_qk_l2norm ? 1 : 0, state_bf16, slots, n_slots, z, norm_w, y,
                     eps};
  hipError_t e = gdn::launch_recurrent_step(args, io == GDN_BF16 ? gdn::IO_BF16 : gdn::IO_F32,
                                            (hipStream_t)stream);
  return e == hipSuccess ? GDN_OK : hip_fail(e, "recurrent_step launch");
}

}  // namespace

gdn_status_t gdn_recurrent_step(const void* x, const float* w, void* conv_state, const void* a,
                                const void* b, const float* A_log, const float* dt_bias,
                                const float* g_opt, const float* beta_opt, float* state, void* o,
                                int B, int Hk, int Hv, int dk, int dv, int K, float scale,
                                int use_qk_l2norm, gdn_dtype_t io, void* stream) {
  return recurrent_step_impl("recurrent_step", x, w, conv_state, a, b, A_log, dt_bias, g_opt,
                             beta_opt, state, 0, o, B, Hk, Hv, dk, dv, K, scale, use_qk_l2norm, io,
                             stream);
}

gdn_status_t gdn_recurrent_step_bf16_state(const void* x, const float* w, void* conv_state,
                                           const void* a, const void* b, const float* A_log,
                                           const float* dt_bias, const float* g_opt,
                                           const float* beta_opt, void* state, void* o, int B,
                                           int Hk, int Hv, int dk, int dv, int K, float scale,
                                           int use_qk_l2norm, gdn_dtype_t io, void* stream) {
  return recurrent_step_impl("recurrent_step_bf16_state", x, w, conv_state, a, b, A_log, dt_bias,
                             g_opt, beta_opt, state, 1, o, B, Hk, Hv, dk, dv, K, scale,
                             use_qk_l2norm, io, stream);
}

gdn_status_t gdn_recurrent_step_slots(const void* x, const float* w, void* conv_state_pool,
                                      const void* a, const void* b, const float* A_log,
                                      const float* dt_bias, const float* g_opt,
                                      const float* beta_opt, void* state_pool,
                                      gdn_dtype_t state_dtype, const int32_t* slots, int n_slots,
                                      void* o, int B, int Hk, int Hv, int dk, int dv, int K,
                                      float scale, int use_qk_l2norm, gdn_dtype_t io,
                                      void* stream) {
  g_err[0] = 0;
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID_ARG, "recurrent_step_slots: unknown state dtype %d",
                (int)state_dtype);
  if (n_slots < 1 || (B > 0 && !slots))
    return fail(GDN_ERR_INVALID_ARG, "recurrent_step_slots: n_slots=%d, slots %s", n_slots,
                slots ? "given" : "NULL");
  return recurrent_step_impl("recurrent_step_slots", x, w, conv_state_pool, a, b, A_log, dt_bias,
                             g_opt, beta_opt, state_pool, state_dtype == GDN_BF16 ? 1 : 0, o, B,
                             Hk, Hv, dk, dv, K, scale, use_qk_l2norm, io, stream, slots, n_slots);
}

gdn_status_t gdn_recurrent_step_norm(const void* x, const float* w, void* conv_state,
                                     const void* a, const void* b, const float* A_log,
                                     const float* dt_bias, const float* g_opt,
                                     const float* beta_opt, void* state, gdn_dtype_t state_dtype,
                                     const void* z, const float* norm_w, float eps, void* o_opt,
                                     void* y, int B, int Hk, int Hv, int dk, int dv, int K,
                                     float scale, int use_qk_l2norm, gdn_dtype_t io,
                                     void* stream) {
  g_err[0] = 0;
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID_ARG, "recurrent_step_norm: unknown state dtype %d",
                (int)state_dtype);
  if (!(eps >= 0.f)) return fail(GDN_ERR_INVALID_ARG, "recurrent_step_norm: eps=%g", (double)eps);
  if (B > 0 && !y) return fail(GDN_ERR_INVALID_ARG, "recurrent_step_norm: NULL y");
  return recurrent_step_impl("recurrent_step_norm", x, w, conv_state, a, b, A_log, dt_bias, g_opt,
                             beta_opt, state, state_dtype == GDN_BF16 ? 1 : 0, o_opt, B, Hk, Hv,
                             dk, dv, K, scale, use_qk_l2norm, io, stream, nullptr, 0, z, norm_w,
                             y, eps);
}

gdn_status_t gdn_gated_rmsnorm(const void* o, const void* z, const float* w, void* y,
                               int64_t rows, int D, float eps, gdn_dtype_t io, void* stream) {
  g_err[0] = 0;
  if (!io_ok(io)) return fail(GDN_ERR_INVALID_ARG, "gated_rmsnorm: unknown io dtype %d", (int)io);
  if (D != 128) return fail(GDN_ERR_UNSUPPORTED, "gated_rmsnorm: row width %d (only 128)", D);
  if (rows < 0 || !(eps >= 0.f))
    return fail(GDN_ERR_INVALID_ARG, "gated_rmsnorm: rows=%lld eps=%g", (long long)rows, (double)eps);
  // 16 rows per block and at most 2^31 - 1 blocks
  if (rows > 0x7fffffffLL * 16)
    return fail(GDN_ERR_INVALID_ARG, "gated_rmsnorm: %lld rows (at most 2^35 - 16)", (long long)rows);
  if (rows > 0) {
    if (!o || !z || !w || !y) return fail(GDN_ERR_INVALID_ARG, "gated_rmsnorm: NULL pointer");
    if (!aligned(o, 16) || !aligned(z, 16) || !aligned(w, 16) || !aligned(y, 16))
      return fail(GDN_ERR_INVALID_ARG, "gated_rmsnorm: pointers must be 16-byte aligned");
  }
  gdn_status_t st = check_device();
  if (st != GDN_OK) return st;
  gdn::NormArgs args{o, z, w, y, rows, eps};
  hipError_t e = gdn::launch_gated_rmsnorm(args, io == GDN_BF16 ? gdn::IO_BF16 : gdn::IO_F32,
                                           (hipStream_t)stream);
  return e == hipSuccess ? GDN_OK : hip_fail(e, "gated_rmsnorm launch");
}

}  // extern "C"
