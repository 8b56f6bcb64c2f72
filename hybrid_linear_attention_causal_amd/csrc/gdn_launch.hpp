// Internal launcher interface between the C ABI (gdn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum IoType { IO_F32 = 0, IO_BF16 = 1 };

struct ConvArgs {
  const void* x;
  const float* w;
  void* y;
  const int32_t* cu;     // may be null (one sequence)
  int Ns;
  int64_t N;
  int Cq;
  const void* state_in;  // may be null
  void* state_out;       // may be null
};

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t stride_q, stride_k, stride_v;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  const float* g_opt;     // both or neither
  const float* beta_opt;
  const float* state_in;  // may be null
  float* state_out;       // may be null
  void* o;
  const int32_t* cu;      // may be null
  int Ns;
  int64_t N;
  int Hk, Hv;
  float scale;
  int use_l2;
  int cu_count;           // compute units of the device (launch shape choice; <= 0: 256)
  // fused conv (x != NULL): the conv window + SiLU of the raw projection rows x [N, Cq] is
  // formed inside the call and written to y [N, Cq] (q, k, v above point into y); the
  // final conv state goes to conv_state_out when given
  const void* x;
  const float* conv_w;
  const void* conv_state_in;
  void* conv_state_out;
  void* y;
  int Cq;
  int conv_state_in_prep;   // one non-empty sequence, conv_state_out not aliasing the input:
                            // the prep workgroup of the last chunk writes the final state
  // gated norm of the core output (yn != NULL): yn = norm_w * o / sqrt(mean(o^2) + eps) *
  // silu(z) per (token, value head) row, o taken as stored; z, yn [N, Hv, 128] io.  Formed by
  // the norm kernel after the core, on the same stream.
  const void* z;
  const float* norm_w;
  void* yn;
  float eps;
};

struct StepArgs {
  const void* x;
  const float* w;
  void* conv_state;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  const float* g_opt;
  const float* beta_opt;
  void* state;            // fp32, or bf16 when state_bf16
  void* o;
  int B, Hk, Hv;
  float scale;
  int use_l2;
  int state_bf16;         // 1: the state is stored as bf16 (read, computed in fp32, rounded back)
  const int32_t* slots;   // NULL: row b uses state b; else slots[b] in [0, n_slots), other = padding
  int n_slots;
  // fused z-gated RMSNorm of o (y != NULL): y = norm_w * o / sqrt(mean(o^2) + eps) * silu(z),
  // o taken as stored (rounded to io); o itself is written only when o != NULL
  const void* z;
  const float* norm_w;
  void* y;
  float eps;
};

struct NormArgs {
  const void* o;
  const void* z;
  const float* w;
  void* y;
  int64_t rows;
  float eps;
};

hipError_t launch_conv1d(const ConvArgs& a, int io, hipStream_t s);
// only the final conv state of a conv call (conv_state_out from x and conv_state_in)
hipError_t launch_conv_state(const ConvArgs& a, int io, hipStream_t s);
// device workspace of the chunked prefill (chunk map + per (chunk, head) records)
size_t chunk_workspace_bytes(int64_t N, int Ns, int Hk, int Hv, bool f32);
hipError_t launch_chunk_prefill(const ChunkArgs& a, void* ws, int io, hipStream_t s);
hipError_t launch_recurrent_step(const StepArgs& a, int io, hipStream_t s);
hipError_t launch_gated_rmsnorm(const NormArgs& a, int io, hipStream_t s);

// the allocation-free prefill's fixed device workspace: its size, and its device address
// on the current device (looked up once per device)
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)128 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace gdn
