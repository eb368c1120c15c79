// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime_api.h>

namespace gdr {

struct RecurrentArgs {
  int N, H, D;            // D = Dk = Dv
  bool in_bf16, out_bf16;
  int gate;               // 0 none, 1 scalar, 2 channel
  bool erase;             // false: additive write, no erase term
  int fuse;               // gdr_fuse flags
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  const void *out_gate;   // SiLU output gate (in_dtype) or nullptr
  float *state;
  void *o;
  hipStream_t stream;
};

struct ChunkArgs {
  int B, T, H, D, chunk;  // D = Dk = Dv
  bool in_bf16, out_bf16;
  int gate;
  bool erase;             // false: additive write, no erase term
  int fuse;               // gdr_fuse flags
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  const void *out_gate;   // SiLU output gate (in_dtype) or nullptr
  const float *initial_state;
  void *o;
  float *final_state;
  hipStream_t stream;
};

hipError_t launch_recurrent_step(const RecurrentArgs &a);
// bf16 q/k/v, MFMA path (D = 128 and 64)
hipError_t launch_chunk_fwd_bf16(const ChunkArgs &a);
bool chunk_fwd_bf16_supported(const ChunkArgs &a);
// bf16 q/k/v with the per-channel gate, MFMA path (D = 128 and 64)
hipError_t launch_chunk_fwd_kda(const ChunkArgs &a);
bool chunk_fwd_kda_supported(const ChunkArgs &a);
// plain fp32 arithmetic path: fp32 or bf16 q/k/v, D <= 64, every gate
hipError_t launch_chunk_fwd_small(const ChunkArgs &a);
bool chunk_fwd_small_supported(const ChunkArgs &a);
// zero or copy the state for T == 0
hipError_t launch_state_passthrough(const float *src, float *dst, long count, hipStream_t stream);

}  // namespace gdr
