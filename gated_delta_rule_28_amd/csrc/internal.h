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

// ---- backward of the chunk forward (bf16 q/k/v/dO, D = 64 or 128, every
//      gate, with or without the erase term) ----
constexpr int kBwdChunk = 32;      // tokens per chunk of the passes and of the workspace
constexpr int kBwdChunkKda = 16;   // the same with the per-channel gate
inline int bwd_chunk(int gate) { return gate == 2 ? kBwdChunkKda : kBwdChunk; }

struct BwdArgs {
  int B, T, H, D;
  int gate;                     // kGateNone, kGateScalar or kGateChannel
  bool erase;                   // false: the additive write (no erase term)
  bool saved;                   // h and U are in the workspace already (a training
                                // forward stored them): no recompute pass
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  const float *initial_state;   // S_0 or nullptr
  const void *d_o;              // dL/do [B, T, H, D], dtype of q
  const float *d_final_state;   // dL/dS_T or nullptr
  void *dq, *dk, *dv;            // fp32, or bf16 when grad_bf16
  bool grad_bf16;
  float *dbeta, *dlog_alpha, *d_initial_state;
  // workspace partitions, per (chain, chunk): the entering state h and U
  // (recompute pass); dh and dY (reverse pass); each chunk's block in the
  // state waves' fragment order (ws_frag, mfma_util.h)
  float *ws_h, *ws_u, *ws_dh, *ws_dy;
  hipStream_t stream;
};

// workspace floats per (chain, chunk): h and dh [D][D], U and dY [C][D]
inline long bwd_ws_floats_per_chunk(int D, int gate) {
  return 2L * D * D + 2L * bwd_chunk(gate) * D;
}
bool chunk_bwd_supported(int D, bool in_bf16, int gate, bool erase, long H);
// the two sequential passes: the forward recomputed (h, U per chunk), then
// the reverse pass (dh, dY per chunk, and dS_0)
hipError_t launch_chunk_bwd_passes(const BwdArgs &a);
// the chunk-parallel gradients dq, dk, dv, dbeta, dlog_alpha
hipError_t launch_chunk_bwd_grads(const BwdArgs &a);
// the same two steps with the per-channel gate (16-token chunks)
hipError_t launch_chunk_bwd_kda_passes(const BwdArgs &a);
hipError_t launch_chunk_bwd_kda_grads(const BwdArgs &a);
// the forward that also stores, per chunk, h and U into the backward's
// workspace partitions (the training forward; bf16, D = 64 or 128)
hipError_t launch_chunk_fwd_bf16_save(const ChunkArgs &a, float *ws_h, float *ws_u);
hipError_t launch_chunk_fwd_kda_save(const ChunkArgs &a, float *ws_h, float *ws_u);

}  // namespace gdr
