// Device-side helpers shared by the gated delta-rule kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum Gate { kGateNone = 0, kGateScalar = 1, kGateChannel = 2 };

// What a chunk kernel computes: the forward, or one of the backward's two
// sequential passes (the forward recomputed, storing per chunk the entering
// state and U; the reverse walk storing the state gradient and dY), or the
// forward that also stores what the first pass would (for training).
enum Mode { kModeFwd = 0, kModeRec = 1, kModeRev = 2, kModeFwdSave = 3 };

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Fused prologue / epilogue (gdr_fuse flags of the C ABI).
enum Fuse { kFuseL2 = 1, kFuseBetaSigmoid = 2, kFuseSoftplus = 4, kFuseGla = 8 };
constexpr float kL2Eps = 1e-6f;   // q, k <- x / sqrt(sum x^2 + eps)

// The activations use the hardware exp2 / log2 / reciprocal (about one ulp
// each): they run per element inside the chunk pipelines, where the
// library's log1p and the IEEE divide cost more than the rest of a stage.
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
// softplus(x) log2(e) = max(x, 0) log2(e) + log2(1 + 2^{-|x| log2(e)}):
// log(1 + e^x) without overflow for large |x|, in base 2, where each step
// is one hardware instruction (exp2; log2 of an argument in (1, 2], so no
// denormal scaling).  The natural-log library call costs about twelve
// instructions per value, which made the per-channel decay transform the
// slowest stage of the fused chunk kernel.
__device__ __forceinline__ float softplus2_f(float x) {
  const float l = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f));
  return fmaf(fmaxf(x, 0.0f), 1.4426950408889634f, l);
}
__device__ __forceinline__ float softplus_f(float x) { return softplus2_f(x) * 0.6931471805599453f; }
// b from the beta input
__device__ __forceinline__ float fused_beta(float b, int fuse) {
  return (fuse & kFuseBetaSigmoid) ? sigmoid_f(b) : b;
}
// log2 a from x when a decay transform is on (gla: GLA's gate, else the
// softplus decay); one softplus either way: log sigmoid(x)^{1/16} =
// -softplus(-x) / 16
__device__ __forceinline__ float decay_transform2(float x, bool gla) {
  const float sp2 = softplus2_f(gla ? -x : x);
  return gla ? sp2 * (-1.0f / 16.0f) : -sp2;
}
// the same in natural-log units
__device__ __forceinline__ float decay_transform(float x, bool gla) {
  return decay_transform2(x, gla) * 0.6931471805599453f;
}
// log a from the log_alpha input: -softplus(x), or GLA's sigmoid(x)^{1/16}
__device__ __forceinline__ float fused_log_alpha(float x, int fuse) {
  if (!(fuse & (kFuseSoftplus | kFuseGla))) return x;
  return decay_transform(x, (fuse & kFuseGla) != 0);
}
// the SiLU output gate applied to an output value
__device__ __forceinline__ float silu_gate(float o, float g) { return o * g * sigmoid_f(g); }

// D += A(16x32) * B(32x16), bf16 operands, fp32 accumulate.  Lane l holds
// A row (l & 15) and B column (l & 15), eight k values per lane (the same k
// set for A and B, so any consistent k order gives the same product); the
// result lane l holds column (l & 15), rows 4*(l >> 4) + 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace gdr
