// C ABI entry points: argument validation on the host, then dispatch to the
// kernel launchers.  No exception crosses this boundary and nothing is
// launched for an invalid call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdr.h"
#include "internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void *p, unsigned bytes) {
  return (reinterpret_cast<uintptr_t>(p) & (uintptr_t)(bytes - 1)) == 0;
}

bool valid_dtype(int d) { return d == GDR_F32 || d == GDR_BF16; }
bool valid_gate(int g) {
  const int base = g & ~GDR_NO_ERASE;
  return base == GDR_GATE_NONE || base == GDR_GATE_SCALAR || base == GDR_GATE_CHANNEL;
}
int gate_kind(int g) { return g & ~GDR_NO_ERASE; }
bool erases(int g) { return (g & GDR_NO_ERASE) == 0; }
bool supported_head(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// gate/log_alpha consistency and common pointer checks for both entry points
int check_common(int Dk, int Dv, int in_dtype, int out_dtype, int gate, const void *q,
                 const void *k, const void *v, const float *beta, const float *log_alpha,
                 const void *o) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !valid_gate(gate)) return GDR_EINVAL;
  if ((gate_kind(gate) == GDR_GATE_NONE) != (log_alpha == nullptr)) return GDR_EINVAL;
  if (!q || !k || !v || !beta || !o) return GDR_EINVAL;
  // q/k/v/o are accessed with 16-byte vectors; beta/log_alpha are scalars
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned(beta, 4) ||
      (log_alpha && !aligned(log_alpha, 4)))
    return GDR_EINVAL;
  if (Dk != Dv || !supported_head(Dk)) return GDR_EUNSUPPORTED;
  return GDR_OK;
}

// fused-prologue flags: known bits, at most one decay transform, and a
// decay transform only with a gate; the output gate is read with vectors
int check_fuse(int fuse, int gate, const void *out_gate) {
  const int known = GDR_FUSE_QK_L2NORM | GDR_FUSE_BETA_SIGMOID | GDR_FUSE_DECAY_SOFTPLUS |
                    GDR_FUSE_DECAY_GLA;
  if (fuse & ~known) return GDR_EINVAL;
  const int decay = fuse & (GDR_FUSE_DECAY_SOFTPLUS | GDR_FUSE_DECAY_GLA);
  if (decay == (GDR_FUSE_DECAY_SOFTPLUS | GDR_FUSE_DECAY_GLA)) return GDR_EINVAL;
  if (decay && gate_kind(gate) == GDR_GATE_NONE) return GDR_EINVAL;
  if (out_gate && !aligned16(out_gate)) return GDR_EINVAL;
  return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_status_str(int status) {
  switch (status) {
    case GDR_OK: return "GDR_OK";
    case GDR_EINVAL: return "GDR_EINVAL: invalid argument";
    case GDR_EUNSUPPORTED: return "GDR_EUNSUPPORTED: shape/dtype/chunk not implemented";
    case GDR_EHIP: return "GDR_EHIP: HIP runtime error on launch";
    case GDR_EWORKSPACE: return "GDR_EWORKSPACE: workspace missing, misaligned or too small";
    default: return "unknown gdr status";
  }
}

int gdr_chunk_fwd(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int out_dtype,
                  int gate, const void *q, const void *k, const void *v, const float *beta,
                  const float *log_alpha, const float *initial_state, void *o,
                  float *final_state, hipStream_t stream) {
  return gdr_chunk_fwd_ex(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, 0, q, k, v, beta,
                          log_alpha, nullptr, initial_state, o, final_state, stream);
}

int gdr_chunk_fwd_ex(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int out_dtype,
                     int gate, int fuse, const void *q, const void *k, const void *v,
                     const float *beta, const float *log_alpha, const void *out_gate,
                     const float *initial_state, void *o, float *final_state,
                     hipStream_t stream) {
  if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDR_EINVAL;
  if (!(chunk == 0 || chunk == 16 || chunk == 32 || chunk == 64)) return GDR_EUNSUPPORTED;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !valid_gate(gate)) return GDR_EINVAL;
  if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return GDR_EINVAL;
  if (check_fuse(fuse, gate, out_gate) != GDR_OK) return GDR_EINVAL;
  if (Dk != Dv || !supported_head(Dk)) return GDR_EUNSUPPORTED;
  // empty token tensors may carry null pointers, so these return before the
  // pointer checks
  if ((long)B * H == 0) return GDR_OK;                   // nothing to compute
  if (T == 0) {                                          // no tokens: S_T = S_0
    if (!final_state || final_state == initial_state) return GDR_OK;
    hipError_t e = gdr::launch_state_passthrough(initial_state, final_state,
                                                 (long)B * H * Dk * Dv, stream);
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
  }
  int st = check_common(Dk, Dv, in_dtype, out_dtype, gate, q, k, v, beta, log_alpha, o);
  if (st != GDR_OK) return st;
  // per-channel log decays are read as rows of Dk floats with 16-byte vectors
  if (gate_kind(gate) == GDR_GATE_CHANNEL && !aligned16(log_alpha)) return GDR_EINVAL;

  gdr::ChunkArgs a;
  a.B = B; a.T = T; a.H = H; a.D = Dk; a.chunk = chunk;
  a.in_bf16 = in_dtype == GDR_BF16; a.out_bf16 = out_dtype == GDR_BF16;
  a.gate = gate_kind(gate);
  a.erase = erases(gate);
  a.fuse = fuse;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
  a.out_gate = out_gate;
  a.initial_state = initial_state; a.o = o; a.final_state = final_state;
  a.stream = stream;

  hipError_t e;
  if (gdr::chunk_fwd_bf16_supported(a)) e = gdr::launch_chunk_fwd_bf16(a);
  else if (gdr::chunk_fwd_kda_supported(a)) e = gdr::launch_chunk_fwd_kda(a);
  else if (gdr::chunk_fwd_small_supported(a)) e = gdr::launch_chunk_fwd_small(a);
  else return GDR_EUNSUPPORTED;
  return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

size_t gdr_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     int in_dtype, int out_dtype, int gate) {
  // every forward kernel keeps its intermediates in registers and LDS
  (void)B; (void)T; (void)H; (void)Dk; (void)Dv; (void)chunk;
  (void)in_dtype; (void)out_dtype; (void)gate;
  return 0;
}

namespace {

// workspace bytes of a supported backward call with at least one token
// (gate: the gate kind, which sets the chunk of the passes)
size_t bwd_workspace(long B, long T, long H, int D, int gate) {
  const int C = gdr::bwd_chunk(gate);
  const long nchunks = (T + C - 1) / C;
  return (size_t)(B * H * nchunks) * (size_t)gdr::bwd_ws_floats_per_chunk(D, gate) * sizeof(float);
}

bool bwd_shape_ok(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int gate) {
  if (Dk != Dv || !(chunk == 0 || chunk == 16 || chunk == 32 || chunk == 64)) return false;
  if (!gdr::chunk_bwd_supported(Dk, in_dtype == GDR_BF16, gate_kind(gate), erases(gate), H))
    return false;
  // one workgroup per (chain, chunk) in the gradient kernel
  const int C = gdr::bwd_chunk(gate_kind(gate));
  const long nchunks = ((long)T + C - 1) / C;
  return (long)B * H * nchunks < 0x7FFFFFFFL;
}

}  // namespace

size_t gdr_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     int in_dtype, int gate) {
  if (B <= 0 || T <= 0 || H <= 0 || !valid_dtype(in_dtype) || !valid_gate(gate)) return 0;
  if (!bwd_shape_ok(B, T, H, Dk, Dv, chunk, in_dtype, gate)) return 0;
  return bwd_workspace(B, T, H, Dk, gate_kind(gate));
}

namespace {

// the workspace partitions of a backward call: h, dh [chain][chunk][D][D];
// U, dY [chain][chunk][C][D] (each chunk's block in fragment order)
void bwd_partitions(gdr::BwdArgs &a, void *workspace) {
  const int C = gdr::bwd_chunk(a.gate);
  const long nblk = (long)a.B * a.H * ((a.T + C - 1) / C);
  float *w = static_cast<float *>(workspace);
  a.ws_h = w;
  a.ws_dh = a.ws_h + nblk * a.D * a.D;
  a.ws_u = a.ws_dh + nblk * a.D * a.D;
  a.ws_dy = a.ws_u + nblk * C * a.D;
}

// gdr_chunk_bwd_ex: gdr_chunk_bwd with dq, dk, dv in grad_dtype, and with
// saved = true gdr_chunk_bwd_saved (the workspace holds h and U from
// gdr_chunk_fwd_train: no recompute pass)
int chunk_bwd_impl(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int grad_dtype,
                   int gate, const void *q, const void *k, const void *v, const float *beta,
                   const float *log_alpha, const float *initial_state, const void *d_o,
                   const float *d_final_state, void *dq, void *dk, void *dv, float *dbeta,
                   float *dlog_alpha, float *d_initial_state, void *workspace,
                   size_t workspace_bytes, hipStream_t stream, bool saved) {
  if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDR_EINVAL;
  if (!valid_dtype(in_dtype) || !valid_dtype(grad_dtype) || !valid_gate(gate)) return GDR_EINVAL;
  if ((gate_kind(gate) == GDR_GATE_NONE) != (log_alpha == nullptr)) return GDR_EINVAL;
  if ((gate_kind(gate) == GDR_GATE_NONE) != (dlog_alpha == nullptr)) return GDR_EINVAL;
  if ((initial_state && !aligned16(initial_state)) || (d_final_state && !aligned16(d_final_state)) ||
      (d_initial_state && !aligned16(d_initial_state)))
    return GDR_EINVAL;
  if (!bwd_shape_ok(B, T, H, Dk, Dv, chunk, in_dtype, gate)) return GDR_EUNSUPPORTED;
  if ((long)B * H == 0) return GDR_OK;                   // nothing to compute
  if (T == 0) {                                          // no tokens: dS_0 = dS_T
    if (!d_initial_state) return GDR_OK;
    hipError_t e = gdr::launch_state_passthrough(d_final_state, d_initial_state,
                                                 (long)B * H * Dk * Dv, stream);
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
  }
  if (!q || !k || !v || !beta || !d_o || !dq || !dk || !dv || !dbeta) return GDR_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned(beta, 4) || !aligned(dbeta, 4) ||
      (log_alpha && !aligned(log_alpha, 4)) || (dlog_alpha && !aligned(dlog_alpha, 4)))
    return GDR_EINVAL;
  const size_t need = bwd_workspace(B, T, H, Dk, gate_kind(gate));
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < need)
    return GDR_EWORKSPACE;

  gdr::BwdArgs a;
  a.B = B; a.T = T; a.H = H; a.D = Dk;
  a.gate = gate_kind(gate);
  a.erase = erases(gate);
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
  a.initial_state = initial_state; a.d_o = d_o; a.d_final_state = d_final_state;
  a.dq = dq; a.dk = dk; a.dv = dv; a.grad_bf16 = grad_dtype == GDR_BF16;
  a.dbeta = dbeta; a.dlog_alpha = dlog_alpha;
  a.d_initial_state = d_initial_state;
  a.saved = saved;
  bwd_partitions(a, workspace);
  a.stream = stream;
  const bool kda = a.gate == GDR_GATE_CHANNEL;
  hipError_t e = kda ? gdr::launch_chunk_bwd_kda_passes(a) : gdr::launch_chunk_bwd_passes(a);
  if (e == hipSuccess) e = kda ? gdr::launch_chunk_bwd_kda_grads(a) : gdr::launch_chunk_bwd_grads(a);
  return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

}  // namespace

int gdr_chunk_bwd(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int gate,
                  const void *q, const void *k, const void *v, const float *beta,
                  const float *log_alpha, const float *initial_state, const void *d_o,
                  const float *d_final_state, float *dq, float *dk, float *dv, float *dbeta,
                  float *dlog_alpha, float *d_initial_state, void *workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  return chunk_bwd_impl(B, T, H, Dk, Dv, chunk, in_dtype, GDR_F32, gate, q, k, v, beta,
                        log_alpha, initial_state, d_o, d_final_state, dq, dk, dv, dbeta,
                        dlog_alpha, d_initial_state, workspace, workspace_bytes, stream, false);
}

int gdr_chunk_bwd_ex(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype,
                     int grad_dtype, int gate, const void *q, const void *k, const void *v,
                     const float *beta, const float *log_alpha, const float *initial_state,
                     const void *d_o, const float *d_final_state, void *dq, void *dk, void *dv,
                     float *dbeta, float *dlog_alpha, float *d_initial_state, void *workspace,
                     size_t workspace_bytes, int saved, hipStream_t stream) {
  return chunk_bwd_impl(B, T, H, Dk, Dv, chunk, in_dtype, grad_dtype, gate, q, k, v, beta,
                        log_alpha, initial_state, d_o, d_final_state, dq, dk, dv, dbeta,
                        dlog_alpha, d_initial_state, workspace, workspace_bytes, stream,
                        saved != 0);
}

int gdr_chunk_bwd_saved(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int gate,
                        const void *q, const void *k, const void *v, const float *beta,
                        const float *log_alpha, const float *initial_state, const void *d_o,
                        const float *d_final_state, float *dq, float *dk, float *dv,
                        float *dbeta, float *dlog_alpha, float *d_initial_state,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return chunk_bwd_impl(B, T, H, Dk, Dv, chunk, in_dtype, GDR_F32, gate, q, k, v, beta,
                        log_alpha, initial_state, d_o, d_final_state, dq, dk, dv, dbeta,
                        dlog_alpha, d_initial_state, workspace, workspace_bytes, stream, true);
}

int gdr_chunk_fwd_train(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype,
                        int out_dtype, int gate, const void *q, const void *k, const void *v,
                        const float *beta, const float *log_alpha, const float *initial_state,
                        void *o, float *final_state, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDR_EINVAL;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype) || !valid_gate(gate)) return GDR_EINVAL;
  if ((gate_kind(gate) == GDR_GATE_NONE) != (log_alpha == nullptr)) return GDR_EINVAL;
  if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return GDR_EINVAL;
  // the supported set of the backward, whose workspace this call fills
  if (!bwd_shape_ok(B, T, H, Dk, Dv, chunk, in_dtype, gate)) return GDR_EUNSUPPORTED;
  if ((long)B * H == 0) return GDR_OK;                   // nothing to compute
  if (T == 0) {                                          // no tokens: S_T = S_0, nothing saved
    if (!final_state || final_state == initial_state) return GDR_OK;
    hipError_t e = gdr::launch_state_passthrough(initial_state, final_state,
                                                 (long)B * H * Dk * Dv, stream);
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
  }
  int st = check_common(Dk, Dv, in_dtype, out_dtype, gate, q, k, v, beta, log_alpha, o);
  if (st != GDR_OK) return st;
  if (gate_kind(gate) == GDR_GATE_CHANNEL && !aligned16(log_alpha)) return GDR_EINVAL;
  const size_t need = bwd_workspace(B, T, H, Dk, gate_kind(gate));
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < need)
    return GDR_EWORKSPACE;

  gdr::ChunkArgs a;
  a.B = B; a.T = T; a.H = H; a.D = Dk; a.chunk = chunk;
  a.in_bf16 = true; a.out_bf16 = out_dtype == GDR_BF16;
  a.gate = gate_kind(gate);
  a.erase = erases(gate);
  a.fuse = 0;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
  a.out_gate = nullptr;
  a.initial_state = initial_state; a.o = o; a.final_state = final_state;
  a.stream = stream;
  gdr::BwdArgs w;
  w.B = B; w.T = T; w.H = H; w.D = Dk; w.gate = gate_kind(gate);
  bwd_partitions(w, workspace);
  const hipError_t e = a.gate == GDR_GATE_CHANNEL
                           ? gdr::launch_chunk_fwd_kda_save(a, w.ws_h, w.ws_u)
                           : gdr::launch_chunk_fwd_bf16_save(a, w.ws_h, w.ws_u);
  return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

int gdr_recurrent_step(int N, int H, int Dk, int Dv, int in_dtype, int out_dtype, int gate,
                       const void *q, const void *k, const void *v, const float *beta,
                       const float *log_alpha, float *state, void *o, hipStream_t stream) {
  return gdr_recurrent_step_ex(N, H, Dk, Dv, in_dtype, out_dtype, gate, 0, q, k, v, beta,
                               log_alpha, nullptr, state, o, stream);
}

int gdr_recurrent_step_ex(int N, int H, int Dk, int Dv, int in_dtype, int out_dtype, int gate,
                          int fuse, const void *q, const void *k, const void *v,
                          const float *beta, const float *log_alpha, const void *out_gate,
                          float *state, void *o, hipStream_t stream) {
  if (N < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDR_EINVAL;
  if ((long)N * H == 0) return GDR_OK;
  int st = check_common(Dk, Dv, in_dtype, out_dtype, gate, q, k, v, beta, log_alpha, o);
  if (st != GDR_OK) return st;
  if (!state || !aligned16(state)) return GDR_EINVAL;
  if (check_fuse(fuse, gate, out_gate) != GDR_OK) return GDR_EINVAL;
  gdr::RecurrentArgs a;
  a.N = N; a.H = H; a.D = Dk;
  a.in_bf16 = in_dtype == GDR_BF16; a.out_bf16 = out_dtype == GDR_BF16;
  a.gate = gate_kind(gate);
  a.erase = erases(gate);
  a.fuse = fuse;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
  a.out_gate = out_gate;
  a.state = state; a.o = o; a.stream = stream;
  hipError_t e = gdr::launch_recurrent_step(a);
  return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

}  // extern "C"
