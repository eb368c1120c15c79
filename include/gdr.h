/*
 * gdr.h -- C ABI of the gated delta-rule forward pass for AMD MI355X (gfx950).
 *
 * The method (page "NLP——线性注意力相关总结", sections "Gated DeltaNet (GDN)"
 * and "Kimi Delta Attention (KDA)"; xhh.club digest "Transformer 入坑笔记（五）",
 * Q&A on Gated DeltaNet and KDA), per (batch, head) chain, token t:
 *
 *   GDN       S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
 *   DeltaNet  the same with a_t = 1
 *   KDA       S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T
 *   output    o_t = S_t^T q_t      (read after the token's own write)
 *
 * with a_t = exp(log_alpha_t) (one scalar per head, or one value per key
 * channel for KDA), b_t = beta_t, S in R^{Dk x Dv}.  No query scale, no
 * feature map and no normaliser are applied: q and k are used as given.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *    library allocates no device memory and keeps no global mutable state.
 *  - All tensors are dense, row-major, with the last dimension contiguous.
 *  - Every call is asynchronous on `stream` (NULL = the default stream).
 *  - Return value: GDR_OK (0) on success, a negative gdr_status otherwise.
 *    Arguments are validated on the host before anything is launched; a
 *    call that fails validation launches nothing and writes nothing.  A
 *    failed launch returns GDR_EHIP.  Device faults surface at the caller's
 *    next synchronisation.  No C++ exception crosses this interface.
 *  - Values are not checked on the device.  Preconditions: log_alpha is
 *    finite and <= 0 (-inf is not supported; a large negative value such as
 *    -50 gives a clean hard reset), beta is finite.  Non-finite inputs
 *    propagate only into the (batch, head) chain they belong to.
 *  - q, k, v, o and every state pointer must be 16-byte aligned; beta and
 *    log_alpha 4-byte aligned, except that gdr_chunk_fwd with
 *    GDR_GATE_CHANNEL needs log_alpha 16-byte aligned (GDR_EINVAL otherwise).
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 4

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_EINVAL = -1,       /* bad argument: null pointer, size <= 0, misaligned, gate mismatch */
  GDR_EUNSUPPORTED = -2, /* valid but not implemented: head size, chunk size, dtype combination */
  GDR_EHIP = -3,         /* the HIP runtime reported an error on launch */
  GDR_EWORKSPACE = -4    /* workspace missing, not 256-byte aligned, or smaller than
                            the matching *_workspace_bytes query */
} gdr_status;

typedef enum gdr_dtype {
  GDR_F32 = 0,
  GDR_BF16 = 1
} gdr_dtype;

typedef enum gdr_gate {
  GDR_GATE_NONE = 0,    /* a_t = 1 (DeltaNet); log_alpha must be NULL      */
  GDR_GATE_SCALAR = 1,  /* GDN: log_alpha [.., H], one value per head      */
  GDR_GATE_CHANNEL = 2, /* KDA: log_alpha [.., H, Dk], one per key channel */
  /* Flag OR'd into any gate: no erase term.  The write is additive,
   *   S_t = a_t S_{t-1} + b_t k_t v_t^T    (Diag(a_t) with the channel gate),
   * which is plain linear attention with no gate and b = 1, the Mamba-2 /
   * SSD decay with the scalar gate and GLA's with the channel gate (page
   * "NLP——线性注意力相关总结", section "Linear Attention"; xhh.club digest,
   * abstract and Q&A).  The same kernels run it without the triangular
   * solve. */
  GDR_NO_ERASE = 0x100
} gdr_gate;

/*
 * Prologue and epilogue fused into gdr_chunk_fwd_ex and gdr_recurrent_step_ex
 * (bit flags in `fuse`): the per-token transforms a layer applies around the
 * recurrence, so the inputs can be passed as the projections produce them.
 *   GDR_FUSE_QK_L2NORM    q, k <- x / sqrt(sum_i x_i^2 + 1e-6) per (token,
 *                         head): the feature map on q and k of
 *                         "线性注意力架构：机制、权衡与跨层路由", section 3,
 *                         eqs. (7)-(8), taken as L2 normalisation
 *   GDR_FUSE_BETA_SIGMOID beta holds a logit: b = 1 / (1 + e^{-beta}), b in
 *                         (0, 1) (xhh.club digest, Q&A on Gated DeltaNet)
 *   GDR_FUSE_DECAY_SOFTPLUS  log_alpha holds x: log a = -softplus(x), a in
 *                         (0, 1)
 *   GDR_FUSE_DECAY_GLA    log_alpha holds x: a = sigmoid(x)^{1/16},
 *                         log a = -softplus(-x) / 16 (GLA's gate, xhh.club
 *                         digest, Q&A on GLA's gate)
 * (the two decay flags exclude each other and need a gate).  The fused
 * epilogue is the SiLU output gate (diosapp tutorial, section 四): with
 * `out_gate` non-NULL ([.., Dv], in_dtype, 16-byte aligned)
 * o <- o * g * sigmoid(g), g = out_gate.
 */
typedef enum gdr_fuse {
  GDR_FUSE_QK_L2NORM = 1,
  GDR_FUSE_BETA_SIGMOID = 2,
  GDR_FUSE_DECAY_SOFTPLUS = 4,
  GDR_FUSE_DECAY_GLA = 8
} gdr_fuse;

/* ABI version of the loaded library (GDR_ABI_VERSION of the build). */
int gdr_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *gdr_status_str(int status);

/*
 * gdr_chunk_fwd -- forward pass over whole sequences, chunk by chunk.
 *
 * Defined by the recurrence above; computed chunkwise (matrix products
 * inside a chunk, the state carried from chunk to chunk, the in-chunk
 * recurrence resolved through a unit-lower-triangular solve -- xhh.club
 * digest, sections on chunked computation and the Gated DeltaNet / KDA
 * Q&A).  The result does not depend on `chunk` beyond rounding.
 *
 *   B, T, H      batch, tokens per sequence (any T >= 1), heads
 *   Dk, Dv       key / value head sizes (supported: Dk == Dv in {16, 32, 64, 128},
 *                bf16 or fp32 q/k/v; other combinations return
 *                GDR_EUNSUPPORTED; fp32 q/k/v and heads below 64 run a plain
 *                fp32 kernel, accurate to fp32 rounding).  With bf16
 *                q/k/v, no gate or the scalar gate and Dk = 128, H * Dk must
 *                stay below 34,000,000 (the kernel addresses one chunk's rows
 *                of a tensor with 32-bit offsets); with the per-channel
 *                gate the bound is 71,000,000 (the fp32 log decays of one
 *                16-token chunk).  Larger shapes return GDR_EUNSUPPORTED (at
 *                Dk = 64 they take the fp32 kernel)
 *   chunk        tokens per chunk: 0 = default, else 16, 32 or 64
 *   in_dtype     dtype of q, k, v (GDR_BF16 or GDR_F32)
 *   out_dtype    dtype of o (GDR_F32 or GDR_BF16)
 *   gate         GDR_GATE_NONE / _SCALAR / _CHANNEL, optionally | GDR_NO_ERASE
 *   q, k         [B, T, H, Dk] in_dtype
 *   v            [B, T, H, Dv] in_dtype
 *   beta         [B, T, H] fp32
 *   log_alpha    NULL iff gate == NONE; [B, T, H] fp32 (SCALAR) or
 *                [B, T, H, Dk] fp32 (CHANNEL)
 *   initial_state [B, H, Dk, Dv] fp32, or NULL for a zero state
 *   o            [B, T, H, Dv] out_dtype (written)
 *   final_state  [B, H, Dk, Dv] fp32, or NULL (not written).  May be the
 *                same pointer as initial_state (in-place carry); any other
 *                overlap between outputs and inputs is not allowed.
 *
 * Accuracy: fp32 state and fp32 accumulation throughout.  With bf16 q/k/v
 * every product whose operand is not an exact bf16 value is evaluated as a
 * sum of bf16 hi/lo parts, keeping errors near fp32 level.
 */
int gdr_chunk_fwd(int B, int T, int H, int Dk, int Dv, int chunk,
                  int in_dtype, int out_dtype, int gate,
                  const void *q, const void *k, const void *v,
                  const float *beta, const float *log_alpha,
                  const float *initial_state,
                  void *o, float *final_state,
                  hipStream_t stream);

/*
 * gdr_chunk_fwd_ex -- gdr_chunk_fwd with the fused prologue and epilogue
 * (`fuse` flags and `out_gate` [B, T, H, Dv] or NULL, as described above).
 * With fuse = 0 and out_gate = NULL it is gdr_chunk_fwd.  Unknown flag bits,
 * both decay flags, a decay flag without a gate or a misaligned out_gate
 * return GDR_EINVAL.
 */
int gdr_chunk_fwd_ex(int B, int T, int H, int Dk, int Dv, int chunk,
                     int in_dtype, int out_dtype, int gate, int fuse,
                     const void *q, const void *k, const void *v,
                     const float *beta, const float *log_alpha,
                     const void *out_gate,
                     const float *initial_state,
                     void *o, float *final_state,
                     hipStream_t stream);

/*
 * gdr_chunk_fwd_workspace_bytes -- device workspace gdr_chunk_fwd needs for
 * these arguments.  Always 0: every forward kernel keeps its intermediates
 * (chunk tiles, the triangular solve, the state) in registers and LDS, so
 * the forward entry points take no workspace argument.  Provided so that a
 * caller can size workspaces the same way for the forward and the backward.
 */
size_t gdr_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     int in_dtype, int out_dtype, int gate);

/*
 * gdr_chunk_bwd_workspace_bytes -- device workspace gdr_chunk_bwd needs for
 * these arguments: per (batch, head) chain and 32-token chunk, two Dk x Dv
 * fp32 states and two 32 x Dv fp32 tiles, 4 (2 Dk Dv + 64 Dv) bytes (2.5 GiB
 * for B = 8, H = 16, T = 4096, Dk = Dv = 128); with GDR_GATE_CHANNEL the
 * chunk is 16 tokens, 4 (2 Dk Dv + 32 Dv) bytes per chain and chunk (4.5 GiB
 * for B = 2, H = 32, T = 8192).  0 when the call is not supported or has no
 * tokens.
 */
size_t gdr_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     int in_dtype, int gate);

/*
 * gdr_chunk_bwd -- gradients of gdr_chunk_fwd (the backward pass of the
 * chunkwise forward, which training runs: diosapp tutorial, section 五;
 * "线性注意力架构：机制、权衡与跨层路由", abstract, on training throughput).
 *
 * Given L with dL/do = d_o and dL/dS_T = d_final_state, it returns the
 * gradients of L with respect to every input of the same forward call:
 *
 *   B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta, log_alpha,
 *   initial_state  exactly as passed to gdr_chunk_fwd.  Supported: bf16
 *                 q/k/v, Dk == Dv in {64, 128}, every gate, with or
 *                 without GDR_NO_ERASE (others return GDR_EUNSUPPORTED)
 *   d_o           [B, T, H, Dv] in_dtype, dL/do
 *   d_final_state [B, H, Dk, Dv] fp32, or NULL for zero
 *   dq, dk        [B, T, H, Dk] fp32 (written)
 *   dv            [B, T, H, Dv] fp32 (written)
 *   dbeta         [B, T, H] fp32 (written)
 *   dlog_alpha    shaped like log_alpha ([B, T, H], or [B, T, H, Dk] with
 *                 GDR_GATE_CHANNEL), fp32 (written); NULL iff gate ==
 *                 GDR_GATE_NONE
 *   d_initial_state [B, H, Dk, Dv] fp32 (written), or NULL (not written)
 *   workspace     device memory of at least gdr_chunk_bwd_workspace_bytes,
 *                 256-byte aligned, owned by the caller; its contents on entry
 *                 are ignored and on return are unspecified.  GDR_EWORKSPACE
 *                 if it is NULL, misaligned or smaller.
 *
 * The outputs must not overlap each other, the inputs or the workspace.  The
 * call recomputes the forward's chunk-boundary states into the workspace,
 * walks the chunks in reverse for the state gradient, then forms every
 * chunk's token gradients in parallel (three kernel launches on `stream`).
 * Accuracy as for gdr_chunk_fwd: fp32 state, hi/lo bf16 products.
 */
int gdr_chunk_bwd(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int gate,
                  const void *q, const void *k, const void *v,
                  const float *beta, const float *log_alpha,
                  const float *initial_state,
                  const void *d_o, const float *d_final_state,
                  float *dq, float *dk, float *dv, float *dbeta, float *dlog_alpha,
                  float *d_initial_state,
                  void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * gdr_chunk_bwd_ex -- gdr_chunk_bwd with the dtype of dq, dk and dv chosen,
 * and gdr_chunk_bwd_saved by a switch (the backward pass of training:
 * diosapp tutorial, section 五).  Training keeps each gradient in its
 * parameter's dtype; with grad_dtype = GDR_BF16 the kernels write bf16
 * gradients directly (half the bytes, and no cast afterwards).
 *
 *   B .. d_final_state  as gdr_chunk_bwd
 *   grad_dtype    GDR_F32 or GDR_BF16 (anything else: GDR_EINVAL): the dtype
 *                 of dq, dk [B, T, H, Dk] and dv [B, T, H, Dv], each the fp32
 *                 gradient rounded to nearest even.  dbeta, dlog_alpha and
 *                 d_initial_state stay fp32, the dtypes of beta, log_alpha
 *                 and the state
 *   dq .. workspace_bytes  as gdr_chunk_bwd (dq, dk, dv 16-byte aligned)
 *   saved         0: as gdr_chunk_bwd; nonzero: as gdr_chunk_bwd_saved (the
 *                 workspace holds what gdr_chunk_fwd_train stored)
 *
 * With grad_dtype = GDR_F32 it is gdr_chunk_bwd (saved = 0) or
 * gdr_chunk_bwd_saved, bit for bit.
 */
int gdr_chunk_bwd_ex(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype,
                     int grad_dtype, int gate,
                     const void *q, const void *k, const void *v,
                     const float *beta, const float *log_alpha,
                     const float *initial_state,
                     const void *d_o, const float *d_final_state,
                     void *dq, void *dk, void *dv, float *dbeta, float *dlog_alpha,
                     float *d_initial_state,
                     void *workspace, size_t workspace_bytes, int saved,
                     hipStream_t stream);

/*
 * gdr_chunk_fwd_train -- gdr_chunk_fwd for training: the same o and
 * final_state, and besides, into `workspace`, the per-chunk states and write
 * residuals that gdr_chunk_bwd's first pass would recompute, so that
 * gdr_chunk_bwd_saved can skip that pass (the forward pass of training, which
 * the backward follows: diosapp tutorial, section 五).
 *
 *   B .. final_state  as gdr_chunk_fwd, within gdr_chunk_bwd's supported set
 *                 (bf16 q/k/v, Dk == Dv in {64, 128}, every gate, with or
 *                 without GDR_NO_ERASE; others return GDR_EUNSUPPORTED);
 *                 no fused options
 *   workspace     device memory of at least gdr_chunk_bwd_workspace_bytes for
 *                 the same shape, chunk, dtype and gate, 256-byte aligned,
 *                 owned by the caller (GDR_EWORKSPACE otherwise).  Written:
 *                 the part gdr_chunk_bwd_saved reads; the rest is untouched.
 *
 * o is the forward's output to the forward's accuracy (for the scalar gate
 * the state is kept unscaled here, so the last bits of o may differ from
 * gdr_chunk_fwd's).  One kernel launch on `stream`.
 */
int gdr_chunk_fwd_train(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype,
                        int out_dtype, int gate, const void *q, const void *k, const void *v,
                        const float *beta, const float *log_alpha, const float *initial_state,
                        void *o, float *final_state, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * gdr_chunk_bwd_saved -- gdr_chunk_bwd after gdr_chunk_fwd_train: the same
 * arguments and results, with `workspace` holding what gdr_chunk_fwd_train
 * stored for the same inputs (q, k, v, beta, log_alpha, initial_state, gate
 * and shape) and unchanged since.  It skips the recompute pass (two kernel
 * launches).  Other workspace contents give meaningless gradients; nothing
 * is read outside the workspace and the inputs.
 */
int gdr_chunk_bwd_saved(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype, int gate,
                        const void *q, const void *k, const void *v,
                        const float *beta, const float *log_alpha,
                        const float *initial_state,
                        const void *d_o, const float *d_final_state,
                        float *dq, float *dk, float *dv, float *dbeta, float *dlog_alpha,
                        float *d_initial_state,
                        void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * gdr_chunk_bwd_noalloc -- gdr_chunk_bwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc.  Same arguments and results
 * without the workspace, which is a static device array of
 * GDR_NOALLOC_SCRATCH_BYTES inside the library (one per GPU the library runs
 * on, held until the process ends); the call allocates nothing.  A call whose
 * gdr_chunk_bwd_workspace_bytes exceeds GDR_NOALLOC_SCRATCH_BYTES (64 MiB:
 * 409 chain-chunks of 32 tokens at Dk = Dv = 128, such as B = 1, H = 4,
 * T = 3264; 455 chain-chunks of 16 tokens with GDR_GATE_CHANNEL) returns
 * GDR_EWORKSPACE and launches nothing.  Every call on a GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  The array's
 * contents between calls are unspecified; nothing in them is read before
 * the call writes it.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gdr_chunk_bwd_noalloc(int B, int T, int H, int Dk, int Dv, int chunk, int in_dtype,
                          int gate, const void *q, const void *k, const void *v,
                          const float *beta, const float *log_alpha,
                          const float *initial_state,
                          const void *d_o, const float *d_final_state,
                          float *dq, float *dk, float *dv, float *dbeta, float *dlog_alpha,
                          float *d_initial_state, hipStream_t stream);

/*
 * gdr_recurrent_step -- one decode step: a single new token for each of N
 * independent sequences, with the fp32 state updated IN PLACE (the
 * constant-size memory that replaces the KV cache; diosapp tutorial,
 * section 一, decoding cost independent of length).
 *
 *   N, H         sequences, heads
 *   Dk, Dv       head sizes (supported: Dk == Dv in {16, 32, 64, 128})
 *   in_dtype     dtype of q, k, v;  out_dtype  dtype of o
 *   gate         as above (GDR_NO_ERASE allowed)
 *   q, k         [N, H, Dk];  v [N, H, Dv]
 *   beta         [N, H] fp32
 *   log_alpha    NULL iff gate == NONE; [N, H] (SCALAR) or [N, H, Dk] (CHANNEL)
 *   state        [N, H, Dk, Dv] fp32, read and overwritten with S_t
 *   o            [N, H, Dv] out_dtype (written); must not overlap state
 */
int gdr_recurrent_step(int N, int H, int Dk, int Dv,
                       int in_dtype, int out_dtype, int gate,
                       const void *q, const void *k, const void *v,
                       const float *beta, const float *log_alpha,
                       float *state, void *o,
                       hipStream_t stream);

/*
 * gdr_recurrent_step_ex -- gdr_recurrent_step with the fused prologue and
 * epilogue (`fuse` flags and `out_gate` [N, H, Dv] or NULL, in_dtype,
 * 16-byte aligned, owned by the caller and only read).  With fuse = 0 and
 * out_gate = NULL it is gdr_recurrent_step.  Unknown flag bits, both decay
 * flags, a decay flag without a gate or a misaligned out_gate return
 * GDR_EINVAL before anything is launched.
 */
int gdr_recurrent_step_ex(int N, int H, int Dk, int Dv,
                          int in_dtype, int out_dtype, int gate, int fuse,
                          const void *q, const void *k, const void *v,
                          const float *beta, const float *log_alpha,
                          const void *out_gate,
                          float *state, void *o,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
