// Chunkwise gated delta-rule forward in plain fp32 arithmetic (VALU), for
// small heads (Dk = Dv <= 64) and for fp32 inputs (Dk = Dv <= 128), all
// three gates.
//
// Same chunk algebra as the MFMA kernel (xhh.club digest "Transformer 入坑笔记
// （五）": products inside a chunk, state carried between chunks, WY form via a
// triangular solve), with the solve done by forward substitution and every
// product evaluated in fp32 FMAs, so it is accurate to fp32 rounding for fp32
// inputs.  Per chunk of n tokens, entering state S, g = in-chunk cumulative
// log decay (a vector per token for the per-channel gate):
//
//   A_rs = b_r sum_c k_rc k_sc e^{g_rc - g_sc}        (s < r)
//   P_rs =     sum_c q_rc k_sc e^{g_rc - g_sc}        (s <= r)
//   (I + A) U = diag(b) (V - (K o e^G) S)             forward substitution
//   O  = (Q o e^G) S + P U
//   S <- Diag(e^{g_last}) S + (K o e^{g_last - G})^T U
//
// (page "NLP——线性注意力相关总结", sections on GDN and KDA; with the scalar
// gate every channel carries the same g, with no gate g = 0.)  One workgroup
// per (batch, head) chain; all intermediates live in LDS.
#include "common.h"
#include "internal.h"

namespace gdr {
namespace {

template <int D, int C>
struct SmemSmall {
  static constexpr int LD = D + 1;
  static constexpr int LC = C + 1;
  float Q[C][LD], K[C][LD], V[C][LD];
  float G[C][LD];      // cumulative log decay per (token, channel)
  float S[D][LD];      // state
  float A[C][LC], P[C][LC];
  float U[C][LD];      // R, then U (in place)
  float beta[C];
  float nrm[2][C];     // fused L2 normalisation: 1 / |q_r|, 1 / |k_r|
};

// q/k/v dtype and o dtype are runtime flags here: this path is about
// exactness, not speed, and it keeps the number of instantiations small.
__device__ __forceinline__ float load_in(const void *p, long i, bool bf) {
  return bf ? (float)((const bf16 *)p)[i] : ((const float *)p)[i];
}

template <int D, int C, int GATE>
__global__ void __launch_bounds__(256)
chunk_fwd_small_kernel(const void *__restrict__ q, const void *__restrict__ k,
                       const void *__restrict__ v, const float *__restrict__ beta,
                       const float *__restrict__ log_alpha, const float *initial_state,
                       void *__restrict__ o, float *final_state, int B, int T, int H,
                       bool in_bf16, bool out_bf16, bool erase, int fuse,
                       const void *__restrict__ out_gate) {
  constexpr int NT = 256;
  __shared__ SmemSmall<D, C> sm;
  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int bb = chain / H, hh = chain % H;

  for (int i = tid; i < D * D; i += NT) {
    const int m = i / D, c = i % D;
    sm.S[m][c] = initial_state ? initial_state[(long)chain * D * D + i] : 0.0f;
  }

  for (int t0 = 0; t0 < T; t0 += C) {
    const int n = min(C, T - t0);
    __syncthreads();
    for (int i = tid; i < C * D; i += NT) {
      const int r = i / D, c = i % D;
      float qv = 0.f, kv = 0.f, vv = 0.f, la = 0.f;
      if (r < n) {
        const long row = ((long)bb * T + t0 + r) * H + hh;
        qv = load_in(q, row * D + c, in_bf16);
        kv = load_in(k, row * D + c, in_bf16);
        vv = load_in(v, row * D + c, in_bf16);
        if (GATE == kGateScalar) la = fused_log_alpha(log_alpha[row], fuse);
        if (GATE == kGateChannel) la = fused_log_alpha(log_alpha[row * D + c], fuse);
      }
      sm.Q[r][c] = qv;
      sm.K[r][c] = kv;
      sm.V[r][c] = vv;
      sm.G[r][c] = la;
    }
    for (int r = tid; r < C; r += NT)
      sm.beta[r] = r < n ? fused_beta(beta[((long)bb * T + t0 + r) * H + hh], fuse) : 0.0f;
    __syncthreads();
    if (fuse & kFuseL2) {
      // q, k rows scaled to unit norm (padded rows stay zero)
      for (int i = tid; i < 2 * C; i += NT) {
        const int r = i % C;
        const float(*X)[SmemSmall<D, C>::LD] = i < C ? sm.Q : sm.K;
        float ss = 0.f;
        for (int c = 0; c < D; ++c) ss += X[r][c] * X[r][c];
        sm.nrm[i / C][r] = rsqrtf(ss + kL2Eps);
      }
      __syncthreads();
      for (int i = tid; i < C * D; i += NT) {
        const int r = i / D, c = i % D;
        sm.Q[r][c] *= sm.nrm[0][r];
        sm.K[r][c] *= sm.nrm[1][r];
      }
      __syncthreads();
    }
    // cumulative log decay down each channel (padded tokens carry 0), the
    // column loaded into registers first
    for (int c = tid; c < D; c += NT) {
      float gc[C];
#pragma unroll
      for (int r = 0; r < C; ++r) gc[r] = sm.G[r][c];
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        acc += gc[r];
        sm.G[r][c] = acc;
      }
    }
    __syncthreads();
    // A and P
    for (int i = tid; i < C * C; i += NT) {
      const int r = i / C, s = i % C;
      float a = 0.f, p = 0.f;
      if (s <= r) {
        for (int c = 0; c < D; ++c) {
          const float dec = (GATE == kGateNone) ? 1.0f : __expf(sm.G[r][c] - sm.G[s][c]);
          const float ks = sm.K[s][c] * dec;
          a += sm.K[r][c] * ks;
          p += sm.Q[r][c] * ks;
        }
      }
      // without the erase term A = 0: the solve below leaves U = diag(b) V
      sm.A[r][s] = (erase && s < r) ? sm.beta[r] * a : 0.0f;
      sm.P[r][s] = p;
    }
    // R = V - (K o e^G) S (R = V without the erase term)
    for (int i = tid; i < C * D; i += NT) {
      const int r = i / D, c = i % D;
      float acc = 0.f;
      for (int m = 0; erase && m < D; ++m) {
        const float x = (GATE == kGateNone) ? sm.K[r][m] : sm.K[r][m] * __expf(sm.G[r][m]);
        acc += x * sm.S[m][c];
      }
      sm.U[r][c] = sm.V[r][c] - acc;
    }
    __syncthreads();
    // (I + A) U = diag(b) R by forward substitution, one lane per column,
    // the column kept in registers (A is read by broadcast, U never goes
    // back to LDS until the column is done)
    if (tid < 64) {
      for (int c = tid; c < D; c += 64) {
        // right-looking: once u[s] is final it updates every later row, so
        // the dependent chain is one FMA per step and the rows' updates are
        // independent
        float u[C];
#pragma unroll
        for (int r = 0; r < C; ++r) u[r] = sm.beta[r] * sm.U[r][c];
#pragma unroll
        for (int s2 = 0; s2 < C - 1; ++s2) {
#pragma unroll
          for (int r = s2 + 1; r < C; ++r) u[r] -= sm.A[r][s2] * u[s2];
        }
#pragma unroll
        for (int r = 0; r < C; ++r) sm.U[r][c] = u[r];
      }
    }
    __syncthreads();
    // O = (Q o e^G) S + P U
    for (int i = tid; i < C * D; i += NT) {
      const int r = i / D, c = i % D;
      if (r >= n) continue;
      float acc = 0.f;
      for (int m = 0; m < D; ++m) {
        const float x = (GATE == kGateNone) ? sm.Q[r][m] : sm.Q[r][m] * __expf(sm.G[r][m]);
        acc += x * sm.S[m][c];
      }
      for (int s = 0; s <= r; ++s) acc += sm.P[r][s] * sm.U[s][c];
      const long oi = (((long)bb * T + t0 + r) * H + hh) * D + c;
      if (out_gate) acc = silu_gate(acc, load_in(out_gate, oi, in_bf16));
      if (out_bf16) ((bf16 *)o)[oi] = (bf16)acc;
      else ((float *)o)[oi] = acc;
    }
    __syncthreads();
    // S <- Diag(e^{g_last}) S + (K o e^{g_last - G})^T U
    for (int i = tid; i < D * D; i += NT) {
      const int m = i / D, c = i % D;
      const float gl = sm.G[C - 1][m];
      float acc = (GATE == kGateNone) ? sm.S[m][c] : __expf(gl) * sm.S[m][c];
      for (int r = 0; r < C; ++r) {
        const float x = (GATE == kGateNone) ? sm.K[r][m] : sm.K[r][m] * __expf(gl - sm.G[r][m]);
        acc += x * sm.U[r][c];
      }
      sm.S[m][c] = acc;
    }
  }
  __syncthreads();
  if (final_state)
    for (int i = tid; i < D * D; i += NT) final_state[(long)chain * D * D + i] = sm.S[i / D][i % D];
}

template <int D, int C>
hipError_t by_gate(const ChunkArgs &a) {
  dim3 grid((unsigned)(a.B * a.H)), block(256);
#define GDR_LAUNCH(G)                                                                          \
  hipLaunchKernelGGL((chunk_fwd_small_kernel<D, C, G>), grid, block, 0, a.stream, a.q, a.k,  \
                     a.v, a.beta, a.log_alpha, a.initial_state, a.o, a.final_state, a.B, a.T, \
                     a.H, a.in_bf16, a.out_bf16, a.erase, a.fuse, a.out_gate)
  if (a.gate == kGateNone) GDR_LAUNCH(kGateNone);
  else if (a.gate == kGateScalar) GDR_LAUNCH(kGateScalar);
  else GDR_LAUNCH(kGateChannel);
#undef GDR_LAUNCH
  return hipGetLastError();
}

template <int D>
hipError_t by_chunk(const ChunkArgs &a) {
  // the chunk only changes rounding; at D = 128 the kernel's LDS holds
  // 16-token chunks (about 109 KB: the state and five 16 x 129 fp32 tiles)
  if constexpr (D == 128) {
    return by_gate<D, 16>(a);
  } else {
    const int c = a.chunk ? a.chunk : (D <= 16 ? 16 : 64);
    if (c == 16) return by_gate<D, 16>(a);
    if (c == 32) return by_gate<D, 32>(a);
    return by_gate<D, 64>(a);
  }
}

}  // namespace

bool chunk_fwd_small_supported(const ChunkArgs &a) {
  return (a.D == 16 || a.D == 32 || a.D == 64 || (a.D == 128 && !a.in_bf16)) &&
         (a.chunk == 0 || a.chunk == 16 || a.chunk == 32 || a.chunk == 64);
}

hipError_t launch_chunk_fwd_small(const ChunkArgs &a) {
  switch (a.D) {
    case 16: return by_chunk<16>(a);
    case 32: return by_chunk<32>(a);
    case 64: return by_chunk<64>(a);
    default: return by_chunk<128>(a);
  }
}

}  // namespace gdr
