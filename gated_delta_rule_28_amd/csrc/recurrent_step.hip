// Single-token decode step of the gated delta rule, fp32 state updated in place.
//
// Per (sequence, head) the step is (page "NLP——线性注意力相关总结", GDN and KDA
// sections; order decay -> predict -> write -> read as in the diosapp
// tutorial, section 四):
//     S' = a S  (or Diag(a) S)        p = S'^T k        d = beta (v - p)
//     S  = S' + k d^T                 o = S^T q = S'^T q + (k . q) d
// and without the erase term d = beta v (the additive write).
// The second form of o lets one pass over S produce both reductions before
// the write, so S is read once and written once: 2 * Dk * Dv * 4 bytes of
// HBM traffic per state, which is the whole cost of the step (HBM-bound).
//
// Work mapping: one workgroup per (sequence, head) state, 2*Dv threads.
// Thread t owns columns 4*(t % (Dv/4)) .. +3 and rows (t / (Dv/4)) * R .. +R-1
// with R = Dk / 8, so a wavefront reads whole 512-byte rows (Dv = 128) with
// 16-byte loads.  The eight row groups combine their partial p and S'^T q
// through LDS.  (Four groups of 32 rows with Dv threads measured 4% slower.)
#include "common.h"
#include "internal.h"

namespace gdr {

template <int DK, int DV, typename InT, typename OutT, int GATE>
__global__ void __launch_bounds__(2 * DV)
recurrent_step_kernel(const InT *__restrict__ q, const InT *__restrict__ k,
                      const InT *__restrict__ v, const float *__restrict__ beta,
                      const float *__restrict__ log_alpha, float *__restrict__ state,
                      OutT *__restrict__ o, bool erase, int fuse,
                      const InT *__restrict__ out_gate) {
  constexpr int NT = 2 * DV;          // threads per state
  constexpr int C4 = DV / 4;          // float4 columns per row
  constexpr int RG = NT / C4;         // row groups (= 8)
  constexpr int R = DK / RG;          // rows per thread
  static_assert(RG == 8 && R * RG == DK, "decode mapping");

  const int t = threadIdx.x;
  const int c4 = t % C4;
  const int rg = t / C4;
  const long sid = blockIdx.x;        // (n * H + h)

  __shared__ float s_k[DK], s_q[DK], s_la[DK];
  __shared__ float s_part[RG][2][DV];
  __shared__ float s_kq[RG];
  __shared__ float s_nrm[2];          // fused L2 normalisation: 1 / |k|, 1 / |q|

  float *S = state + sid * (long)DK * DV;
  // issue the state loads first: they are the whole cost of the step.  The
  // state is touched once per step, so its loads and stores are
  // non-temporal (streamed past the caches; measured ~8% more HBM
  // throughput for this in-place pattern)
  f32x4 s[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (long)(rg * R + i) * DV + 4 * c4));

  for (int i = t; i < DK; i += NT) {
    s_k[i] = to_f32(k[sid * DK + i]);
    s_q[i] = to_f32(q[sid * DK + i]);
    if (GATE == kGateChannel) s_la[i] = fused_log_alpha(log_alpha[sid * DK + i], fuse);
  }
  const float b = fused_beta(beta[sid], fuse);
  float a_head = 1.0f;
  if (GATE == kGateScalar) a_head = __expf(fused_log_alpha(log_alpha[sid], fuse));
  __syncthreads();
  float rk = 1.0f, rq = 1.0f;
  if (fuse & kFuseL2) {
    // |k|^2 and |q|^2 by the first WL threads (lane-strided sums, then a
    // butterfly over exactly those lanes: a workgroup smaller than a wave
    // has no other lanes to read)
    constexpr int WL = NT < 64 ? NT : 64;
    if (t < WL) {
      float sk = 0.f, sq2 = 0.f;
      for (int i = t; i < DK; i += WL) {
        sk += s_k[i] * s_k[i];
        sq2 += s_q[i] * s_q[i];
      }
#pragma unroll
      for (int m = WL / 2; m > 0; m >>= 1) {
        sk += __shfl_xor(sk, m, WL);
        sq2 += __shfl_xor(sq2, m, WL);
      }
      if (t == 0) {
        s_nrm[0] = rsqrtf(sk + kL2Eps);
        s_nrm[1] = rsqrtf(sq2 + kL2Eps);
      }
    }
    __syncthreads();
    rk = s_nrm[0];
    rq = s_nrm[1];
  }

  f32x4 p = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = rg * R + i;
    float a = a_head;
    if (GATE == kGateChannel) a = __expf(s_la[row]);
    s[i] *= a;                                   // S' = decayed state
    const float kr = s_k[row] * rk, qr = s_q[row] * rq;
    p += kr * s[i];
    sq += qr * s[i];
    kq += kr * qr;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s_part[rg][0][4 * c4 + j] = p[j];
    s_part[rg][1][4 * c4 + j] = sq[j];
  }
  if (c4 == 0) s_kq[rg] = kq;
  __syncthreads();

  f32x4 pt = {0.f, 0.f, 0.f, 0.f}, st = {0.f, 0.f, 0.f, 0.f};
  float kqt = 0.f;
#pragma unroll
  for (int g = 0; g < RG; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pt[j] += s_part[g][0][4 * c4 + j];
      st[j] += s_part[g][1][4 * c4 + j];
    }
    kqt += s_kq[g];
  }
  f32x4 vv, d;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vv[j] = to_f32(v[sid * DV + 4 * c4 + j]);
    d[j] = b * (erase ? vv[j] - pt[j] : vv[j]);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float kr = s_k[rg * R + i] * rk;
    __builtin_nontemporal_store(s[i] + kr * d, reinterpret_cast<f32x4 *>(S + (long)(rg * R + i) * DV + 4 * c4));
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = st[j] + kqt * d[j];
      if (out_gate) x = silu_gate(x, to_f32(out_gate[sid * DV + 4 * c4 + j]));
      o[sid * DV + 4 * c4 + j] = from_f32<OutT>(x);
    }
  }
}

template <int D, typename InT, typename OutT, int GATE>
static hipError_t launch_one(const RecurrentArgs &a) {
  dim3 grid((unsigned)((long)a.N * a.H)), block(2 * D);
  hipLaunchKernelGGL((recurrent_step_kernel<D, D, InT, OutT, GATE>), grid, block, 0, a.stream,
                     (const InT *)a.q, (const InT *)a.k, (const InT *)a.v, a.beta, a.log_alpha,
                     a.state, (OutT *)a.o, a.erase, a.fuse, (const InT *)a.out_gate);
  return hipGetLastError();
}

template <int D, typename InT, typename OutT>
static hipError_t by_gate(const RecurrentArgs &a) {
  switch (a.gate) {
    case kGateNone: return launch_one<D, InT, OutT, kGateNone>(a);
    case kGateScalar: return launch_one<D, InT, OutT, kGateScalar>(a);
    default: return launch_one<D, InT, OutT, kGateChannel>(a);
  }
}

template <int D>
static hipError_t by_dtype(const RecurrentArgs &a) {
  if (a.in_bf16) return a.out_bf16 ? by_gate<D, bf16, bf16>(a) : by_gate<D, bf16, float>(a);
  return a.out_bf16 ? by_gate<D, float, bf16>(a) : by_gate<D, float, float>(a);
}

hipError_t launch_recurrent_step(const RecurrentArgs &a) {
  switch (a.D) {
    case 16: return by_dtype<16>(a);
    case 32: return by_dtype<32>(a);
    case 64: return by_dtype<64>(a);
    default: return by_dtype<128>(a);
  }
}

}  // namespace gdr
