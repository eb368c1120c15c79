// Chunkwise KDA forward (per-channel decay), bf16 q/k/v, fp32 state, MFMA (gfx950).
//
// Method.  S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t, a_t in [0,1]^{d_k} (page "NLP——线性注意力相关总结", section
// "Kimi Delta Attention (KDA)"), evaluated chunkwise with the WY form and a
// triangular solve (xhh.club digest "Transformer 入坑笔记（五）", KDA Q&A).
// Per chunk of C = 16 tokens, entering state S, G = in-chunk cumulative
// log decay per (token, channel), g_last its last row:
//
//   A_rs = b_r sum_c k_rc k_sc e^{G_rc - G_sc}   (s < r)      Gram
//   P_rs =     sum_c q_rc k_sc e^{G_rc - G_sc}   (s <= r)     masked scores
//   T'   = (I + A)^{-1} diag(b)
//   U    = T' (V - (K o e^G) S)
//   O    = (Q o e^G) S + P U
//   S   <- Diag(e^{g_last}) S + (K o e^{g_last - G})^T U
//
// Every decay factor in the state products is <= 1 (G is relative to the
// chunk start and decreasing), so K o e^G, Q o e^G and K o e^{g_last - G}
// never overflow.  They are not exact bf16 values, so the state products
// use three MFMAs (hi*hi + hi*lo + lo*hi).
//
// The in-chunk Gram and scores need e^{G_r - G_s} per channel.  The page
// digest notes that these decays can be tiny, so direct division is
// unstable and a log-space, two-level scheme is used.  Here they factor
// about the chunk start: e^{G_r - G_s} = e^{G_r} e^{-G_s}, so the Gram is
// (K o e^G)(K o e^{-G})^T and the scores (Q o e^G)(K o e^{-G})^T, reusing
// the state-side operands on the left.  e^{-G_s} <= e^{-g_last}, so while
// every channel's in-chunk log decay stays above -64 the factored operands
// stay inside the fp32/bf16 range.  A chunk with a channel below that (a
// near-hard reset) takes an exact path instead: every (r, s, c) decay is
// formed directly in fp32.
//
// Mapping as in the scalar-gate kernel: one workgroup per (batch, head, Dv
// slice); DVS/16 state waves keep the state in MFMA accumulators; 4 prep
// waves run two chunks ahead:
//   X(i): waves 0, 1, 3 write chunk i (the threads that own a channel's log
//         decays sum them as they write) and load chunk i+1; wave 2 forms A
//         and solves it, wave 3 forms P, of chunk i-1
//   Y(i): all prep waves derive the decayed operands of chunk i
//   state: chunk i-2 (operand buffers three deep, T' two deep).
#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace gdr {
namespace {

constexpr int KC = 16;               // tokens per chunk
constexpr int KNPW = 4;              // prep waves
constexpr float kMaxSpan = 64.0f;    // per-channel in-chunk log-decay bound of the factored Gram

template <int DK, int DVS>
struct __align__(16) KdaSmem {
  static constexpr int LDK = DK + 8;      // bf16 stride of [16][DK] tiles read by rows
  static constexpr int LDC = DK + 16;     // bf16 stride of C, read transposed (8 rows x 8 banks)
  static constexpr int LDG = DK + 4;      // fp32 stride of G
  static constexpr int LDV = DVS + 16;    // bf16 stride of v rows, read transposed
  static constexpr int LDT = KC;          // bf16 stride of 16x16 tiles, read transposed
  struct __align__(16) Raw {              // staged chunk, natural channel order
    bf16 Q[KC][LDK], K[KC][LDK];
    float G[KC][LDG];                     // log a, then its in-chunk cumulative sum
    float beta[KC];
    int extreme[2];                       // per summing wave: some channel's in-chunk
                                          // log decay < -kMaxSpan
  };
  struct __align__(16) Der {              // operands of one chunk
    bf16 Kh[KC][LDK], Kl[KC][LDK];        // K o e^G, dk permuted
    bf16 Qh[KC][LDK], Ql[KC][LDK];        // Q o e^G, dk permuted
    bf16 Ch[KC][LDC], Cl[KC][LDC];        // K o e^{g_last - G}, natural order
    bf16 Ph[KC][LDT], Pl[KC][LDT];        // P^T: [s][r] = P[r][s]
    float egl[DK];                        // e^{g_last}
  };
  Raw raw[2];
  bf16 V[3][KC][LDV];                     // v rows of this slice, natural order
  Der der[3];
  bf16 Rkh[KC][LDK], Rkl[KC][LDK];        // K o e^{-G}, dk permuted (right operand of A and P)
  float AT[16][20];                       // A^T for the solve
  bf16 Th[2][KC][LDT], Tl[2][KC][LDT];    // T'^T
};

template <int DK, int DVS, typename OutT>
__global__ void __launch_bounds__(64 * (DVS / 16 + KNPW), 1)
chunk_fwd_kda_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                     const bf16 *__restrict__ v, const float *__restrict__ beta,
                     const float *__restrict__ log_alpha, const float *initial_state,
                     OutT *__restrict__ o, float *final_state, int B, int T, int H) {
  constexpr int NSW = DVS / 16;
  constexpr int DV = DK;
  constexpr int NSLICE = DV / DVS;
  constexpr int KKD = DK / 32;
  static_assert((DK == 64 || DK == 128) && (DVS == 32 || DVS == 64) && DVS <= DK, "tile config");
  using SM = KdaSmem<DK, DVS>;
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;

  const int nchain = B * H;
  int chain, slice;
  {
    const int w = blockIdx.x;
    if ((nchain & 7) == 0) {
      chain = ((w >> 3) / NSLICE) * 8 + (w & 7);
      slice = (w >> 3) % NSLICE;
    } else {
      chain = w / NSLICE;
      slice = w % NSLICE;
    }
  }
  const int bb = chain / H, hh = chain % H;
  const int nchunks = (T + KC - 1) / KC;
  const long tok0 = (long)bb * T * H + hh;   // token row of token 0 of this chain
  const long ntok = (long)B * T * H;         // token rows of every input tensor
  const bf16x4 zero4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};

  if (wave < NSW) {
    // =====================================================================
    // state waves
    // =====================================================================
    const int col0 = slice * DVS + 16 * wave;
    f32x4 Sacc[DK / 16];
#pragma unroll
    for (int mb = 0; mb < DK / 16; ++mb) Sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (initial_state) {
      const float *S0 = initial_state + (long)chain * DK * DV;
#pragma unroll
      for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[mb][e] = S0[(long)(16 * mb + 4 * lg + e) * DV + col0 + lr];
    }
    // byte offsets of this lane's output values from a chunk's first row
    int ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ooff[e] = (int)sizeof(OutT) * ((4 * lg + e) * H * DV + col0 + lr);
    __syncthreads();

    for (int it = 0; it < nchunks + 2; ++it) {
      const int s = it - 2;
      f32x4 QS;
      bf16x4 uh4, ul4;
      if (s >= 0) {
        // ---- X: K^ S, Q^ S (three products each), R = V - K^ S, U = T' R ----
        const typename SM::Der &d = sm.der[s % 3];
        bf16x8 Sh[KKD], Sl[KKD];
#pragma unroll
        for (int kk = 0; kk < KKD; ++kk) {
          bf16x4 h0, l0, h1, l1;
          split4<false>(Sacc[2 * kk], h0, l0);
          split4<false>(Sacc[2 * kk + 1], h1, l1);
          Sh[kk] = cat(h0, h1);
          Sl[kk] = cat(l0, l1);
        }
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KKD; ++kk) {
          const bf16x8 kh = ld8(&d.Kh[lr][32 * kk + 8 * lg]);
          const bf16x8 kl = ld8(&d.Kl[lr][32 * kk + 8 * lg]);
          const bf16x8 qh = ld8(&d.Qh[lr][32 * kk + 8 * lg]);
          const bf16x8 ql = ld8(&d.Ql[lr][32 * kk + 8 * lg]);
          a1 = mfma_bf16(kh, Sh[kk], a1);
          a2 = mfma_bf16(qh, Sh[kk], a2);
          a1 = mfma_bf16(kh, Sl[kk], a1);
          a2 = mfma_bf16(qh, Sl[kk], a2);
          a1 = mfma_bf16(kl, Sh[kk], a1);
          a2 = mfma_bf16(ql, Sh[kk], a2);
        }
        QS = a2;
        // V[4 lg + c][16 wave + lr] by a transposing read
        const bf16x4 vv = ld_tr4(&sm.V[s % 3][4 * lg + (lr >> 2)][16 * wave + 4 * (lr & 3)]);
        f32x4 rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[e] = (float)vv[e] - a1[e];
        bf16x4 rh4, rl4;
        split4<false>(rr, rh4, rl4);
        // [T'h | T'l] against [Rh ; Rh] and [Rl ; 0]: slots (half, c) <-> token 4 lg + c
        const bf16x8 ta = cat(ld_tr4(&sm.Th[s & 1][4 * lg + (lr >> 2)][4 * (lr & 3)]),
                              ld_tr4(&sm.Tl[s & 1][4 * lg + (lr >> 2)][4 * (lr & 3)]));
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        u = mfma_bf16(ta, cat(rh4, rh4), u);
        u = mfma_bf16(ta, cat(rl4, zero4), u);
        split4<false>(u, uh4, ul4);
      }
      __syncthreads();
      if (s >= 0) {
        // ---- Y: O = Q^ S + P U; S <- Diag(e^{g_last}) S + (K o e^{g_last-G})^T U ----
        const typename SM::Der &d = sm.der[s % 3];
        const int t0 = s * KC, n = min(KC, T - t0);
        const bf16x8 pa = cat(ld_tr4(&d.Ph[4 * lg + (lr >> 2)][4 * (lr & 3)]),
                              ld_tr4(&d.Pl[4 * lg + (lr >> 2)][4 * (lr & 3)]));
        f32x4 acc = QS;
        acc = mfma_bf16(pa, cat(uh4, uh4), acc);
        acc = mfma_bf16(pa, cat(ul4, zero4), acc);
        // lane holds O rows 4 lg + e of column col0 + lr: stored straight from
        // the accumulator; rows past the end of the sequence are not written
        const long orow = (tok0 + (long)t0 * H) * DV;
        const rsrc_t ro = make_rsrc(o + orow, (long)sizeof(OutT) * (ntok * DV - orow));
        if (n == KC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) buf_st1(from_f32<OutT>(acc[e]), ro, ooff[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * lg + e < n) buf_st1(from_f32<OutT>(acc[e]), ro, ooff[e]);
        }
        const bf16x8 b1 = cat(uh4, uh4), b2 = cat(ul4, zero4);
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb) {
          const f32x4 eg4 = *reinterpret_cast<const f32x4 *>(&d.egl[16 * mb + 4 * lg]);
          const int c0 = 16 * mb + 4 * (lr & 3);
          const bf16x8 a = cat(ld_tr4(&d.Ch[4 * lg + (lr >> 2)][c0]),
                               ld_tr4(&d.Cl[4 * lg + (lr >> 2)][c0]));
          f32x4 sa = Sacc[mb] * eg4;
          sa = mfma_bf16(a, b1, sa);
          sa = mfma_bf16(a, b2, sa);
          Sacc[mb] = sa;
        }
      }
      __syncthreads();
    }

    if (final_state) {
      float *SF = final_state + (long)chain * DK * DV;
#pragma unroll
      for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) SF[(long)(16 * mb + 4 * lg + e) * DV + col0 + lr] = Sacc[mb][e];
    }
    return;
  }

  // =======================================================================
  // prep waves
  // =======================================================================
  const int pw = wave - NSW;
  const int pt = tid - 64 * NSW;       // 0..255
  // Staging runs on prep waves 0, 1 and 3; wave 2 (Gram and solve) runs a
  // loop of its own.  Waves 0 and 1 load k and q (item = RPI tokens x 8
  // columns, 64 items per matrix, so each wave reads one matrix through one
  // buffer descriptor); wave 3 loads v (item = 8 columns of one token) and
  // beta.  Thread c < Dk of waves 0 and 1 also loads the 16 log decays of
  // channel c and sums them as it writes them.  Loads are unconditional
  // inside each wave; rows past the end of the sequence read the next rows
  // (or zeros past the end of a tensor) and are zeroed when written to LDS.
  constexpr int DCS = DK / 8;
  constexpr int RPI = KC * DCS / 64;   // tokens per q/k item (4 at d = 128, 2 at d = 64)
  constexpr int VCS = DVS / 8;
  constexpr int NV = KC * VCS;         // v items (128 or 64)
  constexpr int NVS = NV / 64;         // v items per wave-3 thread
  static_assert(RPI * 64 == KC * DCS && NV % 64 == 0, "staging items");
  const bool is_k = pw == 0;
  const int q_r0 = RPI * (lane / DCS), q_c0 = 8 * (lane % DCS);
  int v_r[NVS], v_c0[NVS];
#pragma unroll
  for (int h = 0; h < NVS; ++h) {
    const int vi = lane + 64 * h;
    v_r[h] = vi / VCS;
    v_c0[h] = 8 * (vi % VCS);
  }
  // one set of 16-byte load slots per staging thread, whatever its tensor:
  // q/k rows on waves 0 and 1, v items on wave 3 (surplus slots re-load the
  // first item), so the staging loads are the same straight-line code on
  // every staging wave
  constexpr int NL = RPI > NVS ? RPI : NVS;
  int soff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    soff[i] = (pw < 2) ? 2 * ((q_r0 + (i < RPI ? i : 0)) * H * DK + q_c0)
                       : 2 * (v_r[i < NVS ? i : 0] * H * DV + slice * DVS + v_c0[i < NVS ? i : 0]);
  const bf16 *ssrc = pw == 0 ? k : (pw == 1 ? q : v);   // wave-uniform
  const int la_c = (pw == 1 && DK > 64) ? 64 + lane : lane;   // channel summed by this thread
  const bool sums = pw < 2 && 64 * pw + lane < DK;           // wave-uniform

  // operands of chunk j (its G was summed in phase X); all four prep waves
  // take a share: thread = (channel pair, tokens)
  auto derive = [&](int j) {
    const typename SM::Raw &rw = sm.raw[j & 1];
    typename SM::Der &d = sm.der[j % 3];
    constexpr int NCP = DK / 2;                 // channel pairs
    constexpr int TPG = KC * NCP / 256;         // tokens per thread
    const int cp = pt % NCP, tq = pt / NCP;
    const int c0 = 2 * cp;
    const f32x2 gl = *reinterpret_cast<const f32x2 *>(&rw.G[KC - 1][c0]);
    if (tq == 0) *reinterpret_cast<f32x2 *>(&d.egl[c0]) = f32x2{__expf(gl[0]), __expf(gl[1])};
    // e^{-g_last}: scales K o e^{g_last - G} to K o e^{-G}; it can overflow
    // only in chunks that take the exact Gram path, which do not read Rk
    const float eng0 = __expf(-gl[0]), eng1 = __expf(-gl[1]);
    const int pc = perm32(c0);
    auto put2 = [](bf16 *hi, bf16 *lo, float x0, float x1) {
      unsigned h, l;
      split2<false>(x0, x1, h, l);
      *reinterpret_cast<unsigned *>(hi) = h;
      *reinterpret_cast<unsigned *>(lo) = l;
    };
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int r = TPG * tq + i;
      const f32x2 g = *reinterpret_cast<const f32x2 *>(&rw.G[r][c0]);
      const float k0 = (float)rw.K[r][c0], k1 = (float)rw.K[r][c0 + 1];
      const float q0 = (float)rw.Q[r][c0], q1 = (float)rw.Q[r][c0 + 1];
      const float e0 = __expf(g[0]), e1 = __expf(g[1]);
      const float c0e = k0 * __expf(gl[0] - g[0]), c1e = k1 * __expf(gl[1] - g[1]);
      put2(&d.Kh[r][pc], &d.Kl[r][pc], k0 * e0, k1 * e1);
      put2(&d.Qh[r][pc], &d.Ql[r][pc], q0 * e0, q1 * e1);
      put2(&d.Ch[r][c0], &d.Cl[r][c0], c0e, c1e);
      put2(&sm.Rkh[r][pc], &sm.Rkl[r][pc], c0e * eng0, c1e * eng1);
    }
  };

  // lower 16x16 tile (X o e^G)-decayed Gram of chunk j: X = K (isq false)
  // or X = Q (isq true); lane holds rows 4 lg + e of column lr
  auto tile = [&](int j, bool isq) -> f32x4 {
    const typename SM::Raw &rw = sm.raw[j & 1];
    const typename SM::Der &d = sm.der[j % 3];
    const bool extreme = rw.extreme[0] | (DK > 64 ? rw.extreme[1] : 0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!extreme) {
      // (X o e^G)(K o e^{-G})^T with X = K or Q, in dk-permuted order; the
      // three products accumulate separately (independent MFMA chains)
      const bf16(*Lh)[SM::LDK] = isq ? d.Qh : d.Kh;
      const bf16(*Ll)[SM::LDK] = isq ? d.Ql : d.Kl;
      f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KKD; ++kk) {
        const bf16x8 ah = ld8(&Lh[lr][32 * kk + 8 * lg]);
        const bf16x8 al = ld8(&Ll[lr][32 * kk + 8 * lg]);
        const bf16x8 bh = ld8(&sm.Rkh[lr][32 * kk + 8 * lg]);
        const bf16x8 bl = ld8(&sm.Rkl[lr][32 * kk + 8 * lg]);
        acc = mfma_bf16(ah, bh, acc);
        a1 = mfma_bf16(ah, bl, a1);
        a2 = mfma_bf16(al, bh, a2);
      }
      acc += a1 + a2;
    } else {
      // exact: every decay e^{G_rc - G_sc} formed directly (s <= r only)
      const bf16(*X)[SM::LDK] = isq ? rw.Q : rw.K;
      const int sc = lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        float sum = 0.0f;
        if (sc <= r) {
          for (int c = 0; c < DK; ++c)
            sum += (float)X[r][c] * (float)rw.K[sc][c] * __expf(rw.G[r][c] - rw.G[sc][c]);
        }
        acc[e] = sum;
      }
    }
    return acc;
  };
  // P of chunk j (lower incl.), split hi/lo, transposed
  auto scores = [&](int j) {
    typename SM::Der &d = sm.der[j % 3];
    const f32x4 acc = tile(j, true);
    const int sc = lr, r0 = 4 * lg;
    f32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (sc <= r0 + e) ? acc[e] : 0.0f;
    bf16x4 h4, l4;
    split4<false>(val, h4, l4);
    *reinterpret_cast<bf16x4 *>(&d.Ph[sc][r0]) = h4;
    *reinterpret_cast<bf16x4 *>(&d.Pl[sc][r0]) = l4;
  };
  // A of chunk j (strict lower, times b), then T' = (I + A)^{-1} diag(b)
  auto gram_solve = [&](int j) {
    const typename SM::Raw &rw = sm.raw[j & 1];
    const f32x4 acc = tile(j, false);
    const int sc = lr, r0 = 4 * lg;
    f32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (sc < r0 + e) ? rw.beta[r0 + e] * acc[e] : 0.0f;
    *reinterpret_cast<f32x4 *>(&sm.AT[sc][r0]) = val;   // AT[s][r] = A[r][s]
    // T = (I + A)^{-1}, lane = column; right-looking forward substitution
    const int col = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.0f : 0.0f;
    // every needed entry of A^T is loaded before the dependent steps (the
    // scheduling barrier keeps the loads there)
    f32x4 a4[15][4];
#pragma unroll
    for (int s2 = 0; s2 < 15; ++s2)
#pragma unroll
      for (int q4 = (s2 + 1) / 4; q4 < 4; ++q4)
        a4[s2][q4] = *reinterpret_cast<const f32x4 *>(&sm.AT[s2][4 * q4]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 15; ++s2) {
#pragma unroll
      for (int r = s2 + 1; r < 16; ++r) x[r] -= a4[s2][r / 4][r % 4] * x[s2];
    }
    if (lane < 16) {
      const float bcol = rw.beta[col];
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      unsigned h8[2][4], l8[2][4];
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        split2<false>(x[r] * bcol, x[r + 1] * bcol, h8[r / 8][(r % 8) / 2], l8[r / 8][(r % 8) / 2]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        *reinterpret_cast<u32x4 *>(&sm.Th[j & 1][col][8 * hf]) = u32x4{h8[hf][0], h8[hf][1], h8[hf][2], h8[hf][3]};
        *reinterpret_cast<u32x4 *>(&sm.Tl[j & 1][col][8 * hf]) = u32x4{l8[hf][0], l8[hf][1], l8[hf][2], l8[hf][3]};
      }
    }
  };

  if (pw == 2) {
    // ---- Gram/solve wave: A and T' of chunk it-1 in phase X, a share of the
    //      derivation of chunk it in phase Y ----
    __syncthreads();
    for (int it = 0; it < nchunks + 2; ++it) {
      if (it >= 1 && it - 1 < nchunks) gram_solve(it - 1);
      __syncthreads();
      if (it < nchunks) derive(it);
      __syncthreads();
    }
    return;
  }

  // ---- staging waves 0, 1, 3 ----
  bf16x8 stg[NL];
  float stl[KC];                       // log decays of channel la_c, rows 0..15
  float stg_b = 0.f;
  auto stage_chunk = [&](int j) {
    const long row0 = tok0 + (long)j * KC * H;
    stg_b = buf_ld1f(make_rsrc(beta + row0, 4 * (ntok - row0)), 4 * (lane & (KC - 1)) * H);
    const rsrc_t r = make_rsrc(ssrc + row0 * DK, 2 * (ntok - row0) * DK);   // DK == DV
#pragma unroll
    for (int i = 0; i < NL; ++i) stg[i] = buf_ld8(r, soff[i]);
    const rsrc_t rl = make_rsrc(log_alpha + row0 * DK, 4 * (ntok - row0) * DK);
#pragma unroll
    for (int rr = 0; rr < KC; ++rr) stl[rr] = buf_ld1f(rl, 4 * (rr * H * DK + la_c));
  };
  auto zero_rows = [](bf16x8 x, bool z) -> bf16x8 {
    if (z) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) x[jj] = (bf16)0.0f;
    }
    return x;
  };

  if (nchunks > 0) stage_chunk(0);
  __syncthreads();

  for (int it = 0; it < nchunks + 2; ++it) {
    // ================= phase X =================
    // every load in flight is one of chunk it's, consumed right here: one
    // wait for all of them on every path
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (it < nchunks) {
      // write staged chunk it; padding tokens (past T) become zeros with log a = 0
      typename SM::Raw &rw = sm.raw[it & 1];
      const int n = min(KC, T - it * KC);
      if (pw < 2) {
        bf16(*dst)[SM::LDK] = is_k ? rw.K : rw.Q;
#pragma unroll
        for (int i = 0; i < RPI; ++i)
          *reinterpret_cast<bf16x8 *>(&dst[q_r0 + i][q_c0]) = zero_rows(stg[i], q_r0 + i >= n);
        if (sums) {
          // in-chunk cumulative log decay of channel la_c; flag the chunk
          // when the factored Gram could leave the floating-point range
          float acc = 0.0f;
#pragma unroll
          for (int rr = 0; rr < KC; ++rr) {
            acc += (rr < n) ? stl[rr] : 0.0f;
            rw.G[rr][la_c] = acc;
          }
          const unsigned long long bad = __ballot(acc < -kMaxSpan);
          if (lane == 0) rw.extreme[pw] = bad != 0ull;
        }
      } else {
#pragma unroll
        for (int h = 0; h < NVS; ++h)
          *reinterpret_cast<bf16x8 *>(&sm.V[it % 3][v_r[h]][v_c0[h]]) = zero_rows(stg[h], v_r[h] >= n);
        if (lane < KC) rw.beta[lane] = (lane < n) ? stg_b : 0.0f;
      }
      if (it + 1 < nchunks) stage_chunk(it + 1);
    }
    if (pw == 3 && it >= 1 && it - 1 < nchunks) scores(it - 1);
    __syncthreads();

    // ================= phase Y =================
    if (it < nchunks) derive(it);
    __syncthreads();
  }
}

template <int DK, int DVS, typename OutT>
hipError_t launch_kda(const ChunkArgs &a) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + KNPW));
  hipLaunchKernelGGL((chunk_fwd_kda_kernel<DK, DVS, OutT>), grid, block, 0, a.stream,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta, a.log_alpha,
                     a.initial_state, (OutT *)a.o, a.final_state, a.B, a.T, a.H);
  return hipGetLastError();
}

template <int DK, int DVS>
hipError_t kda_by_out(const ChunkArgs &a) {
  return a.out_bf16 ? launch_kda<DK, DVS, bf16>(a) : launch_kda<DK, DVS, float>(a);
}

}  // namespace

bool chunk_fwd_kda_supported(const ChunkArgs &a) {
  return a.in_bf16 && (a.D == 128 || a.D == 64) && a.gate == kGateChannel;
}

hipError_t launch_chunk_fwd_kda(const ChunkArgs &a) {
  const long chains = (long)a.B * a.H;
  if (a.D == 128) {
    if (chains * 2 >= 256) return kda_by_out<128, 64>(a);
    return kda_by_out<128, 32>(a);
  }
  if (chains >= 256) return kda_by_out<64, 64>(a);
  return kda_by_out<64, 32>(a);
}

}  // namespace gdr
