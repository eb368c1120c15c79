// Chunkwise gated delta-rule forward, bf16 q/k/v, fp32 state, MFMA (gfx950).
//
// Method.  The recurrence S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t (page "NLP——线性注意力相关总结", section "Gated DeltaNet
// (GDN)"; a_t = 1 is DeltaNet, section "DeltaNet") is evaluated chunk by
// chunk: matrix products inside a chunk, the state passed between chunks,
// and the in-chunk recurrence resolved by a triangular solve in WY form
// (xhh.club digest "Transformer 入坑笔记（五）", sections on chunked computation
// and the Gated DeltaNet Q&A).  For a chunk of C tokens with entering state S,
// g = in-chunk cumulative log decay, gam = e^g, Gam_rs = e^{g_r - g_s}:
//
//   A   = strict_lower(diag(b) (K K^T o Gam))         Gram of the keys
//   T'  = (I + A)^{-1} diag(b)                         unit-lower solve (WY)
//   P   = lower_incl(Q K^T o Gam)                      masked scores
//   U   = T' (V - diag(gam) K S)                       written residuals
//   O   = diag(gam) Q S + P U                          outputs
//   S  <- gam_last S + K^T diag(e^{g_last - g}) U      carried state
//
// Mapping.  One workgroup per (batch, head, Dv-slice of DVS columns): the Dv
// columns of S, U and O are independent given K, b and g.  The workgroup is
// a two-stage software pipeline over chunks of C = 32 tokens:
//
//   state waves (DVS/16 of them) each own 16 state columns and keep them in
//     MFMA accumulators for the whole sequence.  Every state-dependent
//     product (K S, Q S, T'R, P U, K^T U') takes its right operand straight
//     from accumulator registers: an accumulator tile holds rows 4g..4g+3 of
//     column l&15, which is what a 16x16x32 B operand needs once the k order
//     inside each 32-block is permuted (the left operands in LDS are stored
//     with the same permutation).  The serial chain never touches LDS.
//   prep waves (4) run ahead on the key-only work: they stage chunk i+1
//     from HBM in registers while writing chunk i to LDS with its decay
//     cumsum, form K K^T / Q K^T with the decay (A and P), and solve (I + A).
//
// Iteration i has two phases separated by workgroup barriers:
//   X: prep writes chunk i (+ cumsum) and loads i+1; solves the diagonal
//      16x16 blocks of (I + A) of chunk i-1     | state: K S, Q S, U of chunk i-2
//   Y: prep forms the A and P tiles of chunk i and the off-diagonal block
//      of T' of chunk i-1                        | state: O, S update of chunk i-2
// so a chunk buffer lives three iterations (NBUF = 3), T' two.
//
// Precision.  q, k, v are exact bf16 and enter MFMAs unsplit; every derived
// operand (S, R, U, T', P) is split into bf16 hi + lo and multiplied as
// hi*hi + hi*lo + lo*hi (two products when the other side is exact), so
// products carry ~16 significant bits and accumulate in fp32.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace gdr {
namespace {

constexpr int C = 32;      // tokens per chunk
constexpr int NPW = 4;     // prep waves
constexpr int NBUF = 3;    // chunk buffers: a chunk is written 2 iterations before its state pass

// Inclusive prefix sum over lanes 0..31 of a wave with DPP row shifts
// (within 16-lane rows) and a row broadcast of lane 15 into the next row.
// Lanes 32..63 carry values that are not used.
__device__ __forceinline__ float scan32_inclusive(float x) {
  auto shr = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 decltype(ctrl)::value, 0xF, 0xF, true));
  };
  x += shr(x, std::integral_constant<int, 0x111>{});   // row_shr:1
  x += shr(x, std::integral_constant<int, 0x112>{});   // row_shr:2
  x += shr(x, std::integral_constant<int, 0x114>{});   // row_shr:4
  x += shr(x, std::integral_constant<int, 0x118>{});   // row_shr:8
  // row_bcast:15 into rows 1 and 3; rows 0 and 2 add 0
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142,
                                                             0xA, 0xF, false));
  return x;
}

template <int DK, int DVS>
struct __align__(16) PipeSmem {
  static constexpr int LDK = DK + 8;   // bf16 stride of [C][DK] rows (pads banks)
  static constexpr int LDV = DVS + 16; // bf16 stride of [C][DVS] rows (transposing reads
                                       // of 8 rows hit 64 distinct banks)
  static constexpr int LDC = C + 16;   // bf16 stride of [*][C] rows (likewise)
  struct __align__(16) Buf {           // one chunk, live for four iterations
    bf16 Q[C][LDK];                    // q rows, dk permuted
    bf16 K[C][LDK];                    // k rows, dk permuted
    bf16 V[C][LDV];                    // v rows of this slice, natural order
    bf16 Ph[C][LDC], Pl[C][LDC];       // P^T: [s][r] = P[r][s]; rows 16..31 x cols 0..15 stay zero
    float gam[C], ec[C], beta[C], g[C];
  };
  Buf buf[NBUF];
  float ATd[2][16][20];                // diagonal 16x16 blocks of A, transposed: [b][s][r] = A[16b+r][16b+s]
  float A10[2][16][20];                // block (1,0) of A, row-major
  bf16 Th[2][C][LDC], Tl[2][C][LDC];   // T'^T: [s][r] = T'[r][s], T' = (I+A)^{-1} diag(b);
                                       // rows 16..31 x cols 0..15 stay zero
  float TdT[2][16][20];                // diagonal blocks of T = (I+A)^{-1}, transposed:
                                       // [b][c][r] = T[16b+r][16b+c] (solver output)
  float X[16][20];                     // X^T (solver scratch)
};

template <int DK, int DVS, typename OutT, int GATE>
__global__ void __launch_bounds__(64 * (DVS / 16 + NPW), 1)
chunk_fwd_bf16_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                      const bf16 *__restrict__ v, const float *__restrict__ beta,
                      const float *__restrict__ log_alpha, const float *initial_state,
                      OutT *__restrict__ o, float *final_state, int B, int T, int H) {
  constexpr int NSW = DVS / 16;        // state waves; wave w owns value columns 16w..16w+15
  constexpr int NT = 64 * (NSW + NPW);
  constexpr int DV = DK;               // full value width (Dk == Dv)
  constexpr int NSLICE = DV / DVS;
  constexpr int KKD = DK / 32;         // 32-deep k steps over dk
  constexpr int VCS = DVS / 8;         // 8-column segments of the value slice
  static_assert((DK == 64 || DK == 128) && (DVS == 32 || DVS == 64) && DVS <= DK, "tile config");
  using SM = PipeSmem<DK, DVS>;
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: the role split below is a uniform branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;

  // workgroup -> (chain, slice); slices of one chain share an XCD (same L2)
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
  const int nchunks = (T + C - 1) / C;
  const long tok0 = (long)bb * T * H + hh;   // row index of token 0 of this chain

  // the upper-right 16x16 blocks of P and T' are never written: zero once
  for (int i = tid; i < C * SM::LDC; i += NT) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      (&sm.buf[b].Ph[0][0])[i] = (bf16)0.0f;
      (&sm.buf[b].Pl[0][0])[i] = (bf16)0.0f;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      (&sm.Th[b][0][0])[i] = (bf16)0.0f;
      (&sm.Tl[b][0][0])[i] = (bf16)0.0f;
    }
  }

  // Both roles run nchunks + 2 iterations with two barriers each, so every
  // wave executes the same sequence of workgroup barriers.
  if (wave < NSW) {
    // =====================================================================
    // state waves: the serial chunk-to-chunk pass, 16 state columns each
    // =====================================================================
    const int col0 = slice * DVS + 16 * wave;   // first value column of this wave
    // S columns col0 + lr, rows 16 mb + 4 lg + e
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
    __syncthreads();

    // byte offsets of this lane's output values from a chunk's first row
    int ooff[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ooff[rb][e] = (int)sizeof(OutT) * ((16 * rb + 4 * lg + e) * H * DV + col0 + lr);

    // hi/lo bf16 split of the state, the right operand of K S and Q S; it
    // is formed at the end of the previous phase Y, as soon as S is final
    bf16x8 Sh[KKD], Sl[KKD];
    auto split_state = [&]() {
#pragma unroll
      for (int kk = 0; kk < KKD; ++kk) {
        bf16x4 h0, l0, h1, l1;
        split4(Sacc[2 * kk], h0, l0);
        split4(Sacc[2 * kk + 1], h1, l1);
        Sh[kk] = cat(h0, h1);
        Sl[kk] = cat(l0, l1);
      }
    };
    split_state();

    for (int it = 0; it < nchunks + 2; ++it) {
      const int s = it - 2;            // chunk of this iteration
      f32x4 QS[2];                     // carried from phase X to phase Y
      bf16x8 Uh, Ul, Wh, Wl;
      // ---- phase X: K S, Q S, R = V - diag(gam) K S, U = T' R ----
      if (s >= 0) {
        const typename SM::Buf &bs = sm.buf[s % NBUF];
        f32x4 KS[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KKD; ++kk) {
            const bf16x8 ak = ld8(&bs.K[16 * rb + lr][32 * kk + 8 * lg]);
            const bf16x8 aq = ld8(&bs.Q[16 * rb + lr][32 * kk + 8 * lg]);
            a1 = mfma_bf16(ak, Sh[kk], a1);
            a2 = mfma_bf16(aq, Sh[kk], a2);
            a1 = mfma_bf16(ak, Sl[kk], a1);
            a2 = mfma_bf16(aq, Sl[kk], a2);
          }
          KS[rb] = a1;
          QS[rb] = a2;
        }
        bf16x4 rh2[2], rl2[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int r0 = 16 * rb + 4 * lg;
          // V[r0 + c][16 wave + lr], c = 0..3, by a transposing read
          const bf16x4 vv = ld_tr4(&bs.V[r0 + (lr >> 2)][16 * wave + 4 * (lr & 3)]);
          const f32x4 gm4 = (GATE == kGateNone) ? f32x4{1.f, 1.f, 1.f, 1.f}
                                                : *reinterpret_cast<const f32x4 *>(&bs.gam[r0]);
          f32x4 rr;
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[e] = (float)vv[e] - gm4[e] * KS[rb][e];
          split4(rr, rh2[rb], rl2[rb]);
        }
        const bf16x8 Rh = cat(rh2[0], rh2[1]), Rl = cat(rl2[0], rl2[1]);
        const bf16(*Th)[SM::LDC] = sm.Th[s & 1];
        const bf16(*Tl)[SM::LDC] = sm.Tl[s & 1];
        bf16x4 uh[2], ul[2], wh[2], wl[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          // row 16 rb + lr of T', slots = tokens 16 h + 4 lg + c (the R rows)
          const bf16x8 th = cat(ld_tr4(&Th[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                ld_tr4(&Th[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
          const bf16x8 tl = cat(ld_tr4(&Tl[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                ld_tr4(&Tl[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
          f32x4 u = {0.f, 0.f, 0.f, 0.f};
          u = mfma_bf16(th, Rh, u);
          u = mfma_bf16(tl, Rh, u);
          u = mfma_bf16(th, Rl, u);
          split4(u, uh[rb], ul[rb]);
          const f32x4 ec4 = (GATE == kGateNone) ? f32x4{1.f, 1.f, 1.f, 1.f}
                                                : *reinterpret_cast<const f32x4 *>(&bs.ec[16 * rb + 4 * lg]);
          split4(u * ec4, wh[rb], wl[rb]);
        }
        Uh = cat(uh[0], uh[1]);
        Ul = cat(ul[0], ul[1]);
        Wh = cat(wh[0], wh[1]);
        Wl = cat(wl[0], wl[1]);
      }
      __syncthreads();
      // ---- phase Y: O = diag(gam) Q S + P U; S <- gam_last S + K^T U' ----
      if (s >= 0) {
        const typename SM::Buf &bs = sm.buf[s % NBUF];
        const int t0 = s * C, n = min(C, T - t0);
        const long orow = (tok0 + (long)t0 * H) * DV;   // element offset of the chunk's first row
        const rsrc_t ro = make_rsrc(o + orow, (long)sizeof(OutT) * ((long)B * T * H * DV - orow));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 gm4 = (GATE == kGateNone) ? f32x4{1.f, 1.f, 1.f, 1.f}
                                                : *reinterpret_cast<const f32x4 *>(&bs.gam[16 * rb + 4 * lg]);
          f32x4 acc = gm4 * QS[rb];
          const bf16x8 ph = cat(ld_tr4(&bs.Ph[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                ld_tr4(&bs.Ph[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
          const bf16x8 pl = cat(ld_tr4(&bs.Pl[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                ld_tr4(&bs.Pl[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
          acc = mfma_bf16(ph, Uh, acc);
          acc = mfma_bf16(pl, Uh, acc);
          acc = mfma_bf16(ph, Ul, acc);
          // lane holds O rows 16 rb + 4 lg + e of column col0 + lr: stored
          // straight from the accumulator (16 lanes write 16 adjacent values
          // of a row); rows past the end of the sequence are not written
          if (n == C) {
#pragma unroll
            for (int e = 0; e < 4; ++e) buf_st1(from_f32<OutT>(acc[e]), ro, ooff[rb][e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (16 * rb + 4 * lg + e < n) buf_st1(from_f32<OutT>(acc[e]), ro, ooff[rb][e]);
          }
        }
        const float glast = (GATE == kGateNone) ? 1.0f : bs.gam[C - 1];
        // k^T operand (row = dk 16 mb + lr; slots = tokens 16 h + 4 lg + c,
        // the order of the U' rows) by two transposing reads of k; dk
        // 16 mb + 4 j is stored at perm32(16 mb + 4 j) = 8 j + 32 (mb >> 1)
        // + 4 (mb & 1): a lane part plus a constant per mb
        const bf16 *kt = &bs.K[4 * lg + (lr >> 2)][8 * (lr & 3)];
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb) {
          const int dc = 32 * (mb >> 1) + 4 * (mb & 1);
          const bf16x8 a = cat(ld_tr4(kt + dc), ld_tr4(kt + 16 * SM::LDK + dc));
          f32x4 acc = Sacc[mb] * glast;
          acc = mfma_bf16(a, Wh, acc);
          acc = mfma_bf16(a, Wl, acc);
          Sacc[mb] = acc;
        }
        split_state();   // for the next chunk's phase X
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
  // prep waves: stage chunks from HBM, decay cumsum, A / P tiles, the solve
  // =======================================================================
  const int pw = wave - NSW;           // prep wave index 0..NPW-1
  const int pt = tid - 64 * NSW;       // prep thread index 0..255
  // Staging runs on prep waves 0..2 (192 threads); wave 3 solves instead.
  // q/k item = a 4-token x 8-column block of k (index < NI) or q (NI <=
  // index < 2 NI), adjacent lanes on adjacent column segments (128-byte row
  // runs); v item = one 8-column segment of one token of this slice.  Each
  // staging thread takes q/k item pt and v item pt; wave 1 also takes q/k
  // item pt + 128 and wave 2 v item pt + 64 when there are more than 192.
  constexpr int DCS = DK / 8;          // 8-column segments of a q/k row
  constexpr int NI = (C / 4) * DCS;    // items per matrix (<= 128)
  constexpr int NV = C * VCS;          // v items (<= 256)
  constexpr bool QK2 = 2 * NI > 192, V2 = NV > 192;
  static_assert(2 * NI <= 256 && NV <= 256, "staging items exceed the staging threads");
  static_assert(NI % 64 == 0, "q/k items of a wave must all come from one matrix");
  // A wave's q/k items all come from one matrix (NI is a multiple of 64), so
  // each wave reads through one buffer descriptor.  Loads are unconditional:
  // items past the end re-load the last one, rows past the end of the
  // sequence read the next rows (or zeros past the end of the tensor), and
  // only valid items and rows are written to LDS.
  struct QKItem {
    bool valid, is_k;                  // wave-uniform
    int r0, c0;
    int voff[4];                       // byte offsets of rows r0..r0+3 from the chunk's row 0
  };
  struct VItem {
    bool valid;
    int r, c0;
    int voff;
  };
  auto qk_item = [&](int wave_first, int idx) {
    QKItem m;
    m.valid = wave_first < 2 * NI;
    m.is_k = wave_first < NI;
    const int i = min(idx, 2 * NI - 1);
    const int it = m.is_k ? min(i, NI - 1) : i - NI;
    m.r0 = 4 * (it / DCS);
    m.c0 = 8 * (it % DCS);
#pragma unroll
    for (int r = 0; r < 4; ++r) m.voff[r] = 2 * ((m.r0 + r) * H * DK + m.c0);
    return m;
  };
  auto v_item = [&](int idx) {
    VItem m;
    m.valid = idx < NV;
    const int i = min(idx, NV - 1);
    m.r = i / VCS;
    m.c0 = 8 * (i % VCS);
    m.voff = 2 * (m.r * H * DV + slice * DVS + m.c0);
    return m;
  };
  const QKItem qa = qk_item(64 * pw, pt), qb = qk_item(64 * pw + 128, pt + 128);
  const VItem va = v_item(pt), vb = v_item(pt + 64);
  const long qk_total = (long)B * T * H * DK;          // elements of q (and of k, v)
  const bf16 *qa_src = qa.is_k ? k : q, *qb_src = qb.is_k ? k : q;
  bf16x8 stga[4], stgb[4], stgva, stgvb;
  float stg_b = 0.f, stg_la = 0.f;

  auto stage_chunk = [&](int j) {
    const long row0 = tok0 + (long)j * C * H;          // token row of the chunk's first token
    if (pw == 0) {   // b and log a feed wave 0's cumsum; issued first
      const int off = 4 * (lane & (C - 1)) * H;
      stg_b = buf_ld1f(make_rsrc(beta + row0, 4 * ((long)B * T * H - row0)), off);
      if constexpr (GATE == kGateScalar)
        stg_la = buf_ld1f(make_rsrc(log_alpha + row0, 4 * ((long)B * T * H - row0)), off);
    }
    const rsrc_t ra = make_rsrc(qa_src + row0 * DK, 2 * (qk_total - row0 * DK));
#pragma unroll
    for (int i = 0; i < 4; ++i) stga[i] = buf_ld8(ra, qa.voff[i]);
    stgva = buf_ld8(make_rsrc(v + row0 * DV, 2 * (qk_total - row0 * DV)), va.voff);
    if (QK2 && pw == 1) {
      const rsrc_t rb = make_rsrc(qb_src + row0 * DK, 2 * (qk_total - row0 * DK));
#pragma unroll
      for (int i = 0; i < 4; ++i) stgb[i] = buf_ld8(rb, qb.voff[i]);
    }
    if (V2 && pw == 2) stgvb = buf_ld8(make_rsrc(v + row0 * DV, 2 * (qk_total - row0 * DV)), vb.voff);
  };
  auto zero_if = [](bf16x8 x, bool z) -> bf16x8 {
    if (z) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) x[jj] = (bf16)0.0f;
    }
    return x;
  };
  auto write_qk = [&](typename SM::Buf &bf, const QKItem &m, const bf16x8 *x, int n) {
    bf16(*dst)[SM::LDK] = m.is_k ? bf.K : bf.Q;
    const int p0 = perm32(m.c0), p1 = perm32(m.c0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 y = zero_if(x[i], m.r0 + i >= n);
      *reinterpret_cast<bf16x4 *>(&dst[m.r0 + i][p0]) = lo4(y);
      *reinterpret_cast<bf16x4 *>(&dst[m.r0 + i][p1]) = hi4(y);
    }
  };
  auto write_v = [&](typename SM::Buf &bf, const VItem &m, bf16x8 x, int n) {
    *reinterpret_cast<bf16x8 *>(&bf.V[m.r][m.c0]) = zero_if(x, m.r >= n);
  };

  // lower 16x16 tiles of X K^T with the decay, two per wave: A (X = K,
  // strict lower, times b) or P (X = Q, lower incl.) of chunk j
  auto store_tile = [&](typename SM::Buf &bf, int j, f32x4 acc, int ti, int tj, bool isq) {
    const int sc = 16 * tj + lr;
    const int r0 = 16 * ti + 4 * lg;
    const float gs = bf.g[sc];
    const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(&bf.g[r0]);
    f32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dec = (GATE == kGateNone) ? 1.0f : __expf(gr4[e] - gs);
      val[e] = acc[e] * dec;
    }
    if (!isq) {
      const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&bf.beta[r0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = (sc < r0 + e) ? b4[e] * val[e] : 0.0f;
      if (ti == tj) {
        *reinterpret_cast<f32x4 *>(&sm.ATd[ti][lr][4 * lg]) = val;   // A^T of the block
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.A10[j & 1][4 * lg + e][lr] = val[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = (sc <= r0 + e) ? val[e] : 0.0f;
      bf16x4 h4, l4;
      split4(val, h4, l4);
      *reinterpret_cast<bf16x4 *>(&bf.Ph[sc][r0]) = h4;
      *reinterpret_cast<bf16x4 *>(&bf.Pl[sc][r0]) = l4;
    }
  };
  auto two_tiles = [&](typename SM::Buf &bf, int j, bool q1, int ti1, int tj1, bool q2, int ti2,
                       int tj2) {
    const bf16(*X1)[SM::LDK] = q1 ? bf.Q : bf.K;
    const bf16(*X2)[SM::LDK] = q2 ? bf.Q : bf.K;
    f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KKD; ++kk) {
      const int c = 32 * kk + 8 * lg;
      acc1 = mfma_bf16(ld8(&X1[16 * ti1 + lr][c]), ld8(&bf.K[16 * tj1 + lr][c]), acc1);
      acc2 = mfma_bf16(ld8(&X2[16 * ti2 + lr][c]), ld8(&bf.K[16 * tj2 + lr][c]), acc2);
    }
    store_tile(bf, j, acc1, ti1, tj1, q1);
    store_tile(bf, j, acc2, ti2, tj2, q2);
  };

  if (pw == 3) {
    // ---- solver wave: its own loop, so the staging registers of waves
    //      0..2 are not live across the solve ----
    __syncthreads();
    float x[16];                       // column lane & 15 of block (lane >> 4) & 1 of T
    for (int it = 0; it < nchunks + 2; ++it) {
      // phase X: diagonal 16x16 blocks of T = (I + A)^{-1} of chunk it-1;
      // lane = (block, column); right-looking forward substitution: once
      // x_s is final it updates all later rows, so the dependent chain is
      // one FMA per step
      if (it >= 1 && it - 1 < nchunks) {
        const int j = it - 1;
        const int blk = (lane >> 4) & 1, col = lane & 15, o0 = 16 * blk;
        const float(*At)[20] = sm.ATd[blk];   // At[s][r] = A[o0 + r][o0 + s]
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.0f : 0.0f;
        // every needed entry of A^T (rows s, columns r > s: 36 float4) is
        // loaded up front, so the 15 dependent steps wait on no LDS read
        f32x4 a4[15][4];
#pragma unroll
        for (int s2 = 0; s2 < 15; ++s2)
#pragma unroll
          for (int q4 = (s2 + 1) / 4; q4 < 4; ++q4)
            a4[s2][q4] = *reinterpret_cast<const f32x4 *>(&At[s2][4 * q4]);
        // keep the loads ahead of the dependent steps (the scheduler would
        // otherwise sink them next to their uses to save registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s2 = 0; s2 < 15; ++s2) {
#pragma unroll
          for (int r = s2 + 1; r < 16; ++r) x[r] -= a4[s2][r / 4][r % 4] * x[s2];
        }
        if (lane < 32) {   // lanes 32..63 hold duplicates; fp32 T^T rows only
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4 *>(&sm.TdT[blk][col][4 * q4]) =
                f32x4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
        }
      }
      __syncthreads();
      // phase Y: the off-diagonal A and P tiles of chunk it, then the bf16
      // hi/lo diagonal blocks of T' of chunk it-1 from this phase X's solve
      if (it < nchunks) two_tiles(sm.buf[it % NBUF], it, false, 1, 0, true, 1, 0);
      if (it >= 1 && it - 1 < nchunks) {
        const int j = it - 1;
        const float *bj = sm.buf[j % NBUF].beta;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        if (lane < 32) {
          // T'[o0 + r][o0 + col] = T[o0 + r][o0 + col] b_{o0 + col}, r = 0..15,
          // is row o0 + col of T'^T
          // (x still holds this lane's column of T from phase X)
          const int blk = lane >> 4, col = lane & 15, o0 = 16 * blk;
          const float bcol = bj[o0 + col];
          unsigned h8[2][4], l8[2][4];
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            split2(x[r] * bcol, x[r + 1] * bcol, h8[r / 8][(r % 8) / 2], l8[r / 8][(r % 8) / 2]);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            *reinterpret_cast<u32x4 *>(&sm.Th[j & 1][o0 + col][o0 + 8 * hf]) =
                u32x4{h8[hf][0], h8[hf][1], h8[hf][2], h8[hf][3]};
            *reinterpret_cast<u32x4 *>(&sm.Tl[j & 1][o0 + col][o0 + 8 * hf]) =
                u32x4{l8[hf][0], l8[hf][1], l8[hf][2], l8[hf][3]};
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  // ---- staging waves 0..2 ----
  if (nchunks > 0) stage_chunk(0);
  __syncthreads();

  for (int it = 0; it < nchunks + 2; ++it) {
    // phase X: write chunk it (+ decay cumsum on wave 0), stage chunk it+1.
    // Every load in flight is one of chunk it's, consumed right here: one
    // wait for all of them, on every path, so no later register reuse waits
    // on a load that some skipped branch might have left pending.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (it < nchunks) {
      typename SM::Buf &bf = sm.buf[it % NBUF];
      const int n = min(C, T - it * C);
      if (qa.valid) write_qk(bf, qa, stga, n);
      if (QK2 && pw == 1 && qb.valid) write_qk(bf, qb, stgb, n);
      if (va.valid) write_v(bf, va, stgva, n);
      if (V2 && pw == 2 && vb.valid) write_v(bf, vb, stgvb, n);
      if (pw == 0) {
        // in-chunk cumulative log decay: inclusive scan over lanes 0..C-1;
        // padded tokens carry log a = 0 and b = 0
        const float la = scan32_inclusive((lane < n) ? stg_la : 0.0f);
        const float glast = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, la), C - 1));
        if (lane < C) {
          bf.g[lane] = la;
          bf.gam[lane] = __expf(la);
          bf.ec[lane] = __expf(glast - la);
          bf.beta[lane] = (lane < n) ? stg_b : 0.0f;
        }
      }
      if (it + 1 < nchunks) stage_chunk(it + 1);
    }
    __syncthreads();

    // phase Y: the diagonal A (wave 1) and P (wave 2) tiles of chunk it;
    // the off-diagonal block of T' of chunk it-1 (wave 0)
    if (pw >= 1 && it < nchunks) {
      if (pw == 1) two_tiles(sm.buf[it % NBUF], it, false, 0, 0, false, 1, 1);
      else two_tiles(sm.buf[it % NBUF], it, true, 0, 0, true, 1, 1);
    }
    if (pw == 0 && it >= 1 && it - 1 < nchunks) {
      // T10 = -T11 (A10 T00) of chunk it-1 (its diagonal blocks were solved
      // in this iteration's phase X)
      const int j = it - 1;
      const float *bj = sm.buf[j % NBUF].beta;
      f32x4 xa = mm16_split(&sm.A10[j & 1][0][0], 20, &sm.TdT[0][0][0], 20,
                            f32x4{0.f, 0.f, 0.f, 0.f}, lane);
      *reinterpret_cast<f32x4 *>(&sm.X[lr][4 * lg]) = xa;   // X^T
      f32x4 z = mm16_split_lt(&sm.TdT[1][0][0], 20, &sm.X[0][0], 20, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
      const float bc = bj[lr];
      bf16x4 h4, l4;
      split4(-z * bc, h4, l4);
      *reinterpret_cast<bf16x4 *>(&sm.Th[j & 1][lr][16 + 4 * lg]) = h4;
      *reinterpret_cast<bf16x4 *>(&sm.Tl[j & 1][lr][16 + 4 * lg]) = l4;
    }
    __syncthreads();
  }
}

template <int DK, int DVS, typename OutT, int GATE>
hipError_t launch_cfg(const ChunkArgs &a) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + NPW));
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVS, OutT, GATE>), grid, block, 0, a.stream,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta, a.log_alpha,
                     a.initial_state, (OutT *)a.o, a.final_state, a.B, a.T, a.H);
  return hipGetLastError();
}

template <int DK, int DVS, typename OutT>
hipError_t by_gate(const ChunkArgs &a) {
  if (a.gate == kGateNone) return launch_cfg<DK, DVS, OutT, kGateNone>(a);
  return launch_cfg<DK, DVS, OutT, kGateScalar>(a);
}

template <int DK, int DVS>
hipError_t by_out(const ChunkArgs &a) {
  return a.out_bf16 ? by_gate<DK, DVS, bf16>(a) : by_gate<DK, DVS, float>(a);
}

}  // namespace

bool chunk_fwd_bf16_supported(const ChunkArgs &a) {
  // the kernel's chunk is 32 tokens; a requested chunk size only changes
  // rounding, so 0, 16, 32 and 64 all map here
  return a.in_bf16 && (a.D == 128 || a.D == 64) && a.gate != kGateChannel;
}

hipError_t launch_chunk_fwd_bf16(const ChunkArgs &a) {
  // 64 value columns per workgroup once there are >= 256 (chain, slice)
  // pairs to fill the chip; fewer chains use 32-column slices
  const long chains = (long)a.B * a.H;
  if (a.D == 128) {
    if (chains * 2 >= 256) return by_out<128, 64>(a);
    return by_out<128, 32>(a);
  }
  if (chains >= 256) return by_out<64, 64>(a);
  return by_out<64, 32>(a);
}

}  // namespace gdr
