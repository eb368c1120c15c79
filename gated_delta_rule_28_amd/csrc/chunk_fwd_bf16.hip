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
// Without the erase term (S_t = a_t S_{t-1} + b_t k_t v_t^T: linear attention
// and the Mamba-2 / SSD decay, page "NLP——线性注意力相关总结", section "Linear
// Attention"; xhh.club digest, abstract) A = 0, so U = diag(b) V: the same
// kernel skips K S, the A tiles and the solve (template flag ERASE).
//
// Mapping.  One workgroup per (batch, head, Dv-slice of DVS columns): the Dv
// columns of S, U and O are independent given K, b and g.  Chunks are C = 32
// tokens.  Roles:
//
//   state waves (DVS/16 of them) each own 16 state columns and keep them in
//     MFMA accumulators for the whole sequence.  Every state-dependent
//     product (K S, T'R, K^T U') takes its right operand straight from
//     accumulator registers: an accumulator tile holds rows 4g..4g+3 of a
//     column, which is what a 16x16x32 B operand needs when the k axis of S
//     is ordered so that tile pair (2kk, 2kk+1) holds dk 32kk + 8g + j
//     (j < 4) and 32kk + 8g + 4 + j in its rows 4g + j.  q and k then stay
//     in natural dk order in LDS.  The output tile is formed transposed
//     (S^T Q^T and U^T P^T, the same registers as left operands), so that a
//     lane ends up with four adjacent values of one output row: one 16-byte
//     store per lane and row block.
//   prep waves 0..2 bring chunks into LDS with LDS DMA (no registers, no
//     LDS write instructions), scan the log decays and form the decayed
//     K K^T / Q K^T tiles (A and P); prep wave 3 solves the diagonal 16x16
//     blocks of T = (I + A)^{-1} and forms its off-diagonal block.  T is
//     kept without the diag(b) factor: the state waves scale R by b instead,
//     T' R = T (b o R), which takes two passes over T off the solver.
//
// Schedule.  One workgroup barrier per iteration; in iteration i
//   prep waves 0..2: DMA of chunk i+3 issued; decay scan, A tiles and P
//                    tiles of chunk i+1; wait for their DMA of chunk i+2
//   prep wave 3:     T of chunk i (diagonal solve, then the off-diagonal
//                    block)
//   state waves:     K S, Q S, U, O and the S update of chunk i-1
// Every product of iteration i reads only what earlier iterations wrote, so
// the state waves run their whole chunk without a barrier in between.  A
// DMA is waited for a full iteration after it was issued, which hides HBM
// latency; a chunk's input slot lives five iterations (NIN = 5), its P tiles
// three and its T two.
//
// LDS layouts.  q, k rows are 2 DK bytes and v rows 2 DVS bytes with no
// padding; the 16-byte blocks of each row are XOR-permuted by a function of
// the row (swz_qk, swz_v) so that the row reads (16 rows, one block) and
// the transposing reads (8 rows, 4 blocks) of the products hit distinct
// banks.  The DMA lanes fetch the block that belongs at their fixed LDS
// position.
//
// Backward passes (template MODE).  The same pipeline runs the two sequential
// passes of the backward: kModeRec recomputes the forward and stores, per
// chunk, the entering state h and U (no outputs);
// kModeRev walks the chunks in reverse with v = dO, carrying dS, the
// gradient of the state (dS_T in, dS_0 out):
//
//   dU  = diag(e^{g_last - g}) K dS + P^T dO        dY = T^T dU
//   dS <- gam_last dS + Q^T diag(gam) dO - K^T diag(gam b) dY
//
// storing dS (the gradient of the state leaving the chunk) and dY per chunk.
// Both take the prep waves' A, P and T tiles unchanged (T^T and P^T are the
// tiles as stored); the chunk-parallel kernel (chunk_bwd.hip) forms the
// token gradients from what they store.  kModeFwdSave, the training forward,
// is the forward with kModeRec's stores (the state kept unscaled), so that
// the backward can skip its recompute pass.
//
// Precision.  q, k, v are exact bf16 and enter MFMAs unsplit; every derived
// operand (S, R, U, T, P) is split into bf16
// hi + lo and multiplied as hi*hi + hi*lo + lo*hi (two products when the
// other side is exact), so products carry ~16 significant bits and
// accumulate in fp32.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace gdr {
namespace {

constexpr int C = 32;      // tokens per chunk
constexpr int NPW = 4;     // prep waves
constexpr int NIN = 5;     // input slots: chunk j DMA'd from iteration j-3, last read in j+1
constexpr int NPR = 3;     // P slots: chunk j written in iteration j-1, read in j+1
constexpr int NTS = 2;     // T slots: chunk j written in iteration j, read in j+1


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
  static constexpr int LDC = C + 16;   // bf16 stride of [*][C] rows (transposing reads of
                                       // 8 rows hit 64 distinct banks)
  static constexpr int LDT = 24;       // bf16 stride of the 16x16 hi/lo blocks
  struct __align__(16) In {            // one chunk's inputs (LDS DMA) and decay terms
    bf16 Q[C][DK];                     // q rows, blocks permuted by swz_qk
    bf16 K[C][DK];                     // k rows, likewise
    bf16 V[C][DVS];                    // v rows of this slice, blocks permuted by swz_v
    float la[64], beta[64];            // log a and b of the 64 tokens from the chunk start
                                       // (0 past the end of the sequence: the DMA
                                       // reads zeros beyond the chunk's last row)
    float gam[C], ec[C];               // e^g, e^{g_last - g} (times 1/|k| when fused)
    float fq[C], fk[C], bt[C];         // factors of Q S and K S (e^g, times 1/|q|, 1/|k|
                                       // when fused), b (after the fused sigmoid)
    float nrm[2][C];                   // fused L2 normalisation: 1/|q|, 1/|k| per token
    float zsc[4];                      // carried-scale form: [0] the state's factor before
                                       // the update, [1] the scale after it
  };
  struct __align__(16) PT {
    bf16 Ph[C][LDC], Pl[C][LDC];       // P^T: [s][r] = P[r][s]; rows 16..31 x cols 0..15 stay zero
  };
  In in[NIN];
  PT p[NPR];
  float ATd[2][2][16][20];             // per chunk parity, diagonal 16x16 blocks of -A,
                                       // transposed: [.][b][s][r] = -A[16b+r][16b+s]
  bf16 A10h[2][16][LDT], A10l[2][16][LDT];   // block (1,0) of A, transposed: [s][r] = A[16+r][s]
  bf16 Th[NTS][C][LDC], Tl[NTS][C][LDC];   // T^T: [s][r] = T[r][s], T = (I+A)^{-1} (T' = T diag(b));
                                       // rows 16..31 x cols 0..15 stay zero
  float gw[3][C], bw[3][C];            // in-chunk log decay g and b, one copy per tile wave
};

template <int DK, int DVS, typename OutT, int GATE, bool ERASE, bool FUSED, int MODE>
__global__ void __launch_bounds__(64 * (DVS / 16 + NPW), 1)
chunk_fwd_bf16_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                      const bf16 *__restrict__ v, const float *__restrict__ beta,
                      const float *__restrict__ log_alpha, const float *initial_state,
                      OutT *__restrict__ o, float *final_state, int B, int T, int H, int fuse,
                      const bf16 *__restrict__ out_gate, float *__restrict__ ws_a,
                      float *__restrict__ ws_b, float *__restrict__ ws_c) {
  constexpr int NSW = DVS / 16;        // state waves; wave w owns value columns 16w..16w+15
  constexpr int NT = 64 * (NSW + NPW);
  constexpr int DV = DK;               // full value width (Dk == Dv)
  constexpr int NSLICE = DV / DVS;
  constexpr int KKD = DK / 32;         // 32-deep k steps over dk
  constexpr int QB = DK / 8, VB = DVS / 8;      // 16-byte blocks per q/k and v row
  constexpr int QRB = 2 * DK, VRB = 2 * DVS;    // bytes per q/k and v row
  static_assert((DK == 64 || DK == 128) && (DVS == 32 || DVS == 64) && DVS <= DK, "tile config");
  using SM = PipeSmem<DK, DVS>;
  using In = typename SM::In;
  static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
  static_assert(sizeof(In) % 16 == 0 && (C * QRB) % 1024 == 0 && (C * VRB) % 1024 == 0,
                "DMA runs are whole 1 KiB waves");
  static_assert(MODE == kModeFwd || (!FUSED && GATE != kGateChannel),
                "the backward passes run the unfused forms without the per-channel gate");
  constexpr bool WANT_O = MODE == kModeFwd || MODE == kModeFwdSave;   // outputs (Q S, P U, o)
  constexpr bool SAVE = MODE == kModeRec || MODE == kModeFwdSave;     // h and U per chunk
  // Carried-scale form of the state (forward, scalar decay): the state
  // waves hold Z with S = Z_scale * Z, so that the decay of a chunk does not
  // multiply every state element: the scale goes into the row factors of
  // K S and Q S (times Z_scale) and of the update (divided by the scale
  // after it), and Z is multiplied only when the scale would drop below
  // 2^-40 (then by the accumulated scale, which returns to 1).  The scale
  // is kept by the prep wave that forms the factors, chunk by chunk.  (The
  // modes that store the state keep it unscaled.)
  constexpr bool LAZY = MODE == kModeFwd && GATE == kGateScalar;
  constexpr bool WANT_P = MODE != kModeRec;      // the P tiles and q
  __shared__ SM sm;
  // calls without a fused prologue or epilogue compile without their code
  if constexpr (!FUSED) {
    fuse = 0;
    out_gate = nullptr;
  }

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
  // the chunk of pipeline step j (the reverse pass walks the chunks backwards)
  auto chunk_of = [&](int j) { return MODE == kModeRev ? nchunks - 1 - j : j; };

  // byte offset inside a q/k (v) tile of row r, natural 16-byte block b
  auto qk_at = [](int r, int b) { return r * QRB + 16 * (b ^ swz_qk<QB>(r)); };
  auto v_at = [](int r, int b) { return r * VRB + 16 * (b ^ swz_v<VB>(r)); };
  // row reads of q/k: lane (lr, lg) takes row 16 t + lr, dk 32 kk + 8 lg .. +7;
  // the permutation depends on r & 15 = lr only, so tile t adds 16 t rows
  int kq_off[KKD];
#pragma unroll
  for (int kk = 0; kk < KKD; ++kk) kq_off[kk] = qk_at(lr, 4 * kk + lg);

  // the upper-right 16x16 blocks of P and T' are never written: zero once
  for (int i = tid; i < C * SM::LDC; i += NT) {
#pragma unroll
    for (int b = 0; b < NPR; ++b) {
      (&sm.p[b].Ph[0][0])[i] = (bf16)0.0f;
      (&sm.p[b].Pl[0][0])[i] = (bf16)0.0f;
    }
#pragma unroll
    for (int b = 0; b < NTS; ++b) {
      (&sm.Th[b][0][0])[i] = (bf16)0.0f;
      (&sm.Tl[b][0][0])[i] = (bf16)0.0f;
    }
  }

  // Every role runs two prologue barriers and nchunks + 1 iterations of one
  // barrier, so all waves execute the same sequence of workgroup barriers.
  if (wave < NSW) {
    // =====================================================================
    // state waves: the serial chunk-to-chunk pass, 16 state columns each
    // =====================================================================
    const int col0 = slice * DVS + 16 * wave;   // first value column of this wave
    const bool gated = out_gate != nullptr;
    // Sacc[mb][e] = S[srow(mb, e)][col0 + lr]
    auto srow = [&](int mb, int e) { return 32 * (mb >> 1) + 8 * lg + 4 * (mb & 1) + e; };
    f32x4 Sacc[DK / 16];
#pragma unroll
    for (int mb = 0; mb < DK / 16; ++mb) Sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (initial_state) {
      const float *S0 = initial_state + (long)chain * DK * DV;
#pragma unroll
      for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[mb][e] = S0[(long)srow(mb, e) * DV + col0 + lr];
    }
    __syncthreads();
    __syncthreads();

    // The output tile is formed transposed (Q S and P U as S^T Q^T and
    // U^T P^T: the same operand registers, swapped), so lane (lr, lg) holds
    // O[16 rb + lr][col0 + 4 lg + e], e = 0..3: four adjacent values of one
    // row, written by one 16-byte store.  Element offsets of those values
    // from a chunk's first row, and the byte offset of the first in o;
    // unsigned 32-bit, like the buffer offset they feed (the host bounds one
    // chunk's rows of a 4-byte tensor below 4 GiB, so neither wraps)
    unsigned oel[2][4], ooff[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        oel[rb][e] = (unsigned)(16 * rb + lr) * (unsigned)(H * DV) + (unsigned)(col0 + 4 * lg + e);
      ooff[rb] = (unsigned)sizeof(OutT) * oel[rb][0];
    }
    // v, transposing read: rows 16 rb + 4 lg + (lr >> 2), columns
    // 16 wave + 4 (lr & 3) .. +3 (an 8-byte half of a 16-byte block)
    const int v_off = v_at(4 * lg + (lr >> 2), 2 * wave + ((lr & 3) >> 1)) + 8 * (lr & 1);
    // k^T operand of the state update for tile mb: rows (tokens) 4 lg + (lr >> 2)
    // (+16), dk srow(mb, 0) + 4 (lr & 3) .. +3 = natural block (lr & 3) +
    // 4 (mb >> 1), half mb & 1
    int kt_off[KKD];
#pragma unroll
    for (int kk = 0; kk < KKD; ++kk) kt_off[kk] = qk_at(4 * lg + (lr >> 2), (lr & 3) + 4 * kk);

    // hi/lo bf16 split of the state, the right operand of K S and Q S; it
    // is formed right after the previous chunk's update
    bf16x8 Sh[KKD], Sl[KKD];
    auto split_state = [&]() {
#pragma unroll
      for (int kk = 0; kk < KKD; ++kk) split8_keep(Sacc[2 * kk], Sacc[2 * kk + 1], Sh[kk], Sl[kk]);
    };

    // the fused output gate of this lane's O values, loaded one chunk ahead
    // (the state waves are the serial path: a load used in the same chunk
    // would expose its latency every chunk) and turned into the factor
    // g sigmoid(g) (1 without a gate) before the O products, which are then
    // only multiplied: a branch between an MFMA and the read of its result
    // can hide the wait states that read needs
    // The loads are unconditional: without a gate, or past the last chunk,
    // the descriptor is empty and they read zeros without touching memory.
    f32x4 og[2] = {};
    u32x2 og_next[2] = {};               // four bf16 gate values per row block
    auto load_gate = [&](int c) {
      const bool valid = gated && c < nchunks;
      const int n = valid ? min(C, T - c * C) : 1;
      const long orow = valid ? (tok0 + (long)c * C * H) * DV : 0;
      const rsrc_t rg = make_rsrc32(out_gate + orow,
                                    valid ? 2u * ((unsigned)(n - 1) * H * DV + DV) : 0u);
      // the lane's four adjacent values of a row: one 8-byte load
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) og_next[rb] = buf_ld_b64(rg, 2u * oel[rb][0]);
    };

    for (int it = 0; it < nchunks + 1; ++it) {
      const int s = it - 1;            // chunk of this iteration
     if constexpr (MODE == kModeRev) {
      if (s >= 0) {
        // the hi/lo split of dS for this chunk's products: after the barrier,
        // in the same block as the products, so the scheduler can overlap the
        // split with their issue
        split_state();
        const int c = nchunks - 1 - s;   // chunks run last to first
        const In &bs = *at_off(&sm.in[0], slot_off(s % NIN, (int)sizeof(In)));
        const typename SM::PT &ps = *at_off(&sm.p[0], slot_off(s % NPR, (int)sizeof(typename SM::PT)));
        const int tso = slot_off(s % NTS, (int)sizeof(sm.Th[0]));
        const bf16(*Th)[SM::LDC] = at_off(&sm.Th[0][0], tso);
        const bf16(*Tl)[SM::LDC] = at_off(&sm.Tl[0][0], tso);
        const char *Kb = reinterpret_cast<const char *>(&bs.K[0][0]);
        const char *Qb = reinterpret_cast<const char *>(&bs.Q[0][0]);
        const char *Vb = reinterpret_cast<const char *>(&bs.V[0][0]);
        // dS, the gradient of the state leaving chunk c
        float *dh = ws_a + ((long)chain * nchunks + c) * (DK * DV);
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_nontemporal_store(Sacc[mb][e], dh + ws_frag(DK / 16, col0 >> 4, mb, e, lg, lr));
        // K dS
        f32x4 KS[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4 a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KKD; ++kk) {
            const bf16x8 ak = ld8(reinterpret_cast<const bf16 *>(Kb + 16 * rb * QRB + kq_off[kk]));
            a1 = mfma_bf16(ak, Sh[kk], a1);
            a1 = mfma_bf16(ak, Sl[kk], a1);
          }
          KS[rb] = a1;
        }
        // dO of this lane's column, rows 16 rb + 4 lg + c (transposing reads
        // of the v slot, which holds dO in this mode): the B operand of P^T dO
        bf16x4 dov[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          dov[rb] = ld_tr4(reinterpret_cast<const bf16 *>(Vb + 16 * rb * VRB + v_off));
        const bf16x8 Dd = cat(dov[0], dov[1]);
        // dU = diag(e^{g_last - g}) K dS + P^T dO; row r of P^T is row r of
        // the stored P^T tile, k = tokens {4 lg + j} u {16 + 4 lg + j}
        bf16x4 duh[2], dul[2];
        f32x4 du[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 ec4 = *reinterpret_cast<const f32x4 *>(&bs.ec[16 * rb + 4 * lg]);
          f32x4 acc = ec4 * KS[rb];
          const bf16x8 ph = cat(*reinterpret_cast<const bf16x4 *>(&ps.Ph[16 * rb + lr][4 * lg]),
                                *reinterpret_cast<const bf16x4 *>(&ps.Ph[16 * rb + lr][16 + 4 * lg]));
          const bf16x8 pl = cat(*reinterpret_cast<const bf16x4 *>(&ps.Pl[16 * rb + lr][4 * lg]),
                                *reinterpret_cast<const bf16x4 *>(&ps.Pl[16 * rb + lr][16 + 4 * lg]));
          acc = mfma_bf16(ph, Dd, acc);
          acc = mfma_bf16(pl, Dd, acc);
          du[rb] = acc;
          split4(acc, duh[rb], dul[rb]);
        }
        const bf16x8 DUh = cat(duh[0], duh[1]), DUl = cat(dul[0], dul[1]);
        // dY = T^T dU (stored), and the update's right operands gam dO and
        // -gam b dY
        float *dyb = ws_b + ((long)chain * nchunks + c) * (C * DV);
        bf16x4 bqh[2], bql[2], bkh[2], bkl[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          // without the erase term T = I: dY = dU
          f32x4 y = du[rb];
          if constexpr (ERASE) {
            const bf16x8 th = cat(*reinterpret_cast<const bf16x4 *>(&Th[16 * rb + lr][4 * lg]),
                                  *reinterpret_cast<const bf16x4 *>(&Th[16 * rb + lr][16 + 4 * lg]));
            const bf16x8 tl = cat(*reinterpret_cast<const bf16x4 *>(&Tl[16 * rb + lr][4 * lg]),
                                  *reinterpret_cast<const bf16x4 *>(&Tl[16 * rb + lr][16 + 4 * lg]));
            y = f32x4{0.f, 0.f, 0.f, 0.f};
            y = mfma_bf16(th, DUh, y);
            y = mfma_bf16(tl, DUh, y);
            y = mfma_bf16(th, DUl, y);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_nontemporal_store(y[e], dyb + ws_frag(C / 16, col0 >> 4, rb, e, lg, lr));
          const f32x4 gm4 = *reinterpret_cast<const f32x4 *>(&bs.gam[16 * rb + 4 * lg]);
          const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&bs.bt[16 * rb + 4 * lg]);
          f32x4 gd;
#pragma unroll
          for (int e = 0; e < 4; ++e) gd[e] = gm4[e] * (float)dov[rb][e];
          split4(gd, bqh[rb], bql[rb]);
          if constexpr (ERASE) split4(-(gm4 * b4) * y, bkh[rb], bkl[rb]);
        }
        const bf16x8 Bqh = cat(bqh[0], bqh[1]), Bql = cat(bql[0], bql[1]);
        bf16x8 Bkh = {}, Bkl = {};
        if constexpr (ERASE) {
          Bkh = cat(bkh[0], bkh[1]);
          Bkl = cat(bkl[0], bkl[1]);
        }
        const float glast = (GATE == kGateNone) ? 1.0f : bs.gam[C - 1];
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb) {
          const int off = kt_off[mb >> 1] + 8 * (mb & 1);
          const bf16x8 ak = cat(ld_tr4(reinterpret_cast<const bf16 *>(Kb + off)),
                                ld_tr4(reinterpret_cast<const bf16 *>(Kb + off + 16 * QRB)));
          const bf16x8 aq = cat(ld_tr4(reinterpret_cast<const bf16 *>(Qb + off)),
                                ld_tr4(reinterpret_cast<const bf16 *>(Qb + off + 16 * QRB)));
          f32x4 acc = Sacc[mb] * glast;
          if constexpr (ERASE) {   // dS = gam_last dS' + Q^T diag(gam) dO - K^T diag(gam b) dY
            acc = mfma_bf16(ak, Bkh, acc);
            acc = mfma_bf16(ak, Bkl, acc);
          }
          acc = mfma_bf16(aq, Bqh, acc);
          acc = mfma_bf16(aq, Bql, acc);
          Sacc[mb] = acc;
        }
      }
     } else {
      f32x4 QS[2];
      bf16x8 Uh, Ul, Wh, Wl;
      if constexpr (FUSED) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            og[rb][e] = gated ? silu_gate(1.0f, bf16_bits_to_f32(
                                    e & 1 ? og_next[rb][e >> 1] >> 16 : og_next[rb][e >> 1] & 0xffffu))
                              : 1.0f;
        load_gate(it);
      }
      // ---- K S, Q S, R = V - diag(gam) K S, U = T' R ----
      if (s >= 0) {
        const In &bs = *at_off(&sm.in[0], slot_off(s % NIN, (int)sizeof(In)));
        const char *Kb = reinterpret_cast<const char *>(&bs.K[0][0]);
        const char *Qb = reinterpret_cast<const char *>(&bs.Q[0][0]);
        const char *Vb = reinterpret_cast<const char *>(&bs.V[0][0]);
        if constexpr (SAVE) {
          // the state entering chunk s
          float *hb = ws_a + ((long)chain * nchunks + s) * (DK * DV);
#pragma unroll
          for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              __builtin_nontemporal_store(Sacc[mb][e], hb + ws_frag(DK / 16, col0 >> 4, mb, e, lg, lr));
        }
        // the hi/lo split of S for this chunk's products: after the barrier,
        // in the same block as K S and Q S, so the scheduler can overlap the
        // split with their issue
        split_state();
        f32x4 KS[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KKD; ++kk) {
            if constexpr (ERASE && !WANT_O) {
              const bf16x8 ak = ld8(reinterpret_cast<const bf16 *>(Kb + 16 * rb * QRB + kq_off[kk]));
              a1 = mfma_bf16(ak, Sh[kk], a1);
              a1 = mfma_bf16(ak, Sl[kk], a1);
            } else if constexpr (ERASE) {
              const bf16x8 aq = ld8(reinterpret_cast<const bf16 *>(Qb + 16 * rb * QRB + kq_off[kk]));
              const bf16x8 ak = ld8(reinterpret_cast<const bf16 *>(Kb + 16 * rb * QRB + kq_off[kk]));
              // K S, and Q S transposed (S^T Q^T: operands swapped)
              a1 = mfma_bf16(ak, Sh[kk], a1);
              a2 = mfma_bf16(Sh[kk], aq, a2);
              a1 = mfma_bf16(ak, Sl[kk], a1);
              a2 = mfma_bf16(Sl[kk], aq, a2);
            } else if constexpr (WANT_O) {
              // no erase term: Q S only (and nothing in the recompute pass)
              const bf16x8 aq = ld8(reinterpret_cast<const bf16 *>(Qb + 16 * rb * QRB + kq_off[kk]));
              a2 = mfma_bf16(Sh[kk], aq, a2);
              a2 = mfma_bf16(Sl[kk], aq, a2);
            }
          }
          KS[rb] = a1;
          QS[rb] = a2;
        }
        bf16x4 rh2[2], rl2[2];
        f32x4 rv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int r0 = 16 * rb + 4 * lg;
          // V[r0 + c][16 wave + lr], c = 0..3, by a transposing read
          const bf16x4 vv = ld_tr4(reinterpret_cast<const bf16 *>(Vb + 16 * rb * VRB + v_off));
          const f32x4 gm4 = *reinterpret_cast<const f32x4 *>(&bs.fk[r0]);
          const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&bs.bt[r0]);
          // b o R: T' R = T diag(b) R with T kept unscaled; without the
          // erase term R = V and U = b o V
          f32x4 rr;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rr[e] = (ERASE ? (float)vv[e] - gm4[e] * KS[rb][e] : (float)vv[e]) * b4[e];
          rv[rb] = rr;
          split4(rr, rh2[rb], rl2[rb]);
        }
        const bf16x8 Rh = cat(rh2[0], rh2[1]), Rl = cat(rl2[0], rl2[1]);
        bf16x4 uh[2], ul[2], wh[2], wl[2];
        if constexpr (!ERASE) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            uh[rb] = rh2[rb];
            ul[rb] = rl2[rb];
            if constexpr (SAVE) {   // U = b o V
              float *ubp = ws_b + ((long)chain * nchunks + s) * (C * DV);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                __builtin_nontemporal_store(rv[rb][e], ubp + ws_frag(C / 16, col0 >> 4, rb, e, lg, lr));
            }
            const f32x4 ec4 = *reinterpret_cast<const f32x4 *>(&bs.ec[16 * rb + 4 * lg]);
            split4(rv[rb] * ec4, wh[rb], wl[rb]);
          }
        } else {
          const int tso = slot_off(s % NTS, (int)sizeof(sm.Th[0]));
          const bf16(*Th)[SM::LDC] = at_off(&sm.Th[0][0], tso);
          const bf16(*Tl)[SM::LDC] = at_off(&sm.Tl[0][0], tso);
  #pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            // row 16 rb + lr of T, slots = tokens 16 h + 4 lg + c (the R rows)
            const bf16x8 th = cat(ld_tr4(&Th[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                  ld_tr4(&Th[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
            const bf16x8 tl = cat(ld_tr4(&Tl[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                  ld_tr4(&Tl[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            u = mfma_bf16(th, Rh, u);
            u = mfma_bf16(tl, Rh, u);
            u = mfma_bf16(th, Rl, u);
            if constexpr (SAVE) {
              float *ubp = ws_b + ((long)chain * nchunks + s) * (C * DV);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                __builtin_nontemporal_store(u[e], ubp + ws_frag(C / 16, col0 >> 4, rb, e, lg, lr));
            }
            split4(u, uh[rb], ul[rb]);
            const f32x4 ec4 = *reinterpret_cast<const f32x4 *>(&bs.ec[16 * rb + 4 * lg]);
            split4(u * ec4, wh[rb], wl[rb]);
          }
        }
        Uh = cat(uh[0], uh[1]);
        Ul = cat(ul[0], ul[1]);
        Wh = cat(wh[0], wh[1]);
        Wl = cat(wl[0], wl[1]);
      }
      // ---- O = diag(gam) Q S + P U; S <- gam_last S + K^T U' ----
      if (s >= 0) {
        const In &bs = *at_off(&sm.in[0], slot_off(s % NIN, (int)sizeof(In)));
        const typename SM::PT &ps = *at_off(&sm.p[0], slot_off(s % NPR, (int)sizeof(typename SM::PT)));
        const int t0 = s * C, n = min(C, T - t0);
        const long orow = (tok0 + (long)t0 * H) * DV;   // element offset of the chunk's first row
        // the chunk's rows: smaller than 4 GiB (the host checks the shape)
        const rsrc_t ro = make_rsrc32(o + orow, (unsigned)sizeof(OutT) * ((unsigned)(n - 1) * H * DV + DV));
        f32x4 oacc[2];
#pragma unroll
        for (int rb = 0; rb < 2 && WANT_O; ++rb) {
          // O^T = diag(gam) (Q S)^T + U^T P^T: this lane's values are all of
          // token 16 rb + lr
          f32x4 acc = bs.fq[16 * rb + lr] * QS[rb];
          // row 16 rb + lr of P (k = tokens {4 lg + j} u {16 + 4 lg + j}),
          // the B operand of U^T P^T
          const bf16x8 ph = cat(ld_tr4(&ps.Ph[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                ld_tr4(&ps.Ph[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
          const bf16x8 pl = cat(ld_tr4(&ps.Pl[4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]),
                                ld_tr4(&ps.Pl[16 + 4 * lg + (lr >> 2)][16 * rb + 4 * (lr & 3)]));
          acc = mfma_bf16(Uh, ph, acc);
          acc = mfma_bf16(Uh, pl, acc);
          acc = mfma_bf16(Ul, ph, acc);
          oacc[rb] = acc;
        }
        const char *Kb = reinterpret_cast<const char *>(&bs.K[0][0]);
        float glast = (GATE == kGateNone) ? 1.0f : bs.gam[C - 1];
        if constexpr (LAZY) {
          // the state's factor before this update: 1 unless the scale is
          // folded back in (a wave-uniform value and branch)
          glast = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                __builtin_bit_cast(int, bs.zsc[0])));
          if (glast != 1.0f) {
#pragma unroll
            for (int mb = 0; mb < DK / 16; ++mb) Sacc[mb] = Sacc[mb] * glast;
          }
          glast = 1.0f;
        }
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb) {
          const char *p = Kb + kt_off[mb >> 1] + 8 * (mb & 1);
          const bf16x8 a = cat(ld_tr4(reinterpret_cast<const bf16 *>(p)),
                               ld_tr4(reinterpret_cast<const bf16 *>(p + 16 * QRB)));
          f32x4 acc = Sacc[mb] * glast;
          acc = mfma_bf16(a, Wh, acc);
          acc = mfma_bf16(a, Wl, acc);
          Sacc[mb] = acc;
        }
        // lane holds O[16 rb + lr][col0 + 4 lg .. +3], stored straight from
        // the accumulator by one wide store (the 4 lanes of a row write its
        // 16 adjacent values).  Rows past the end of the sequence lie beyond
        // the descriptor (row r >= n starts at r H DV >= (n - 1) H DV + DV
        // elements) and are dropped: no branch on the row count
#pragma unroll
        for (int rb = 0; rb < 2 && WANT_O; ++rb) {
          f32x4 acc = oacc[rb];
          if constexpr (FUSED) acc = acc * og[rb];
          buf_st4(acc, ro, ooff[rb], OutT{});
        }
      }
     }
      __syncthreads();
    }

    if (final_state) {
      // the carried scale after the last chunk (1 without chunks)
      float zf = 1.0f;
      if (LAZY && nchunks > 0)
        zf = at_off(&sm.in[0], slot_off((nchunks - 1) % NIN, (int)sizeof(In)))->zsc[1];
      float *SF = final_state + (long)chain * DK * DV;
#pragma unroll
      for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) SF[(long)srow(mb, e) * DV + col0 + lr] = Sacc[mb][e] * zf;
    }
    return;
  }

  // =======================================================================
  // prep waves
  // =======================================================================
  const int pw = wave - NSW;           // prep wave index 0..NPW-1

  // The A tile (K K^T: strict lower, times b) and the P tile (Q K^T: lower
  // inclusive) at one position (ti, tj), with the decay: both take the key
  // rows of block tj as their right operand (read once, and once in all on
  // the diagonal, where A's left operand is the same rows) and the same
  // factors e^{g_r - g_s} (formed once).  Lane (lr, lg) ends up with rows
  // 16 ti + 4 lg + e of column 16 tj + lr.  g and b are the calling wave's
  // copies; with the fused normalisation A takes the row factor 1/|k_r| and
  // P 1/|q_r|, both the column factor 1/|k_s|.
  auto tile_pair = [&](const In &bf, const float *g, const float *bw, int ti, int tj, f32x4 &va,
                       f32x4 &vp) {
    const char *Kc = reinterpret_cast<const char *>(&bf.K[0][0]);
    const char *Qc = reinterpret_cast<const char *>(&bf.Q[0][0]);
    f32x4 aa = {0.f, 0.f, 0.f, 0.f}, ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KKD; ++kk) {
      const bf16x8 kt = ld8(reinterpret_cast<const bf16 *>(Kc + 16 * tj * QRB + kq_off[kk]));
      if constexpr (ERASE) {
        const bf16x8 ki =
            (ti == tj) ? kt : ld8(reinterpret_cast<const bf16 *>(Kc + 16 * ti * QRB + kq_off[kk]));
        aa = mfma_bf16(ki, kt, aa);
      }
      if constexpr (WANT_P)
        ap = mfma_bf16(ld8(reinterpret_cast<const bf16 *>(Qc + 16 * ti * QRB + kq_off[kk])), kt, ap);
    }
    const int sc = 16 * tj + lr;
    const int r0 = 16 * ti + 4 * lg;
    const float gs = g[sc];
    const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(&g[r0]);
    // the norms are read whether or not they were formed and picked by a
    // select: a branch here would sit between the tiles' MFMAs and the reads
    // of their results, which can hide the wait states those reads need
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&bw[r0]);
    const float nks = bf.nrm[1][sc];
    const f32x4 nkr = *reinterpret_cast<const f32x4 *>(&bf.nrm[1][r0]);
    const f32x4 nqr = *reinterpret_cast<const f32x4 *>(&bf.nrm[0][r0]);
    const bool l2 = (fuse & kFuseL2) != 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dec = (GATE == kGateNone) ? 1.0f : __expf(gr4[e] - gs);
      const float fa = l2 ? b0[e] * nkr[e] * nks : b0[e];
      const float fp = l2 ? nqr[e] * nks : 1.0f;
      va[e] = (sc < r0 + e) ? fa * aa[e] * dec : 0.0f;
      vp[e] = (sc <= r0 + e) ? fp * ap[e] * dec : 0.0f;
    }
  };
  auto store_p = [&](typename SM::PT &pt, f32x4 val, int ti, int tj) {
    bf16x4 h4, l4;
    split4(val, h4, l4);
    *reinterpret_cast<bf16x4 *>(&pt.Ph[16 * tj + lr][16 * ti + 4 * lg]) = h4;
    *reinterpret_cast<bf16x4 *>(&pt.Pl[16 * tj + lr][16 * ti + 4 * lg]) = l4;
  };

  if (pw == 3) {
    // ---- solver wave: T = (I + A)^{-1} of chunk it, stored unscaled (the
    //      state waves scale R by b, as T' R = T (b o R)) ----
    __syncthreads();
    __syncthreads();
    for (int it = 0; it < nchunks + 1; ++it) {
      if (ERASE && it < nchunks) {   // no solve without the erase term
        const int j = it;
        const int tso = slot_off(j % NTS, (int)sizeof(sm.Th[0]));
        const int ao = slot_off(j & 1, (int)sizeof(sm.ATd[0]));
        const int a10o = slot_off(j & 1, (int)sizeof(sm.A10h[0]));
        // diagonal 16x16 blocks (A tiles from the last iteration); lane =
        // (block, column); right-looking forward substitution: once x_s is
        // final it updates all later rows, so the dependent chain is one FMA
        // per step.  Lane col of a 16-lane row holds column col of -A; step s
        // takes column s from lane s by a row broadcast (DPP row_newbcast)
        // folded into the FMA, so A is read from LDS once, without
        // broadcast reads
        {
          const int blk = (lane >> 4) & 1, col = lane & 15, o0 = 16 * blk;
          float na[16];                          // na[r] = -A[o0 + r][o0 + col]
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(&(*at_off(&sm.ATd[0], ao))[blk][col][4 * q4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) na[4 * q4 + e] = t[e];
          }
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.0f : 0.0f;
#pragma unroll
          for (int s2 = 0; s2 < 15; ++s2) {
#pragma unroll
            for (int r = s2 + 1; r < 16; ++r)
              asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                           : "+v"(x[r]) : "v"(na[r]), "v"(x[s2]), "i"(s2));
          }
          // T^T[o0 + col][o0 + r] = x[r], hi/lo (lanes 32..63 hold duplicates)
          if (lane < 32) {
            unsigned h8[2][4], l8[2][4];
#pragma unroll
            for (int r = 0; r < 16; r += 2) split2(x[r], x[r + 1], h8[r / 8][(r % 8) / 2], l8[r / 8][(r % 8) / 2]);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              *reinterpret_cast<u32x4 *>(&at_off(&sm.Th[0][0], tso)[o0 + col][o0 + 8 * hf]) =
                  u32x4{h8[hf][0], h8[hf][1], h8[hf][2], h8[hf][3]};
              *reinterpret_cast<u32x4 *>(&at_off(&sm.Tl[0][0], tso)[o0 + col][o0 + 8 * hf]) =
                  u32x4{l8[hf][0], l8[hf][1], l8[hf][2], l8[hf][3]};
            }
          }
        }
        wave_lds_sync();
        // block (1,0), T10 = -T11 A10 T00, from the diagonal blocks just
        // written: two 16x16x16 split products, the first result fed to the
        // second as its B operand straight from the accumulator
        bf16(*Th)[SM::LDC] = at_off(&sm.Th[0][0], tso);
        bf16(*Tl)[SM::LDC] = at_off(&sm.Tl[0][0], tso);
        // Y1 = A10 T00: A operand A10[m][4 lg ..] = column m of A10^T rows 4 lg..;
        // B operand T00[4 lg ..][n] = row n of T^T
        const bf16x4 ah = ld_tr4(&at_off(&sm.A10h[0][0], a10o)[4 * lg + (lr >> 2)][4 * (lr & 3)]);
        const bf16x4 al = ld_tr4(&at_off(&sm.A10l[0][0], a10o)[4 * lg + (lr >> 2)][4 * (lr & 3)]);
        const bf16x4 bh = *reinterpret_cast<const bf16x4 *>(&Th[lr][4 * lg]);
        const bf16x4 bl = *reinterpret_cast<const bf16x4 *>(&Tl[lr][4 * lg]);
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        y = mfma16_bf16(ah, bh, y);
        y = mfma16_bf16(ah, bl, y);
        y = mfma16_bf16(al, bh, y);
        bf16x4 yh, yl;
        split4(y, yh, yl);
        // Z = T11 Y1: A operand T11[m][4 lg ..] = column 16 + m of T^T rows 16 + 4 lg..
        const bf16x4 th = ld_tr4(&Th[16 + 4 * lg + (lr >> 2)][16 + 4 * (lr & 3)]);
        const bf16x4 tl = ld_tr4(&Tl[16 + 4 * lg + (lr >> 2)][16 + 4 * (lr & 3)]);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mfma16_bf16(th, yh, z);
        z = mfma16_bf16(th, yl, z);
        z = mfma16_bf16(tl, yh, z);
        // lane holds Z[4 lg + e][lr]: T^T[lr][16 + 4 lg + e] = -Z
        bf16x4 h4, l4;
        split4(-z, h4, l4);
        *reinterpret_cast<bf16x4 *>(&Th[lr][16 + 4 * lg]) = h4;
        *reinterpret_cast<bf16x4 *>(&Tl[lr][16 + 4 * lg]) = l4;
      }
      __syncthreads();
    }
    return;
  }

  // ---- prep waves 0..2: LDS DMA, decay scan, A and P tiles ----
  // DMA shares: wave 0 v (+ log a, b), wave 1 k, wave 2 q.  Instruction i of
  // a matrix fills LDS bytes 1024 i .. +1023 of its tile: lane l lands at
  // row i RPI + l / BPR, stored block l % BPR, and fetches the natural block
  // that the row's permutation puts there.
  constexpr int NQI = C * QRB / 1024, NVI = C * VRB / 1024;
  constexpr int NI = (NQI > NVI) ? NQI : NVI;
  constexpr bool SCALAR = (GATE == kGateScalar);
  constexpr int N0 = NVI + 1 + (SCALAR ? 1 : 0);   // DMA instructions per chunk, wave 0
  constexpr int N12 = NQI;                         // waves 1 and 2
  unsigned voff[NI];
  float zscale = 1.0f;                 // carried scale of the state entering the next chunk (wave 0)
  if (pw == 0) {
    constexpr int BPR = VRB / 16, RPI = 1024 / VRB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + lane / BPR, sb = lane % BPR;
      voff[i] = (unsigned)row * (2u * H * DV) + (unsigned)(2 * slice * DVS + 16 * (sb ^ swz_v<VB>(row)));
    }
  } else {
    constexpr int BPR = QRB / 16, RPI = 1024 / QRB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + lane / BPR, sb = lane % BPR;
      voff[i] = (unsigned)row * (2u * H * DK) + (unsigned)(16 * (sb ^ swz_qk<QB>(row)));
    }
  }
  const unsigned soff = (unsigned)(lane * H * 4);   // log a / b of token `lane`

  auto issue = [&](int j) {
    In &dst = sm.in[j % NIN];
    const int cj = chunk_of(j);
    const int n = min(C, T - cj * C);
    const long row0 = tok0 + (long)cj * C * H;        // token row of the chunk's first token
    if (pw == 0) {
      // v rows (all slices' columns of rows < n are inside the descriptor)
      const u32x4 rv = rsrc_words(v + row0 * DV, 2u * ((unsigned)(n - 1) * H * DV + DV));
      const unsigned lv = lds_addr(&dst.V[0][0]);
#pragma unroll
      for (int i = 0; i < NVI; ++i) lds_dma16(rv, voff[i], lv + 1024 * i);
      lds_dma4(rsrc_words(beta + row0, 4u * ((unsigned)(n - 1) * H + 1)), soff, lds_addr(&dst.beta[0]));
      if constexpr (SCALAR)
        lds_dma4(rsrc_words(log_alpha + row0, 4u * ((unsigned)(n - 1) * H + 1)), soff, lds_addr(&dst.la[0]));
    } else {
      if (!WANT_P && pw == 2) return;                  // q feeds only P and Q S
      const bf16 *src = (pw == 1) ? k : q;
      const u32x4 rq = rsrc_words(src + row0 * DK, 2u * ((unsigned)(n - 1) * H * DK + DK));
      const unsigned lq = lds_addr(pw == 1 ? &dst.K[0][0] : &dst.Q[0][0]);
#pragma unroll
      for (int i = 0; i < NQI; ++i) lds_dma16(rq, voff[i], lq + 1024 * i);
    }
  };
  // wait for every DMA of chunk j when chunk j+1 was issued after it
  auto wait_prev = [&](bool newer_issued) {
    if (newer_issued) {
      if (pw == 0) wait_vmcnt<N0>();
      else wait_vmcnt<N12>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // The tiles of chunk j on waves 0..2.  Each wave takes the in-chunk
  // cumulative log decay itself (an inclusive scan over lanes 0..C-1;
  // tokens past the end carry log a = 0 and b = 0) into its own copy of g,
  // so no tile waits on another wave; wave 0 also writes e^g and
  // e^{g_last - g} for the state waves.  Shares, by position: wave 0 the
  // off-diagonal block (A10 and P10), wave 1 the second diagonal block,
  // wave 2 the first (A and P of one position share their key operands and
  // decay factors).
  auto tiles = [&](int j) {
    In &bf = *at_off(&sm.in[0], slot_off(j % NIN, (int)sizeof(In)));
    float *g = sm.gw[pw], *bw = sm.bw[pw];
    // padded tokens carry log a = 0 and b = 0 after the fused transforms too
    const int n = min(C, T - chunk_of(j) * C);
    const float la = (SCALAR && lane < n) ? fused_log_alpha(bf.la[lane], fuse) : 0.0f;
    const float sc = scan32_inclusive(la);
    const float bl = (lane < n) ? fused_beta(bf.beta[lane], fuse) : 0.0f;
    if (lane < C) {
      g[lane] = sc;
      bw[lane] = bl;
    }
    if (pw == 0) {
      // the state waves' factors: e^g for Q S and K S (times 1/|q|, 1/|k|),
      // e^{g_last - g} (times 1/|k|) for the update, b
      const float glast = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), C - 1));
      // carried scale: z = scale entering the chunk; the state factor before
      // the update and the scale after it (uniform)
      float z = 1.0f, zinv = 1.0f;
      if constexpr (LAZY) {
        const float zn = zscale * __expf(glast);
        const bool fold = zn < 0x1p-40f;
        z = zscale;
        zscale = fold ? 1.0f : zn;
        zinv = 1.0f / zscale;
        if (lane == 0) {
          bf.zsc[0] = fold ? zn : 1.0f;
          bf.zsc[1] = zscale;
        }
      }
      if (lane < C) {
        const float gm = (GATE == kGateNone) ? 1.0f : __expf(sc);
        const float e = (GATE == kGateNone) ? 1.0f : __expf(glast - sc);
        const bool l2 = (fuse & kFuseL2) != 0;
        const float nq = bf.nrm[0][lane], nk = bf.nrm[1][lane];
        const float rq = l2 ? nq : 1.0f, rk = l2 ? nk : 1.0f;
        bf.gam[lane] = gm;
        bf.fq[lane] = gm * rq * z;
        bf.fk[lane] = gm * rk * z;
        bf.ec[lane] = e * rk * zinv;
        bf.bt[lane] = bl;
      }
    }
    wave_lds_sync();
    typename SM::PT &pt = *at_off(&sm.p[0], slot_off(j % NPR, (int)sizeof(typename SM::PT)));
    const int a10o = slot_off(j & 1, (int)sizeof(sm.A10h[0]));
    const int ao = slot_off(j & 1, (int)sizeof(sm.ATd[0]));
    f32x4 va, vp;
    if (pw == 0) {
      tile_pair(bf, g, bw, 1, 0, va, vp);
      if constexpr (ERASE) {
        bf16x4 h4, l4;
        split4(va, h4, l4);
        *reinterpret_cast<bf16x4 *>(&at_off(&sm.A10h[0][0], a10o)[lr][4 * lg]) = h4;
        *reinterpret_cast<bf16x4 *>(&at_off(&sm.A10l[0][0], a10o)[lr][4 * lg]) = l4;
      }
      if constexpr (WANT_P) store_p(pt, vp, 1, 0);
    } else {
      // wave 1: block (1,1); wave 2: block (0,0)
      const int b = (pw == 1) ? 1 : 0;
      if (pw == 1) tile_pair(bf, g, bw, 1, 1, va, vp);
      else tile_pair(bf, g, bw, 0, 0, va, vp);
      if constexpr (ERASE) *reinterpret_cast<f32x4 *>(&(*at_off(&sm.ATd[0], ao))[b][lr][4 * lg]) = -va;
      if constexpr (WANT_P) store_p(pt, vp, b, b);
    }
  };

  // fused L2 normalisation: 1/|row| of chunk j's k (wave 1) or q (wave 2),
  // formed by the wave whose DMA brought the rows, right after its wait;
  // lane = (row, half row)
  auto norms = [&](int j) {
    In &bf = *at_off(&sm.in[0], slot_off(j % NIN, (int)sizeof(In)));
    const char *X = reinterpret_cast<const char *>(pw == 1 ? &bf.K[0][0] : &bf.Q[0][0]);
    const int r = lane & (C - 1), h = lane / C;
    // the two lanes of a row take complementary halves of its blocks, in an
    // order rotated by a function of the row that is distinct over the 16
    // lanes of one ds_read_b128 pass (rows 256 bytes apart would otherwise
    // all hit the same banks)
    const int rot = (r & 3) + 4 * ((r >> 3) & 3);
    float ss4[4] = {0.f, 0.f, 0.f, 0.f};   // four independent sums: short chains
#pragma unroll
    for (int b = 0; b < QB / 2; ++b) {
      const int blk = (b + h * (QB / 2) + rot) & (QB - 1);
      const u32x4 w4 = *reinterpret_cast<const u32x4 *>(X + r * QRB + 16 * blk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // x0^2 + x1^2 of a bf16 pair, one packed dot product
        // (through a scalar: a bit_cast of the vector element itself reads
        // element 0 with this compiler)
        const unsigned u = w4[i];
        const bf16x2 x2 = __builtin_bit_cast(bf16x2, u);
        ss4[i] = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, ss4[i], false);
      }
    }
    float ss = (ss4[0] + ss4[1]) + (ss4[2] + ss4[3]);
    ss += __shfl_xor(ss, C);
    if (lane < C) bf.nrm[pw == 1 ? 1 : 0][lane] = rsqrtf(ss + kL2Eps);
  };
  const bool l2 = (fuse & kFuseL2) && (pw == 1 || pw == 2);

  // prologue: chunks 0..2 in flight; chunks 0 and 1 landed (and normalised);
  // the tiles of chunk 0 formed
  if (nchunks > 0) issue(0);
  if (nchunks > 1) issue(1);
  if (nchunks > 2) issue(2);
  wait_prev(nchunks > 2);
  if (l2 && nchunks > 0) norms(0);
  if (l2 && nchunks > 1) norms(1);
  __syncthreads();
  if (nchunks > 0) tiles(0);
  __syncthreads();

  for (int it = 0; it < nchunks + 1; ++it) {
    // DMA of chunk it+3; tiles of chunk it+1 (landed by the last barrier);
    // then wait for this wave's DMA of chunk it+2
    const bool more = it + 3 < nchunks;
    if (more) issue(it + 3);
    if (it + 1 < nchunks) tiles(it + 1);
    wait_prev(more);
    if (l2 && it + 2 < nchunks) norms(it + 2);
    __syncthreads();
  }
}

template <int DK, int DVS, typename OutT, int GATE, bool ERASE, bool FUSED>
hipError_t launch_fused(const ChunkArgs &a) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + NPW));
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVS, OutT, GATE, ERASE, FUSED, kModeFwd>), grid,
                     block, 0, a.stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     a.beta, a.log_alpha, a.initial_state, (OutT *)a.o, a.final_state, a.B, a.T,
                     a.H, a.fuse, (const bf16 *)a.out_gate, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

// the forward that also stores h and U per chunk (the recompute pass's
// stores) at one tile configuration
template <int DK, int DVS, typename OutT, int GATE, bool ERASE>
hipError_t launch_save(const ChunkArgs &a, float *ws_h, float *ws_u) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + NPW));
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVS, OutT, GATE, ERASE, false, kModeFwdSave>),
                     grid, block, 0, a.stream, (const bf16 *)a.q, (const bf16 *)a.k,
                     (const bf16 *)a.v, a.beta, a.log_alpha, a.initial_state, (OutT *)a.o,
                     a.final_state, a.B, a.T, a.H, 0, nullptr, ws_h, ws_u, nullptr);
  return hipGetLastError();
}

template <int DK, int DVS, typename OutT>
hipError_t save_by_gate(const ChunkArgs &a, float *ws_h, float *ws_u) {
  if (a.erase) {
    if (a.gate == kGateNone) return launch_save<DK, DVS, OutT, kGateNone, true>(a, ws_h, ws_u);
    return launch_save<DK, DVS, OutT, kGateScalar, true>(a, ws_h, ws_u);
  }
  if (a.gate == kGateNone) return launch_save<DK, DVS, OutT, kGateNone, false>(a, ws_h, ws_u);
  return launch_save<DK, DVS, OutT, kGateScalar, false>(a, ws_h, ws_u);
}

template <int DK, int DVS>
hipError_t save_by_out(const ChunkArgs &a, float *ws_h, float *ws_u) {
  return a.out_bf16 ? save_by_gate<DK, DVS, bf16>(a, ws_h, ws_u)
                    : save_by_gate<DK, DVS, float>(a, ws_h, ws_u);
}

// the backward's two sequential passes at one tile configuration (the first
// skipped when a training forward has stored its results)
template <int DK, int DVS, int GATE, bool ERASE>
hipError_t launch_passes(const BwdArgs &a) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + NPW));
  if (!a.saved) {
    hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVS, float, GATE, ERASE, false, kModeRec>),
                       grid, block, 0, a.stream, (const bf16 *)a.q, (const bf16 *)a.k,
                       (const bf16 *)a.v, a.beta, a.log_alpha, a.initial_state, nullptr, nullptr,
                       a.B, a.T, a.H, 0, nullptr, a.ws_h, a.ws_u, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<DK, DVS, float, GATE, ERASE, false, kModeRev>), grid,
                     block, 0, a.stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.d_o,
                     a.beta, a.log_alpha, a.d_final_state, nullptr, a.d_initial_state, a.B, a.T,
                     a.H, 0, nullptr, a.ws_dh, a.ws_dy, nullptr);
  return hipGetLastError();
}

template <int DK, int DVS>
hipError_t passes_by_gate(const BwdArgs &a) {
  if (a.erase) {
    if (a.gate == kGateNone) return launch_passes<DK, DVS, kGateNone, true>(a);
    return launch_passes<DK, DVS, kGateScalar, true>(a);
  }
  if (a.gate == kGateNone) return launch_passes<DK, DVS, kGateNone, false>(a);
  return launch_passes<DK, DVS, kGateScalar, false>(a);
}

template <int DK, int DVS, typename OutT, int GATE, bool ERASE>
hipError_t launch_cfg(const ChunkArgs &a) {
  if (a.fuse != 0 || a.out_gate != nullptr) return launch_fused<DK, DVS, OutT, GATE, ERASE, true>(a);
  return launch_fused<DK, DVS, OutT, GATE, ERASE, false>(a);
}

template <int DK, int DVS, typename OutT>
hipError_t by_gate(const ChunkArgs &a) {
  if (a.erase) {
    if (a.gate == kGateNone) return launch_cfg<DK, DVS, OutT, kGateNone, true>(a);
    return launch_cfg<DK, DVS, OutT, kGateScalar, true>(a);
  }
  if (a.gate == kGateNone) return launch_cfg<DK, DVS, OutT, kGateNone, false>(a);
  return launch_cfg<DK, DVS, OutT, kGateScalar, false>(a);
}

template <int DK, int DVS>
hipError_t by_out(const ChunkArgs &a) {
  return a.out_bf16 ? by_gate<DK, DVS, bf16>(a) : by_gate<DK, DVS, float>(a);
}

}  // namespace

bool chunk_fwd_bf16_supported(const ChunkArgs &a) {
  // the kernel's chunk is 32 tokens; a requested chunk size only changes
  // rounding, so 0, 16, 32 and 64 all map here.  Its per-chunk buffer
  // descriptors span one chunk's rows of a [*, H, D] tensor and must stay
  // below 4 GiB (H * D below ~34 million)
  const long chunk_bytes = (long)4 * ((long)(C - 1) * a.H * a.D + a.D);
  return a.in_bf16 && (a.D == 128 || a.D == 64) && a.gate != kGateChannel &&
         chunk_bytes < 0xFFFFFFFFL;
}

bool chunk_bwd_supported(int D, bool in_bf16, int gate, bool erase, long H) {
  // the per-chunk buffer descriptors (of the widest rows: fp32 [*, H, D]) are
  // 32-bit; the bound of the 32-token chunk covers the 16-token one too
  const long chunk_bytes = (long)4 * ((long)(C - 1) * H * D + D);
  (void)erase;   // both forms: with the erase term and without (additive write)
  return in_bf16 && (D == 128 || D == 64) && chunk_bytes < 0xFFFFFFFFL &&
         (gate == kGateNone || gate == kGateScalar || gate == kGateChannel);
}

hipError_t launch_chunk_bwd_passes(const BwdArgs &a) {
  static_assert(C == kBwdChunk, "the workspace holds this kernel's chunks");
  // the forward's launch shapes: 64-column slices once there are >= 256
  // (chain, slice) pairs, 32-column slices below
  const long chains = (long)a.B * a.H;
  if (a.D == 128) {
    if (chains * 2 >= 256) return passes_by_gate<128, 64>(a);
    return passes_by_gate<128, 32>(a);
  }
  if (chains >= 256) return passes_by_gate<64, 64>(a);
  return passes_by_gate<64, 32>(a);
}

hipError_t launch_chunk_fwd_bf16_save(const ChunkArgs &a, float *ws_h, float *ws_u) {
  static_assert(C == kBwdChunk, "the workspace holds this kernel's chunks");
  const long chains = (long)a.B * a.H;   // the forward's launch shapes
  if (a.D == 128) {
    if (chains * 2 >= 256) return save_by_out<128, 64>(a, ws_h, ws_u);
    return save_by_out<128, 32>(a, ws_h, ws_u);
  }
  if (chains >= 256) return save_by_out<64, 64>(a, ws_h, ws_u);
  return save_by_out<64, 32>(a, ws_h, ws_u);
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
