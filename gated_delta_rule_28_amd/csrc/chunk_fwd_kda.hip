// Chunkwise KDA forward (per-channel decay), bf16 q/k/v, fp32 state, MFMA (gfx950).
//
// Method.  S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t, a_t in [0,1]^{d_k} (page "NLP——线性注意力相关总结", section
// "Kimi Delta Attention (KDA)"), evaluated chunkwise with the WY form and a
// triangular solve (xhh.club digest "Transformer 入坑笔记（五）", KDA Q&A).
// Per chunk of C = 16 tokens, entering state S, G = in-chunk cumulative
// log decay per (token, channel), g_last its last row:
//
//   K^ = K o e^G,  Q^ = Q o e^G,  R^ = K o e^{-G}
//   A_rs = b_r (K^ R^T)_rs   (s < r)      Gram
//   P_rs =     (Q^ R^T)_rs   (s <= r)     masked scores
//   T'   = (I + A)^{-1} diag(b)
//   U    = T' (V - K^ S)
//   O    = Q^ S + P U
//   S   <- Diag(e^{g_last}) (S + R^T U)
//
// The last line is Diag(e^{g_last}) S + (K o e^{g_last - G})^T U with the
// per-channel factor taken out of the product, so one derived key operand
// (R^) serves the Gram, the scores and the state update.  The in-chunk
// decays e^{G_r - G_s} factor about the chunk start; the page digest notes
// that they can be tiny, so direct division is avoided and the factors stay
// in range: K^ and Q^ are at most |k|, |q|, and R^ is at most e^{64} |k|
// while every channel's in-chunk log decay stays above -64.  A chunk with a
// channel below that (a near-hard reset) takes an exact path: its Gram and
// scores are formed with every decay e^{G_rc - G_sc} directly in fp32, and
// its state update uses K o e^{g_last - G} with the factor applied first.
//
// Derived operands are not exact bf16, so every product takes three MFMAs
// (hi*hi + hi*lo + lo*hi).
//
// Without the erase term (S_t = Diag(a_t) S_{t-1} + b_t k_t v_t^T, GLA's
// per-channel decay; xhh.club digest, abstract and Q&A) A = 0 and
// U = diag(b) V: the same kernel skips K^, K^ S, the Gram and the solve
// (template flag ERASE).
//
// Mapping.  One workgroup per (batch, head, Dv slice of DVS columns); DVS/16
// state waves keep the state in MFMA accumulators with the k axis ordered as
// in the scalar-gate kernel (tile pair (2kk, 2kk+1) holds dk 32kk + 8g + j and
// 32kk + 8g + 4 + j in rows 4g + j), so K^ S, Q^ S take the state straight
// from registers and the update reads R^ transposed from a row-major tile.
// Four or six prep waves; one workgroup barrier per iteration; in iteration i
//   wave 0: LDS DMA of log a and b of chunk i+3; derives chunk i (a share)
//   wave 1: LDS DMA of q, k of chunk i+3; sums the log decays of chunk i+1;
//           derives chunk i (a share)
//   wave 2: scores of chunk i-1; derives chunk i (a share)
//   wave 3: Gram and solve of chunk i-1 (without the erase term: derives
//           chunk i, a share)
//   waves 4, 5 (32-column slices): derive chunk i (shares)
//   LDS DMA of v of chunk i: wave 5, or wave 2 with four prep waves
//   state:  chunk i-2
//   with a fused decay transform, the state waves (and with six prep waves
//   also waves 3 and 5) transform chunk i+2's decay pre-activations, a share
//   of its rows each
// Raw inputs live four iterations (DMA to derivation), derived operands
// three, v three, T' and P two.
//
// Backward passes (template MODE).  kModeRec recomputes the forward and
// stores, per chunk, the entering state h and U (no outputs, no scores);
// kModeRev walks the chunks in reverse with v = dO and the state gradient X
// (the gradient of the state leaving the chunk; dS_T in, dS_0 out) in the
// accumulators, the adjoint of the lines above:
//
//   Y1  = Diag(e^{g_last}) X                     (the exact path: Y1 = X)
//   dU  = R^ Y1 + P^T dO,   dY = T^T dU          (T = (I + A)^{-1}, unscaled)
//   X  <- Y1 + Q^ ^T dO - K^ ^T diag(b) dY      (the exact path: e^{g_last} o Y1)
//
// storing X and dY per chunk; the solver stores T instead of T' in that mode.
// The chunk-parallel kernel (chunk_bwd_kda.hip) forms the token gradients.
// kModeFwdSave, the training forward, is the forward with kModeRec's stores.
#include <cstddef>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace gdr {
namespace {

constexpr int KC = 16;               // tokens per chunk
// prep waves: 4, or 6 with 32-column slices (8 waves, two per SIMD)
template <int DVS>
constexpr int kda_npw() { return DVS == 32 ? 6 : 4; }
constexpr float kMaxSpan = 64.0f;    // per-channel in-chunk log-decay bound of the factored form
// The in-chunk log decays are kept in base-2 units (G = log2 of the decay
// products), so that every factor e^{...} is one hardware exp2.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxSpan2 = kMaxSpan * kLog2e;   // the bound in those units
constexpr int NRAW = 4;              // raw slots: chunk j from iteration j-3 to j
constexpr int NDER = 3;              // derived slots: chunk j from iteration j to j+2
constexpr int NVB = 3;               // v slots: chunk j from iteration j to j+2

template <int DK, int DVS>
struct __align__(16) KdaSmem {
  static constexpr int LDX = 20;          // fp32 stride of the 16x16 exact-path and solve tiles
  struct __align__(16) Raw {              // one chunk as the DMA leaves it
    bf16 Q[KC][DK], K[KC][DK];            // natural channel order
    float G[KC][DK];                      // log a, summed in place into G (base 2)
    float beta[64];                       // b of the 64 tokens from the chunk start (16 used)
    float nrm[2][KC];                     // fused L2 normalisation: 1/|q|, 1/|k| per token
    int flag[4];                          // [0]: some channel's in-chunk log decay < -kMaxSpan
  };
  struct __align__(16) Der {              // operands of one chunk, rows permuted by swz_qk
    bf16 Kh[KC][DK], Kl[KC][DK];          // K^ = K o e^G
    bf16 Qh[KC][DK], Ql[KC][DK];          // Q^ = Q o e^G
    bf16 Rh[KC][DK], Rl[KC][DK];          // R^ = K o e^{-G} (exact path: K o e^{g_last - G})
    float egl[DK];                        // e^{g_last}
    float egp[DK];                        // the factor after the update: e^{g_last}, or 1 on
                                          // the exact path (which applies it first)
    float beta[KC];
    int flag[4];
  };
  Raw raw[NRAW];
  Der der[NDER];
  bf16 V[NVB][KC][DVS];                   // v rows of this slice, blocks permuted by swz_v
  bf16 Th[2][KC][KC], Tl[2][KC][KC];      // T'^T: [s][r] = T'[r][s]
  bf16 Ph[2][KC][KC], Pl[2][KC][KC];      // P^T
  float xA[2][KC][LDX];                   // exact path: -A^T ([s][r] = -A[r][s])
  float xP[2][KC][LDX];                   // exact path: P^T
  float At[KC][LDX];                      // -A^T of the chunk being solved
};

// ws_a, ws_b: the backward passes' per-chunk stores ([chain][chunk] of
// [DK][DV] and [KC][DV] fp32): h and U (kModeRec), X and dY (kModeRev)
template <int DK, int DVS, typename OutT, bool ERASE, bool FUSED, int MODE>
__global__ void __launch_bounds__(64 * (DVS / 16 + kda_npw<DVS>()), 1)
chunk_fwd_kda_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                     const bf16 *__restrict__ v, const float *__restrict__ beta,
                     const float *__restrict__ log_alpha, const float *initial_state,
                     OutT *__restrict__ o, float *final_state, int B, int T, int H, int fuse,
                     const bf16 *__restrict__ out_gate, float *__restrict__ ws_a,
                     float *__restrict__ ws_b) {
  constexpr int NSW = DVS / 16;
  constexpr int DV = DK;
  constexpr int NSLICE = DV / DVS;
  constexpr int KKD = DK / 32;
  constexpr int QB = DK / 8, VB = DVS / 8;      // 16-byte blocks per q/k and v row
  constexpr int QRB = 2 * DK, VRB = 2 * DVS;    // bytes per q/k and v row
  static_assert((DK == 64 || DK == 128) && (DVS == 32 || DVS == 64) && DVS <= DK, "tile config");
  static_assert(MODE == kModeFwd || !FUSED, "the backward passes take no fused options");
  constexpr bool WANT_O = MODE == kModeFwd || MODE == kModeFwdSave;   // outputs (Q^ S, P U, o)
  constexpr bool SAVE = MODE == kModeRec || MODE == kModeFwdSave;     // h and U per chunk
  constexpr bool WANT_P = MODE != kModeRec;    // Q^ and the P tiles
  // calls without a fused prologue or epilogue compile without their code
  if constexpr (!FUSED) {
    fuse = 0;
    out_gate = nullptr;
  }
  using SM = KdaSmem<DK, DVS>;
  static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
  static_assert(sizeof(typename SM::Raw) % 16 == 0 && sizeof(typename SM::Der) % 16 == 0 &&
                    (KC * QRB) % 1024 == 0 && (KC * VRB) % 1024 == 0,
                "DMA runs are whole 1 KiB waves");
  __shared__ SM sm;
  static_assert(sizeof(sm.Th[0]) == sizeof(sm.Ph[0]), "T' and P slots share one offset");

  const int tid = threadIdx.x, lane = tid & 63;
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
  const int nchunks = (T + KC - 1) / KC;
  const long tok0 = (long)bb * T * H + hh;   // token row of token 0 of this chain
  // the sequence chunk of pipeline position j (the reverse pass runs last to first)
  auto chunk_of = [&](int j) { return MODE == kModeRev ? nchunks - 1 - j : j; };

  // byte offset inside a derived tile of row r, natural 16-byte block b
  auto qk_at = [](int r, int b) { return r * QRB + 16 * (b ^ swz_qk<QB>(r)); };
  // row reads: lane (lr, lg) takes row lr, dk 32 kk + 8 lg .. +7
  int kq_off[KKD];
#pragma unroll
  for (int kk = 0; kk < KKD; ++kk) kq_off[kk] = qk_at(lr, 4 * kk + lg);

  // With a fused decay transform (two transcendentals per element) the waves
  // that wait at the barrier for much of an iteration in that kernel turn
  // chunk j's decay pre-activations into log2 a in place in iteration
  // j - 2, a share of the rows each; the raw DMA waves then wait
  // for their loads within the iteration that issues them (a chunk's loads
  // land well inside one iteration), so chunk j is in LDS from iteration
  // j - 2 on, and its sums in iteration j - 1 add the transformed values.
  const bool xf = FUSED && (fuse & (kFuseSoftplus | kFuseGla)) != 0;
  // The transform's rows are shared by the waves that have time to spare:
  // the state waves, and with six prep waves also the solver and the v DMA
  // wave (prep waves 3 and 5), two row passes each, the state waves the
  // rest.  A pass is TPRX rows of 64 lanes, a lane one channel pair; NP
  // passes from pass pb, straight-line.  Padded tokens get log a = 0.
  constexpr int NCPX = DK / 2, TPRX = 64 / NCPX, NPT = KC / TPRX;
  constexpr int XSIDE = (DVS == 32) ? 2 * NPT / 16 : 0;        // passes of waves 3 and 5 each
  constexpr int XSTATE = (NPT - 2 * XSIDE) / (DVS / 16);       // passes of each state wave
  static_assert(XSTATE * (DVS / 16) + 2 * XSIDE == NPT, "transform shares cover the chunk");
  auto xform = [&](int j, int pb, auto np_) {
    constexpr int NP = decltype(np_)::value;
    typename SM::Raw &rw = *at_off(&sm.raw[0], slot_off(j % NRAW, (int)sizeof(typename SM::Raw)));
    const int n = min(KC, T - chunk_of(j) * KC);
    const int c0 = 2 * (lane % NCPX), r0 = TPRX * pb + lane / NCPX;
    const bool gla = (fuse & kFuseGla) != 0;
    f32x2 x[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) x[i] = *reinterpret_cast<const f32x2 *>(&rw.G[r0 + TPRX * i][c0]);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const float keep = (r0 + TPRX * i < n) ? 1.0f : 0.0f;
      *reinterpret_cast<f32x2 *>(&rw.G[r0 + TPRX * i][c0]) =
          f32x2{decay_transform2(x[i][0], gla), decay_transform2(x[i][1], gla)} * keep;
    }
  };
  // this wave's share: the state waves, then waves 3 and 5 of six prep waves
  auto xform_share = [&](int j) {
    if (wave < DVS / 16) {
      xform(j, XSTATE * wave, std::integral_constant<int, XSTATE>{});
    } else if constexpr (XSIDE > 0) {
      const int p = wave - DVS / 16;
      if (p == 3) xform(j, NPT - 2 * XSIDE, std::integral_constant<int, XSIDE>{});
      if (p == 5) xform(j, NPT - XSIDE, std::integral_constant<int, XSIDE>{});
    }
  };
  const bool xpart = wave < DVS / 16 || (DVS == 32 && (wave - DVS / 16 == 3 || wave - DVS / 16 == 5));

  // Every role runs three prologue barriers and nchunks + 2 iterations of
  // one barrier, so all waves execute the same sequence of workgroup barriers.
  if (wave < NSW) {
    // =====================================================================
    // state waves: the serial pass, 16 state columns each
    // =====================================================================
    const int col0 = slice * DVS + 16 * wave;
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
    if (xf) {
      if (nchunks > 0) xform_share(0);
      if (nchunks > 1) xform_share(1);
    }
    __syncthreads();
    __syncthreads();

    // element and byte offsets of this lane's output values from a chunk's
    // first row, unsigned 32-bit like the buffer offset they feed (the host
    // bounds one chunk's rows of a 4-byte tensor below 4 GiB)
    unsigned oel[4], ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      oel[e] = (unsigned)(4 * lg + e) * (unsigned)(H * DV) + (unsigned)(col0 + lr);
      ooff[e] = (unsigned)sizeof(OutT) * oel[e];
    }
    // v, transposing read: rows 4 lg + (lr >> 2), columns 16 wave + 4 (lr & 3) .. +3
    const int v_off = (4 * lg + (lr >> 2)) * VRB +
                      16 * ((2 * wave + ((lr & 3) >> 1)) ^ swz_v<VB>(4 * lg + (lr >> 2))) + 8 * (lr & 1);
    // R^T operand of the update for tile mb: rows (tokens) 4 lg + (lr >> 2),
    // dk srow(mb, 0) + 4 (lr & 3) .. +3 = natural block (lr & 3) + 4 (mb >> 1), half mb & 1
    int kt_off[KKD];
#pragma unroll
    for (int kk = 0; kk < KKD; ++kk) kt_off[kk] = qk_at(4 * lg + (lr >> 2), (lr & 3) + 4 * kk);
    const bf16x4 zero4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};

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

    // the fused output gate of this lane's O values, loaded one chunk ahead
    // (the state waves are the serial path: a load used in the same chunk
    // would expose its latency every chunk) and turned into the factor
    // g sigmoid(g) (1 without a gate) before the O products, which are then
    // only multiplied: a branch between an MFMA and the read of its result
    // can hide the wait states that read needs
    // The loads are unconditional: without a gate, or outside the chunks,
    // the descriptor is empty and they read zeros without touching memory.
    const bool gated = out_gate != nullptr;
    f32x4 og = {};
    unsigned og_next[4] = {};
    // this lane's K^ and Q^ fragments (hi, lo) of the chunk the next
    // iteration multiplies, read one iteration ahead: a chunk's derived slot
    // is complete from the iteration after its derivation, and the reads
    // would otherwise start every chunk's serial products with an LDS round
    // trip.  Before the first chunk (and past the last) they read a slot
    // that is not used, which is harmless.
    // (The reverse pass reads R^ into the K^ registers: its first product is
    // R^ Y1.)
    bf16x8 fkh[KKD], fkl[KKD], fqh[KKD], fql[KKD];
    auto load_kq = [&](int c) {
      const typename SM::Der &d = *at_off(&sm.der[0], slot_off(c % NDER, (int)sizeof(typename SM::Der)));
      const char *Kh = reinterpret_cast<const char *>(MODE == kModeRev ? &d.Rh[0][0] : &d.Kh[0][0]);
      const char *Kl = reinterpret_cast<const char *>(MODE == kModeRev ? &d.Rl[0][0] : &d.Kl[0][0]);
      const char *Qh = reinterpret_cast<const char *>(&d.Qh[0][0]);
      const char *Ql = reinterpret_cast<const char *>(&d.Ql[0][0]);
#pragma unroll
      for (int kk = 0; kk < KKD; ++kk) {
        if constexpr (WANT_O) {
          fqh[kk] = ld8(reinterpret_cast<const bf16 *>(Qh + kq_off[kk]));
          fql[kk] = ld8(reinterpret_cast<const bf16 *>(Ql + kq_off[kk]));
        }
        if constexpr (ERASE || MODE == kModeRev) {
          fkh[kk] = ld8(reinterpret_cast<const bf16 *>(Kh + kq_off[kk]));
          fkl[kk] = ld8(reinterpret_cast<const bf16 *>(Kl + kq_off[kk]));
        }
      }
    };
    for (int it = 0; it < nchunks + 2; ++it) {
      const int s = it - 2;
      if constexpr (FUSED) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          og[e] = gated ? silu_gate(1.0f, bf16_bits_to_f32(og_next[e])) : 1.0f;
        const int c = s + 1;
        const bool valid = gated && c >= 0 && c < nchunks;
        const int n = valid ? min(KC, T - c * KC) : 1;
        const long orow = valid ? (tok0 + (long)c * KC * H) * DV : 0;
        const rsrc_t rg = make_rsrc32(out_gate + orow,
                                      valid ? 2u * ((unsigned)(n - 1) * H * DV + DV) : 0u);
#pragma unroll
        for (int e = 0; e < 4; ++e) og_next[e] = buf_ld_u16(rg, 2u * oel[e]);
      }
      if (MODE == kModeRev && s >= 0) {
        const typename SM::Der &d = *at_off(&sm.der[0], slot_off(s % NDER, (int)sizeof(typename SM::Der)));
        const int t1 = slot_off(s & 1, (int)sizeof(sm.Th[0]));
        const int exact = __builtin_amdgcn_readfirstlane(d.flag[0]);
        const int c = nchunks - 1 - s;   // chunks run last to first
        // X, the gradient of the state leaving chunk c
        float *xp = ws_a + ((long)chain * nchunks + c) * (DK * DV);
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_nontemporal_store(Sacc[mb][e], xp + ws_frag(DK / 16, col0 >> 4, mb, e, lg, lr));
        // Y1 = X times the factor the forward applied after its update
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb)
          Sacc[mb] = Sacc[mb] * *reinterpret_cast<const f32x4 *>(&d.egp[srow(mb, 0)]);
        split_state();
        // ---- dU = R^ Y1 + P^T dO (R^ rows in the K^ registers) ----
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KKD; ++kk) {
          a1 = mfma_bf16(fkh[kk], Sh[kk], a1);
          a1 = mfma_bf16(fkh[kk], Sl[kk], a1);
          a1 = mfma_bf16(fkl[kk], Sh[kk], a1);
        }
        // dO rows 4 lg + c of this lane's column (the v slot holds dO)
        const bf16x4 dov = ld_tr4(reinterpret_cast<const bf16 *>(
            reinterpret_cast<const char *>(&sm.V[0][0][0]) + slot_off(s % NVB, (int)sizeof(sm.V[0])) + v_off));
        // row lr of P^T is row lr of the stored tile; dO is exact bf16
        const bf16x8 pa = cat(*reinterpret_cast<const bf16x4 *>(&at_off(&sm.Ph[0][0], t1)[lr][4 * lg]),
                              *reinterpret_cast<const bf16x4 *>(&at_off(&sm.Pl[0][0], t1)[lr][4 * lg]));
        f32x4 du = mfma_bf16(pa, cat(dov, dov), a1);
        // ---- dY = T^T dU (without the erase term T = I) ----
        f32x4 y = du;
        if constexpr (ERASE) {
          bf16x4 duh, dul;
          split4(du, duh, dul);
          const bf16x8 ta = cat(*reinterpret_cast<const bf16x4 *>(&at_off(&sm.Th[0][0], t1)[lr][4 * lg]),
                                *reinterpret_cast<const bf16x4 *>(&at_off(&sm.Tl[0][0], t1)[lr][4 * lg]));
          y = f32x4{0.f, 0.f, 0.f, 0.f};
          y = mfma_bf16(ta, cat(duh, duh), y);
          y = mfma_bf16(ta, cat(dul, zero4), y);
        }
        float *yp = ws_b + ((long)chain * nchunks + c) * (KC * DV);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_nontemporal_store(y[e], yp + ws_frag(KC / 16, col0 >> 4, 0, e, lg, lr));
        // ---- X <- Y1 + Q^ ^T dO - K^ ^T diag(b) dY (the exact path: e^{g_last} o Y1) ----
        if (exact) {
#pragma unroll
          for (int mb = 0; mb < DK / 16; ++mb)
            Sacc[mb] = Sacc[mb] * *reinterpret_cast<const f32x4 *>(&d.egl[srow(mb, 0)]);
        }
        bf16x4 drh = zero4, drl = zero4;
        if constexpr (ERASE) {
          const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&d.beta[4 * lg]);
          split4(-(b4 * y), drh, drl);
        }
        const bf16x8 bq = cat(dov, dov), bk1 = cat(drh, drh), bk2 = cat(drl, zero4);
        const char *Qh = reinterpret_cast<const char *>(&d.Qh[0][0]);
        const char *Ql = reinterpret_cast<const char *>(&d.Ql[0][0]);
        const char *Kh = reinterpret_cast<const char *>(&d.Kh[0][0]);
        const char *Kl = reinterpret_cast<const char *>(&d.Kl[0][0]);
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb) {
          const int off = kt_off[mb >> 1] + 8 * (mb & 1);
          const bf16x8 aq = cat(ld_tr4(reinterpret_cast<const bf16 *>(Qh + off)),
                                ld_tr4(reinterpret_cast<const bf16 *>(Ql + off)));
          f32x4 acc = mfma_bf16(aq, bq, Sacc[mb]);
          if constexpr (ERASE) {
            const bf16x8 ak = cat(ld_tr4(reinterpret_cast<const bf16 *>(Kh + off)),
                                  ld_tr4(reinterpret_cast<const bf16 *>(Kl + off)));
            acc = mfma_bf16(ak, bk1, acc);
            acc = mfma_bf16(ak, bk2, acc);
          }
          Sacc[mb] = acc;
        }
      }
      if (MODE != kModeRev && s >= 0) {
        const typename SM::Der &d = *at_off(&sm.der[0], slot_off(s % NDER, (int)sizeof(typename SM::Der)));
        const int t1 = slot_off(s & 1, (int)sizeof(sm.Th[0]));   // T' and P slots (same size)
        const int exact = __builtin_amdgcn_readfirstlane(d.flag[0]);
        if constexpr (SAVE) {   // the state entering chunk s
          float *hp = ws_a + ((long)chain * nchunks + s) * (DK * DV);
#pragma unroll
          for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              __builtin_nontemporal_store(Sacc[mb][e], hp + ws_frag(DK / 16, col0 >> 4, mb, e, lg, lr));
        }
        // ---- K^ S, Q^ S (three products each), R = V - K^ S, U = T' R ----
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KKD; ++kk) {
          const bf16x8 qh = fqh[kk], ql = fql[kk];
          if constexpr (ERASE && !WANT_O) {
            const bf16x8 kh = fkh[kk], kl = fkl[kk];
            a1 = mfma_bf16(kh, Sh[kk], a1);
            a1 = mfma_bf16(kh, Sl[kk], a1);
            a1 = mfma_bf16(kl, Sh[kk], a1);
          } else if constexpr (ERASE) {
            const bf16x8 kh = fkh[kk], kl = fkl[kk];
            a1 = mfma_bf16(kh, Sh[kk], a1);
            a2 = mfma_bf16(qh, Sh[kk], a2);
            a1 = mfma_bf16(kh, Sl[kk], a1);
            a2 = mfma_bf16(qh, Sl[kk], a2);
            a1 = mfma_bf16(kl, Sh[kk], a1);
            a2 = mfma_bf16(ql, Sh[kk], a2);
          } else if constexpr (WANT_O) {
            a2 = mfma_bf16(qh, Sh[kk], a2);
            a2 = mfma_bf16(qh, Sl[kk], a2);
            a2 = mfma_bf16(ql, Sh[kk], a2);
          }
        }
        const bf16x4 vv = ld_tr4(reinterpret_cast<const bf16 *>(
            reinterpret_cast<const char *>(&sm.V[0][0][0]) + slot_off(s % NVB, (int)sizeof(sm.V[0])) + v_off));
        f32x4 rr;
        bf16x4 uh4, ul4;
        if constexpr (ERASE) {
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[e] = (float)vv[e] - a1[e];
          bf16x4 rh4, rl4;
          split4(rr, rh4, rl4);
          // [T'h | T'l] against [Rh ; Rh] and [Rl ; 0]: slots (half, c) <-> token 4 lg + c
          const bf16x8 ta = cat(ld_tr4(&at_off(&sm.Th[0][0], t1)[4 * lg + (lr >> 2)][4 * (lr & 3)]),
                                ld_tr4(&at_off(&sm.Tl[0][0], t1)[4 * lg + (lr >> 2)][4 * (lr & 3)]));
          f32x4 u = {0.f, 0.f, 0.f, 0.f};
          u = mfma_bf16(ta, cat(rh4, rh4), u);
          u = mfma_bf16(ta, cat(rl4, zero4), u);
          split4(u, uh4, ul4);
          rr = u;
        } else {
          // no erase term: U = diag(b) V
          const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&d.beta[4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[e] = b4[e] * (float)vv[e];
          split4(rr, uh4, ul4);
        }
        if constexpr (SAVE) {   // U of chunk s (rr holds it on both paths)
          float *up = ws_b + ((long)chain * nchunks + s) * (KC * DV);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_nontemporal_store(rr[e], up + ws_frag(KC / 16, col0 >> 4, 0, e, lg, lr));
        }

        // ---- O = Q^ S + P U ----
       if constexpr (WANT_O) {
        const int t0 = s * KC, n = min(KC, T - t0);
        const bf16x8 pa = cat(ld_tr4(&at_off(&sm.Ph[0][0], t1)[4 * lg + (lr >> 2)][4 * (lr & 3)]),
                              ld_tr4(&at_off(&sm.Pl[0][0], t1)[4 * lg + (lr >> 2)][4 * (lr & 3)]));
        f32x4 acc = a2;
        acc = mfma_bf16(pa, cat(uh4, uh4), acc);
        acc = mfma_bf16(pa, cat(ul4, zero4), acc);
        const long orow = (tok0 + (long)t0 * H) * DV;
        if constexpr (FUSED) acc = acc * og;
        // the chunk's rows: smaller than 4 GiB (the host checks the shape)
        const rsrc_t ro = make_rsrc32(o + orow, (unsigned)sizeof(OutT) * ((unsigned)(n - 1) * H * DV + DV));
        if (n == KC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) buf_st1(from_f32<OutT>(acc[e]), ro, ooff[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * lg + e < n) buf_st1(from_f32<OutT>(acc[e]), ro, ooff[e]);
        }
       }

        // ---- S <- Diag(e^{g_last}) (S + R^T U) (exact path: factor first) ----
        // The exact path's factor is a wave-uniform branch taken only by
        // such chunks; the factor after the update is 1 on that path (egp),
        // so the common path pays one multiply per element.  Sacc is last
        // written by a VALU multiply on every path, so no MFMA result is read
        // across the branch.
        if (exact) {
#pragma unroll
          for (int mb = 0; mb < DK / 16; ++mb)
            Sacc[mb] = Sacc[mb] * *reinterpret_cast<const f32x4 *>(&d.egl[srow(mb, 0)]);
        }
        const bf16x8 b1 = cat(uh4, uh4), b2 = cat(ul4, zero4);
        const char *Rh = reinterpret_cast<const char *>(&d.Rh[0][0]);
        const char *Rl = reinterpret_cast<const char *>(&d.Rl[0][0]);
#pragma unroll
        for (int mb = 0; mb < DK / 16; ++mb) {
          const f32x4 ep4 = *reinterpret_cast<const f32x4 *>(&d.egp[srow(mb, 0)]);
          const int off = kt_off[mb >> 1] + 8 * (mb & 1);
          const bf16x8 a = cat(ld_tr4(reinterpret_cast<const bf16 *>(Rh + off)),
                               ld_tr4(reinterpret_cast<const bf16 *>(Rl + off)));
          f32x4 sa = mfma_bf16(a, b1, Sacc[mb]);
          sa = mfma_bf16(a, b2, sa);
          Sacc[mb] = sa * ep4;
        }
        split_state();
      }
      if (xf && it + 2 < nchunks) xform_share(it + 2);
      load_kq(s + 1 < 0 ? 0 : s + 1);
      __syncthreads();
    }

    if (final_state) {
      float *SF = final_state + (long)chain * DK * DV;
#pragma unroll
      for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) SF[(long)srow(mb, e) * DV + col0 + lr] = Sacc[mb][e];
    }
    return;
  }

  // =======================================================================
  // prep waves
  // =======================================================================
  const int pw = wave - NSW;
  // v is loaded by a wave that only derives when there is one
  constexpr int PW_V = (kda_npw<DVS>() == 6) ? 5 : 2;

  // 16x16 tile L R^T of derived operands (hi/lo both sides, three
  // independent MFMA chains); lane holds rows 4 lg + e of column lr
  auto tile = [&](const bf16 *Lh, const bf16 *Ll, const bf16 *Rh, const bf16 *Rl) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, a1 = acc, a2 = acc;
#pragma unroll
    for (int kk = 0; kk < KKD; ++kk) {
      const int off = kq_off[kk] / 2;
      const bf16x8 ah = ld8(Lh + off), al = ld8(Ll + off);
      const bf16x8 bh = ld8(Rh + off), bl = ld8(Rl + off);
      acc = mfma_bf16(ah, bh, acc);
      a1 = mfma_bf16(ah, bl, a1);
      a2 = mfma_bf16(al, bh, a2);
    }
    return acc + a1 + a2;
  };

  if (ERASE && pw == 3) {
    // ---- Gram and solve of chunk it-1: T' = (I + A)^{-1} diag(b) ----
    __syncthreads();
    if (xf && xpart) {
      if (nchunks > 0) xform_share(0);
      if (nchunks > 1) xform_share(1);
    }
    __syncthreads();
    __syncthreads();
    for (int it = 0; it < nchunks + 2; ++it) {
      const int j = it - 1;
      if (ERASE && j >= 0 && j < nchunks) {   // no solve without the erase term
        const typename SM::Der &d = *at_off(&sm.der[0], slot_off(j % NDER, (int)sizeof(typename SM::Der)));
        const int t1 = slot_off(j & 1, (int)sizeof(sm.Th[0]));
        const int exact = __builtin_amdgcn_readfirstlane(d.flag[0]);
        const float(*src)[SM::LDX] = sm.At;
        if (!exact) {
          const f32x4 acc = tile(&d.Kh[0][0], &d.Kl[0][0], &d.Rh[0][0], &d.Rl[0][0]);
          const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&d.beta[4 * lg]);
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = (lr < 4 * lg + e) ? -b4[e] * acc[e] : 0.0f;
          *reinterpret_cast<f32x4 *>(&sm.At[lr][4 * lg]) = val;   // [s][r] = -A[r][s]
          wave_lds_sync();
        } else {
          src = at_off(&sm.xA[0][0], slot_off(j & 1, (int)sizeof(sm.xA[0])));
        }
        // right-looking forward substitution, lane = column col (each
        // 16-lane row holds all columns); lane col keeps column col of -A
        // and step s takes column s from lane s by a row broadcast folded
        // into the FMA
        const int col = lr;
        float na[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 t = *reinterpret_cast<const f32x4 *>(&src[col][4 * q4]);
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
        // T'^T[col][r] = T[r][col] b_col, hi/lo (lanes 16..63 hold duplicates);
        // the reverse pass takes T^T itself (b_col = 1)
        if (lane < 16) {
          const float bcol = MODE == kModeRev ? 1.0f : d.beta[col];
          unsigned h8[2][4], l8[2][4];
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            split2(x[r] * bcol, x[r + 1] * bcol, h8[r / 8][(r % 8) / 2], l8[r / 8][(r % 8) / 2]);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            *reinterpret_cast<u32x4 *>(&at_off(&sm.Th[0][0], t1)[col][8 * hf]) = u32x4{h8[hf][0], h8[hf][1], h8[hf][2], h8[hf][3]};
            *reinterpret_cast<u32x4 *>(&at_off(&sm.Tl[0][0], t1)[col][8 * hf]) = u32x4{l8[hf][0], l8[hf][1], l8[hf][2], l8[hf][3]};
          }
        }
      }
      if (xf && xpart && it + 2 < nchunks) xform_share(it + 2);
      __syncthreads();
    }
    return;
  }

  // ---- prep waves 0..2: LDS DMA, log-decay sums, derivation, scores ----
  // DMA shares: wave 0 log a (+ b), wave 1 q and k, wave 2 v.  Instruction i
  // of a tile fills LDS bytes 1024 i .. +1023 of it.
  constexpr int NQI = KC * QRB / 1024;         // per q or k tile
  constexpr int NLI = KC * 4 * DK / 1024;      // log a tile
  constexpr int NVI = KC * VRB / 1024;         // v tile
  constexpr int N0 = NLI + 1, N1 = 2 * NQI, N2 = NVI;
  constexpr int NI = (NLI > NQI) ? NLI : NQI;
  unsigned voff[NI];
  if (pw == 0) {
    constexpr int BPR = 4 * DK / 16, RPI = 1024 / (4 * DK);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + lane / BPR;
      voff[i] = (unsigned)row * (4u * H * DK) + 16u * (lane % BPR);
    }
  } else if (pw == 1) {
    constexpr int BPR = QRB / 16, RPI = 1024 / QRB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + lane / BPR;
      voff[i] = (unsigned)row * (2u * H * DK) + 16u * (lane % BPR);
    }
  } else {
    constexpr int BPR = VRB / 16, RPI = 1024 / VRB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + lane / BPR, sb = lane % BPR;
      voff[i] = (unsigned)row * (2u * H * DV) + (unsigned)(2 * slice * DVS + 16 * (sb ^ swz_v<VB>(row)));
    }
  }
  const unsigned soff = (unsigned)(lane * H * 4);   // b of token `lane`

  // q, k, log a and b of chunk j (waves 0 and 1)
  auto issue_raw = [&](int j) {
    typename SM::Raw &dst = sm.raw[j % NRAW];
    const int n = min(KC, T - chunk_of(j) * KC);
    const long row0 = tok0 + (long)chunk_of(j) * KC * H;
    if (pw == 0) {
      const u32x4 rl = rsrc_words(log_alpha + row0 * DK, 4u * ((unsigned)(n - 1) * H * DK + DK));
      const unsigned ll = lds_addr(&dst.G[0][0]);
#pragma unroll
      for (int i = 0; i < NLI; ++i) lds_dma16(rl, voff[i], ll + 1024 * i);
      lds_dma4(rsrc_words(beta + row0, 4u * ((unsigned)(n - 1) * H + 1)), soff, lds_addr(&dst.beta[0]));
    } else {
      const u32x4 rq = rsrc_words(q + row0 * DK, 2u * ((unsigned)(n - 1) * H * DK + DK));
      const u32x4 rk = rsrc_words(k + row0 * DK, 2u * ((unsigned)(n - 1) * H * DK + DK));
      const unsigned lq = lds_addr(&dst.Q[0][0]), lk = lds_addr(&dst.K[0][0]);
#pragma unroll
      for (int i = 0; i < NQI; ++i) lds_dma16(rq, voff[i], lq + 1024 * i);
#pragma unroll
      for (int i = 0; i < NQI; ++i) lds_dma16(rk, voff[i], lk + 1024 * i);
    }
  };
  // v of chunk j, this slice's columns (wave 2)
  auto issue_v = [&](int j) {
    const int n = min(KC, T - chunk_of(j) * KC);
    const long row0 = tok0 + (long)chunk_of(j) * KC * H;
    const u32x4 rv = rsrc_words(v + row0 * DV, 2u * ((unsigned)(n - 1) * H * DV + DV));
    const unsigned lv = lds_addr(&sm.V[j % NVB][0][0]);
#pragma unroll
    for (int i = 0; i < NVI; ++i) lds_dma16(rv, voff[i], lv + 1024 * i);
  };

  // in-chunk cumulative log decay of chunk j in base 2, in place (wave 1):
  // lane = a channel pair; padded tokens read log a = 0; flags a chunk
  // whose factored operands could leave the floating-point range
  auto gsum = [&](int j) {
    typename SM::Raw &rw = *at_off(&sm.raw[0], slot_off(j % NRAW, (int)sizeof(typename SM::Raw)));
    constexpr int NCP = DK / 2;
    const int c0 = 2 * (lane % NCP);
    const float lscale = xf ? 1.0f : kLog2e;   // transformed values are log2 a already
    f32x2 acc = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      const f32x2 x = *reinterpret_cast<const f32x2 *>(&rw.G[r][c0]);
      acc = f32x2{fmaf(x[0], lscale, acc[0]), fmaf(x[1], lscale, acc[1])};
      if (lane < NCP) *reinterpret_cast<f32x2 *>(&rw.G[r][c0]) = acc;
    }
    const unsigned long long bad = __ballot(acc[0] < -kMaxSpan2 || acc[1] < -kMaxSpan2);
    if (lane == 0) rw.flag[0] = bad != 0ull;
  };
  // the fused L2 norms are shared by NGW waves
  constexpr int NGW = (kda_npw<DVS>() == 6) ? 4 : 2;
  // index of this wave among the NGW norm waves, or -1
  const int gsum_idx = (kda_npw<DVS>() == 6) ? (pw < 2 ? pw : (pw >= 4 ? pw - 2 : -1))
                                             : (pw < 2 ? pw : -1);
  auto sums = [&](int j) {
    if (pw == 1) gsum(j);
  };

  // fused L2 normalisation of chunk j: 1/|q_r| and 1/|k_r|, shared by the
  // NGW summing waves: wave gi takes 32 / NGW of the (matrix, row) pairs,
  // LPR lanes to a row, and sums across those lanes
  constexpr int NRM_R = 2 * KC / NGW, LPR = 64 / NRM_R, CPL = DK / LPR;
  static_assert(NRM_R * LPR == 64 && CPL % 8 == 0, "shared norms");
  auto norms = [&](int j, int gi) {
    typename SM::Raw &rw = *at_off(&sm.raw[0], slot_off(j % NRAW, (int)sizeof(typename SM::Raw)));
    const int mr = gi * NRM_R + lane / LPR;          // (matrix, row) pair
    const int m = mr / KC, r = mr % KC, part = lane % LPR;
    const char *X = reinterpret_cast<const char *>(m ? &rw.K[r][0] : &rw.Q[r][0]) + 2 * CPL * part;
    float ss4[4] = {0.f, 0.f, 0.f, 0.f};   // four independent sums: short chains
#pragma unroll
    for (int b = 0; b < CPL / 8; ++b) {
      const u32x4 w4 = *reinterpret_cast<const u32x4 *>(X + 16 * b);
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
    // sum over the LPR lanes of the row with DPP moves (no LDS round trip):
    // within quads, then the upper quad into the lower one, which holds the
    // writing lane (part 0)
    static_assert(LPR == 4 || LPR == 8, "norm lanes");
    auto dpp = [](float x, auto ctrl) {
      return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
          0, __builtin_bit_cast(int, x), decltype(ctrl)::value, 0xF, 0xF, true));
    };
    ss += dpp(ss, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
    ss += dpp(ss, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
    if constexpr (LPR == 8) ss += dpp(ss, std::integral_constant<int, 0x104>{});   // row_shl:4
    if (part == 0) rw.nrm[m][r] = rsqrtf(ss + kL2Eps);
  };

  // derived operands of chunk j: a work row is 64 lanes = (channel pair,
  // token), shared by every prep wave but the solver's; wave 0 takes the
  // most (it only issues DMA besides), wave 2 the fewest (it forms the
  // scores).  Boundaries in 16ths of the NRW rows: 4 waves 0|7|12|16, 6
  // waves 0|4|7|9|13|16 (waves 0, 1, 2, 4, 5).  Without the erase term
  // there is no solve and wave 3 derives too, while wave 1 (q, k DMA and the
  // decay sums, then the critical role) derives less: 0|5|8|12|16 and
  // 0|2|3|5|9|13|16 (measured on the KDA shape: 2,904 -> 2,528 cycles per
  // iteration).
  constexpr int NPW = kda_npw<DVS>();
  constexpr int NDW = ERASE ? NPW - 1 : NPW;   // deriving waves
  constexpr int NCP = DK / 2, TPR = 64 / NCP, NRW = KC / TPR;
  const int dw = (ERASE && pw >= 3) ? pw - 1 : pw;   // index among the deriving waves
  auto row_bound = [&](int w) {
    if constexpr (NPW == 6) {
      constexpr int b[6] = {0, 4, 7, 9, 13, 16};
      constexpr int bn[7] = {0, 2, 3, 5, 9, 13, 16};
      return (ERASE ? b[w] : bn[w]) * NRW / 16;
    } else {
      constexpr int b[4] = {0, 7, 12, 16};
      constexpr int bn[5] = {0, 5, 8, 12, 16};
      return (ERASE ? b[w] : bn[w]) * NRW / 16;
    }
  };
  auto derive = [&](int j) {
    const typename SM::Raw &rw = *at_off(&sm.raw[0], slot_off(j % NRAW, (int)sizeof(typename SM::Raw)));
    // the derived slot's LDS address, array base included, as an opaque
    // wave-uniform value: the row loop's six stores then differ by constant
    // offsets below 64 KiB, which the store instructions carry (with the
    // base left constant the offsets exceed that field)
    int dso = __builtin_amdgcn_readfirstlane((j % NDER) * (int)sizeof(typename SM::Der) + (int)offsetof(SM, der));
    asm volatile("" : "+s"(dso));   // emits nothing; hides the constant part
    typename SM::Der &d = *reinterpret_cast<typename SM::Der *>(reinterpret_cast<char *>(&sm) + dso);
    const int exact = __builtin_amdgcn_readfirstlane(rw.flag[0]);
    const int cp = lane % NCP, c0 = 2 * cp;
    const f32x2 gl = *reinterpret_cast<const f32x2 *>(&rw.G[KC - 1][c0]);
    if (pw == 0) {
      if (lane < NCP) {
        const f32x2 eg = {__builtin_amdgcn_exp2f(gl[0]), __builtin_amdgcn_exp2f(gl[1])};
        *reinterpret_cast<f32x2 *>(&d.egl[c0]) = eg;
        *reinterpret_cast<f32x2 *>(&d.egp[c0]) = exact ? f32x2{1.0f, 1.0f} : eg;
      }
      if (lane < KC) d.beta[lane] = (lane < min(KC, T - chunk_of(j) * KC)) ? fused_beta(rw.beta[lane], fuse) : 0.0f;
      if (lane == 0) d.flag[0] = exact;
    }
    const int rb0 = row_bound(dw), rb1 = row_bound(dw + 1);
    const bool l2f = (fuse & kFuseL2) != 0;
    const int coff = 2 * (c0 & 7);                 // byte offset inside the 16-byte block
    auto put = [&](bf16 (*hi)[DK], bf16 (*lo)[DK], int r, float x0, float x1) {
      unsigned h, l;
      split2(x0, x1, h, l);
      const int off = qk_at(r, c0 >> 3) + coff;
      *reinterpret_cast<unsigned *>(reinterpret_cast<char *>(&hi[0][0]) + off) = h;
      *reinterpret_cast<unsigned *>(reinterpret_cast<char *>(&lo[0][0]) + off) = l;
    };
    // R^ = K o e^{-G}, on the exact path K o e^{g_last - G}: one row loop
    // per path (exact is wave-uniform), so the common one has no shift
    auto rows = [&](auto exact_path) {
      constexpr bool EX = decltype(exact_path)::value;
      for (int w = rb0; w < rb1; ++w) {
        const int r = w * TPR + lane / NCP;
        const f32x2 g = *reinterpret_cast<const f32x2 *>(&rw.G[r][c0]);
        const unsigned kb = *reinterpret_cast<const unsigned *>(&rw.K[r][c0]);
        const unsigned qb = *reinterpret_cast<const unsigned *>(&rw.Q[r][c0]);
        const float k0 = __builtin_bit_cast(float, kb << 16), k1 = __builtin_bit_cast(float, kb & 0xffff0000u);
        const float q0 = __builtin_bit_cast(float, qb << 16), q1 = __builtin_bit_cast(float, qb & 0xffff0000u);
        // the fused norms are read whether or not they were formed and
        // picked by a select (no branch in the row loop)
        const float nq = rw.nrm[0][r], nk = rw.nrm[1][r];
        const float rq = l2f ? nq : 1.0f, rk = l2f ? nk : 1.0f;
        const float x0 = __builtin_amdgcn_exp2f(g[0]), x1 = __builtin_amdgcn_exp2f(g[1]);
        const float f0 = __builtin_amdgcn_exp2f(EX ? gl[0] - g[0] : -g[0]) * rk;
        const float f1 = __builtin_amdgcn_exp2f(EX ? gl[1] - g[1] : -g[1]) * rk;
        if constexpr (ERASE) put(d.Kh, d.Kl, r, k0 * (x0 * rk), k1 * (x1 * rk));   // K^ feeds only K^ S and A
        if constexpr (WANT_P) put(d.Qh, d.Ql, r, q0 * (x0 * rq), q1 * (x1 * rq));
        put(d.Rh, d.Rl, r, k0 * f0, k1 * f1);
      }
    };
    if (exact) rows(std::true_type{});
    else rows(std::false_type{});
    if (exact) {
      // exact Gram and scores: every decay formed directly; entry (r, s)
      // of both tiles per item, 256 items over the deriving waves
      for (int idx = 64 * dw + lane; idx < KC * KC; idx += 64 * NDW) {
        const int r = idx / KC, s = idx % KC;
        float sa = 0.0f, sp = 0.0f;
        if (s <= r) {
          for (int c = 0; c < DK; ++c) {
            const float ks = (float)rw.K[s][c] * __builtin_amdgcn_exp2f(rw.G[r][c] - rw.G[s][c]);
            sa += (float)rw.K[r][c] * ks;
            sp += (float)rw.Q[r][c] * ks;
          }
        }
        if (fuse & kFuseL2) {
          sa *= rw.nrm[1][r] * rw.nrm[1][s];
          sp *= rw.nrm[0][r] * rw.nrm[1][s];
        }
        const float br = (r < min(KC, T - chunk_of(j) * KC)) ? fused_beta(rw.beta[r], fuse) : 0.0f;
        if constexpr (ERASE) sm.xA[j & 1][s][r] = (s < r) ? -br * sa : 0.0f;
        sm.xP[j & 1][s][r] = sp;
      }
    }
  };

  // P of chunk j (lower incl.), split hi/lo, transposed (wave 2)
  auto scores = [&](int j) {
    const typename SM::Der &d = *at_off(&sm.der[0], slot_off(j % NDER, (int)sizeof(typename SM::Der)));
    const int t1 = slot_off(j & 1, (int)sizeof(sm.Ph[0]));
    const int exact = __builtin_amdgcn_readfirstlane(d.flag[0]);
    f32x4 val;
    if (!exact) {
      const f32x4 acc = tile(&d.Qh[0][0], &d.Ql[0][0], &d.Rh[0][0], &d.Rl[0][0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = (lr <= 4 * lg + e) ? acc[e] : 0.0f;
    } else {
      val = *reinterpret_cast<const f32x4 *>(&sm.xP[j & 1][lr][4 * lg]);
    }
    bf16x4 h4, l4;
    split4(val, h4, l4);
    *reinterpret_cast<bf16x4 *>(&at_off(&sm.Ph[0][0], t1)[lr][4 * lg]) = h4;
    *reinterpret_cast<bf16x4 *>(&at_off(&sm.Pl[0][0], t1)[lr][4 * lg]) = l4;
  };

  auto wait_own = [&](bool newer_issued) {
    if (newer_issued) {
      if (pw == 0) wait_vmcnt<N0>();
      else if (pw == 1) wait_vmcnt<N1>();
      else wait_vmcnt<N2>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // prologue: raw chunks 0..2 in flight, 0 and 1 landed (all three with a
  // fused decay transform, whose participants then transform 0 and 1),
  // chunk 0 summed
  if (pw < 2) {
    if (nchunks > 0) issue_raw(0);
    if (nchunks > 1) issue_raw(1);
    if (nchunks > 2) issue_raw(2);
    wait_own(!xf && nchunks > 2);
  }
  const bool l2 = (fuse & kFuseL2) && gsum_idx >= 0;
  __syncthreads();
  if (xf && xpart) {   // the transform of chunks 0 and 1 (fused decay)
    if (nchunks > 0) xform_share(0);
    if (nchunks > 1) xform_share(1);
  }
  __syncthreads();
  if (nchunks > 0) sums(0);
  if (l2 && nchunks > 0) norms(0, gsum_idx);
  __syncthreads();

  for (int it = 0; it < nchunks + 2; ++it) {
    if (pw < 2) {
      const bool more = it + 3 < nchunks;
      if (more) issue_raw(it + 3);
      if (it + 1 < nchunks) sums(it + 1);
      if (l2 && it + 1 < nchunks) norms(it + 1, gsum_idx);
      if (it < nchunks) derive(it);
      wait_own(more && !xf);
    } else {
      const bool more = it < nchunks;
      if (pw == PW_V && more) issue_v(it);
      if (l2 && it + 1 < nchunks) norms(it + 1, gsum_idx);
      if (WANT_P && pw == 2 && it >= 1 && it - 1 < nchunks) scores(it - 1);
      if (it < nchunks) derive(it);
      if (xf && xpart && it + 2 < nchunks) xform_share(it + 2);
      if (pw == PW_V) wait_own(more);
    }
    __syncthreads();
  }
}

template <int DK, int DVS, typename OutT, bool ERASE, bool FUSED>
hipError_t launch_kda_fused(const ChunkArgs &a) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + kda_npw<DVS>()));
  hipLaunchKernelGGL((chunk_fwd_kda_kernel<DK, DVS, OutT, ERASE, FUSED, kModeFwd>), grid, block, 0,
                     a.stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta,
                     a.log_alpha, a.initial_state, (OutT *)a.o, a.final_state, a.B, a.T, a.H,
                     a.fuse, (const bf16 *)a.out_gate, nullptr, nullptr);
  return hipGetLastError();
}

// the forward that also stores h and U per chunk (the recompute pass's
// stores) at one tile configuration
template <int DK, int DVS, typename OutT, bool ERASE>
hipError_t launch_kda_save(const ChunkArgs &a, float *ws_h, float *ws_u) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + kda_npw<DVS>()));
  hipLaunchKernelGGL((chunk_fwd_kda_kernel<DK, DVS, OutT, ERASE, false, kModeFwdSave>), grid, block,
                     0, a.stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta,
                     a.log_alpha, a.initial_state, (OutT *)a.o, a.final_state, a.B, a.T, a.H, 0,
                     nullptr, ws_h, ws_u);
  return hipGetLastError();
}

template <int DK, int DVS>
hipError_t kda_save_by_out(const ChunkArgs &a, float *ws_h, float *ws_u) {
  if (a.erase)
    return a.out_bf16 ? launch_kda_save<DK, DVS, bf16, true>(a, ws_h, ws_u)
                      : launch_kda_save<DK, DVS, float, true>(a, ws_h, ws_u);
  return a.out_bf16 ? launch_kda_save<DK, DVS, bf16, false>(a, ws_h, ws_u)
                    : launch_kda_save<DK, DVS, float, false>(a, ws_h, ws_u);
}

// the backward's two sequential passes at one tile configuration (the first
// skipped when a training forward has stored its results)
template <int DK, int DVS, bool ERASE>
hipError_t launch_kda_passes(const BwdArgs &a) {
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(64 * (DVS / 16 + kda_npw<DVS>()));
  if (!a.saved) {
    hipLaunchKernelGGL((chunk_fwd_kda_kernel<DK, DVS, float, ERASE, false, kModeRec>), grid, block,
                       0, a.stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                       a.beta, a.log_alpha, a.initial_state, nullptr, nullptr, a.B, a.T, a.H, 0,
                       nullptr, a.ws_h, a.ws_u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_fwd_kda_kernel<DK, DVS, float, ERASE, false, kModeRev>), grid, block, 0,
                     a.stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.d_o, a.beta,
                     a.log_alpha, a.d_final_state, nullptr, a.d_initial_state, a.B, a.T, a.H, 0,
                     nullptr, a.ws_dh, a.ws_dy);
  return hipGetLastError();
}

template <int DK, int DVS>
hipError_t kda_passes_by_erase(const BwdArgs &a) {
  return a.erase ? launch_kda_passes<DK, DVS, true>(a) : launch_kda_passes<DK, DVS, false>(a);
}

template <int DK, int DVS, typename OutT, bool ERASE>
hipError_t launch_kda(const ChunkArgs &a) {
  if (a.fuse != 0 || a.out_gate != nullptr) return launch_kda_fused<DK, DVS, OutT, ERASE, true>(a);
  return launch_kda_fused<DK, DVS, OutT, ERASE, false>(a);
}

template <int DK, int DVS>
hipError_t kda_by_out(const ChunkArgs &a) {
  if (a.erase) return a.out_bf16 ? launch_kda<DK, DVS, bf16, true>(a) : launch_kda<DK, DVS, float, true>(a);
  return a.out_bf16 ? launch_kda<DK, DVS, bf16, false>(a) : launch_kda<DK, DVS, float, false>(a);
}

}  // namespace

bool chunk_fwd_kda_supported(const ChunkArgs &a) {
  // the chunk-sized buffer descriptors of the log decays (the widest rows)
  // are 32-bit
  return a.in_bf16 && (a.D == 128 || a.D == 64) && a.gate == kGateChannel &&
         4.0 * ((double)(KC - 1) * a.H * a.D + a.D) < 4294967295.0;
}

hipError_t launch_chunk_bwd_kda_passes(const BwdArgs &a) {
  static_assert(KC == kBwdChunkKda, "the workspace holds this kernel's chunks");
  // the forward's launch shapes
  const long chains = (long)a.B * a.H;
  if (a.D == 128) {
    if (chains * 2 >= 256) return kda_passes_by_erase<128, 64>(a);
    return kda_passes_by_erase<128, 32>(a);
  }
  if (chains >= 256) return kda_passes_by_erase<64, 64>(a);
  return kda_passes_by_erase<64, 32>(a);
}

hipError_t launch_chunk_fwd_kda_save(const ChunkArgs &a, float *ws_h, float *ws_u) {
  const long chains = (long)a.B * a.H;   // the forward's launch shapes
  if (a.D == 128) {
    if (chains * 2 >= 256) return kda_save_by_out<128, 64>(a, ws_h, ws_u);
    return kda_save_by_out<128, 32>(a, ws_h, ws_u);
  }
  if (chains >= 256) return kda_save_by_out<64, 64>(a, ws_h, ws_u);
  return kda_save_by_out<64, 32>(a, ws_h, ws_u);
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
