// Chunk-parallel gradients of the chunkwise KDA forward (per-channel decay;
// bf16 q/k/v/dO, fp32 state, MFMA, gfx950; dq, dk, dv written as fp32 or as
// bf16 rounded to nearest even, template argument GT).
//
// The forward per chunk of C = 16 tokens (page "NLP——线性注意力相关总结",
// section "Kimi Delta Attention (KDA)"; xhh.club digest "Transformer 入坑笔记
// （五）", KDA Q&A), with entering state h, G the in-chunk cumulative log
// decay per (token, channel) and g_last its last row:
//
//   K^ = K o e^G,  Q^ = Q o e^G,  R^ = K o e^{-G},  Kb = K o e^{g_last - G}
//   M = strict_lower(K^ R^^T),  A = diag(b) M,  T = (I + A)^{-1}
//   P = lower_incl(Q^ R^^T)
//   R = V - K^ h,  U = T diag(b) R
//   O = Q^ h + P U,  h' = Diag(e^{g_last}) h + Kb^T U
//
// is differentiated in reverse.  The KDA chunk kernel's recompute and reverse
// passes leave per chunk h, U, dh (the gradient of h') and dY = T^T dU with
// dU = Kb dh + P^T dO; given those, each chunk's gradients are independent:
//
//   dV = diag(b) dY,  dA = -strict_lower(dY U^T),  dM = diag(b) dA
//   dP = lower_incl(dO U^T)
//   db_r = dY_r . v_r - K^_r . (dY h^T)_r + sum_s dA_rs M_rs
//   dQ   = e^G o (dO h^T + dP R^)
//   dK^  = -diag(b) dY h^T + dM R^,   dR^ = dM^T K^ + dP^T Q^,  dKb = U dh^T
//   dK   = e^G o dK^ + e^{-G} o dR^ + e^{g_last - G} o dKb
//   dG   = Q o dQ + K o (e^G o dK^ - e^{-G} o dR^ - e^{g_last - G} o dKb)
//   dG_last += colsum(K o e^{g_last - G} o dKb) + e^{g_last} o rowsum(h o dh)
//   dlog a_t = sum_{r >= t} dG_r            (G is a within-chunk cumsum)
//
// A product with R^ times e^G, or with K^ or Q^ times e^{-G}, carries the
// decay e^{G_r - G_s} of each channel; it stays in range while every
// channel's in-chunk log decay is above -64.  A chunk below that (a near-hard
// reset) forms P, M and the three decayed products with every e^{G_rc - G_sc}
// directly in fp32.  Without the erase term (GLA's per-channel decay) T = I
// and R = V: A, M and the dY h^T terms vanish and db_r = dY_r . v_r
// (template flag ERASE).
//
// One workgroup of four waves per (chain, chunk).  q, k and dO are exact
// bf16 and enter MFMAs unsplit; every derived operand (h, dh, U, dY, K^, Q^,
// R^ and the n x n gradient matrices) is split into bf16 hi + lo, so products
// carry ~16 significant bits with fp32 accumulation.
#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace gdr {
namespace {

constexpr int C = kBwdChunkKda;   // tokens per chunk (the KDA kernel's)
constexpr int NW = 4;             // waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;
// the per-channel in-chunk log-decay bound of the factored products, base 2
constexpr float kMaxSpan2 = 64.0f * kLog2e;

template <int DK>
struct __align__(16) KdaBwdSmem {
  static constexpr int LDB = DK + 8;   // bf16 row stride: 16-byte row reads of 16 rows hit
                                       // distinct banks
  static constexpr int LDG = DK + 4;   // fp32 row stride of G
  static constexpr int LDN = C + 1;    // fp32 [C][C]
  static constexpr int LDX = C + 8;    // bf16 [C][C] hi / lo
  bf16 Q[C][LDB], K[C][LDB], D[C][LDB];                    // q, k, dO
  bf16 Kh[C][LDB], Kl[C][LDB], Qh[C][LDB], Ql[C][LDB];     // K^, Q^
  bf16 Rh[C][LDB], Rl[C][LDB];                             // R^
  bf16 Uh[C][LDB], Ul[C][LDB], Yh[C][LDB], Yl[C][LDB];     // U, dY split once
  float G[C][LDG];     // log a, then G in base 2, then dG (natural log units)
  float P[C][LDN], M[C][LDN];
  float dA[C][LDN];    // dA, then dM
  float dP[C][LDN];
  bf16 dPh[C][LDX], dPl[C][LDX], dMh[C][LDX], dMl[C][LDX];       // rows
  bf16 dPTh[C][LDX], dPTl[C][LDX], dMTh[C][LDX], dMTl[C][LDX];   // transposed
  float beta[C], dba[C], dbm[C];   // b; sum_v dY V; sum_s dA M
  float dbp[NW][C];                // per-wave K^_r . (dY h^T)_r
  float dgl[DK];                   // the g_last terms of dG, per channel
};

__device__ __forceinline__ void split1(float x, bf16 &h, bf16 &l) {
  h = (bf16)x;
  l = (bf16)(x - (float)h);
}

template <int DK, bool ERASE, typename GT>
__global__ void __launch_bounds__(64 * NW, 2)
chunk_bwd_kda_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                     const bf16 *__restrict__ v, const float *__restrict__ beta,
                     const float *__restrict__ log_alpha, const bf16 *__restrict__ d_o,
                     const float *__restrict__ ws_h, const float *__restrict__ ws_u,
                     const float *__restrict__ ws_dh, const float *__restrict__ ws_dy,
                     GT *__restrict__ dq, GT *__restrict__ dk, GT *__restrict__ dv,
                     float *__restrict__ dbeta, float *__restrict__ dlog_alpha, int B, int T,
                     int H) {
  constexpr int DV = DK;
  constexpr int NTW = DK / 64;         // 16-channel tiles per wave
  constexpr int KKV = DV / 32;         // 32-deep k steps over dv
  constexpr int KKD = DK / 32;         // and over dk
  using SM = KdaBwdSmem<DK>;
  static_assert(sizeof(SM) <= 80 * 1024, "two workgroups per CU");
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nchunks = (T + C - 1) / C;
  const int chain = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int bb = chain / H, hh = chain % H;
  const int n = min(C, T - c * C);                           // valid rows of this chunk
  const long row0 = ((long)bb * T + (long)c * C) * H + hh;   // token row of the chunk's row 0
  auto trow = [&](int r) { return row0 + (long)r * H; };
  const long wsS = ((long)chain * nchunks + c) * (DK * DV);  // h, dh of this chunk
  const long wsR = ((long)chain * nchunks + c) * (C * DV);   // U, dY of this chunk
  const bf16x4 zero4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};

  // ---- P0: inputs into LDS; dV = b dY; sum_v dY V ----
  {
    constexpr int TPR = DV / 8;        // threads per row, 8 columns each
    if (tid < C * TPR) {
      const int r = tid / TPR, c8 = 8 * (tid % TPR);
      const bool ok = r < n;
      u32x4 xq = {0u, 0u, 0u, 0u}, xk = xq, xd = xq, xv = xq;
      f32x4 la0 = {0.f, 0.f, 0.f, 0.f}, la1 = la0;
      if (ok) {   // rows past the sequence's end read as zero (log a = 0)
        const long off = trow(r) * DK + c8;
        xq = *reinterpret_cast<const u32x4 *>(q + off);
        xk = *reinterpret_cast<const u32x4 *>(k + off);
        xd = *reinterpret_cast<const u32x4 *>(d_o + trow(r) * DV + c8);
        xv = *reinterpret_cast<const u32x4 *>(v + trow(r) * DV + c8);
        la0 = *reinterpret_cast<const f32x4 *>(log_alpha + off);
        la1 = *reinterpret_cast<const f32x4 *>(log_alpha + off + 4);
      }
      const long o = wsR + ws_tile_off(C, r, c8);   // 8 contiguous
      const f32x4 u0 = *reinterpret_cast<const f32x4 *>(ws_u + o);
      const f32x4 u1 = *reinterpret_cast<const f32x4 *>(ws_u + o + 4);
      const f32x4 y0 = *reinterpret_cast<const f32x4 *>(ws_dy + o);
      const f32x4 y1 = *reinterpret_cast<const f32x4 *>(ws_dy + o + 4);
      const float b = ok ? beta[trow(r)] : 0.0f;
      *reinterpret_cast<u32x4 *>(&sm.Q[r][c8]) = xq;
      *reinterpret_cast<u32x4 *>(&sm.K[r][c8]) = xk;
      *reinterpret_cast<u32x4 *>(&sm.D[r][c8]) = xd;
      *reinterpret_cast<f32x4 *>(&sm.G[r][c8]) = la0;
      *reinterpret_cast<f32x4 *>(&sm.G[r][c8 + 4]) = la1;
      bf16x4 h0, l0, h1, l1;
      split4(u0, h0, l0);
      split4(u1, h1, l1);
      *reinterpret_cast<bf16x8 *>(&sm.Uh[r][c8]) = cat(h0, h1);
      *reinterpret_cast<bf16x8 *>(&sm.Ul[r][c8]) = cat(l0, l1);
      split4(y0, h0, l0);
      split4(y1, h1, l1);
      *reinterpret_cast<bf16x8 *>(&sm.Yh[r][c8]) = cat(h0, h1);
      *reinterpret_cast<bf16x8 *>(&sm.Yl[r][c8]) = cat(l0, l1);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, xv);
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) dot += y0[j] * (float)vb[j] + y1[j] * (float)vb[4 + j];
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) dot += __shfl_xor(dot, m);
      if (tid % TPR == 0) {
        sm.dba[r] = dot;
        sm.beta[r] = b;
      }
      if (ok) {
        st4(dv + trow(r) * DV + c8, y0 * b);
        st4(dv + trow(r) * DV + c8 + 4, y1 * b);
      }
    }
  }
  __syncthreads();

  // ---- P0b: G (base 2) per channel; the chunk's range flag; K^, Q^, R^ ----
  int exact;
  {
    constexpr int NPART = 64 * NW / DK;   // threads per channel
    constexpr int RP = C / NPART;         // rows each derives
    const int ch = tid % DK, part = tid / DK;
    float g[C];
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      acc = fmaf(sm.G[r][ch], kLog2e, acc);
      g[r] = acc;
    }
    // every thread has read its column's log a before any G is written
    exact = __syncthreads_or(acc < -kMaxSpan2);
#pragma unroll
    for (int r = 0; r < C; ++r) {
      if (r / RP != part) continue;
      sm.G[r][ch] = g[r];
      const float kv = (float)sm.K[r][ch], qv = (float)sm.Q[r][ch];
      const float eg = __builtin_amdgcn_exp2f(g[r]);
      // R^ is not used (and could overflow) on the exact path
      const float eng = exact ? 0.0f : __builtin_amdgcn_exp2f(-g[r]);
      split1(kv * eg, sm.Kh[r][ch], sm.Kl[r][ch]);
      split1(qv * eg, sm.Qh[r][ch], sm.Ql[r][ch]);
      split1(kv * eng, sm.Rh[r][ch], sm.Rl[r][ch]);
    }
  }
  __syncthreads();

  // ---- P1: the 16 x 16 tiles, one per wave: P, M, dA, dP ----
  {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    const int s = lr;   // lane holds rows 4 lg + e of column s
    if (wave < 2) {
      const bool is_p = wave == 0;
      if (is_p || ERASE) {
        if (!exact) {
          const bf16(*Ah)[SM::LDB] = is_p ? sm.Qh : sm.Kh;
          const bf16(*Al)[SM::LDB] = is_p ? sm.Ql : sm.Kl;
          f32x4 a1 = t, a2 = t;
#pragma unroll
          for (int kk = 0; kk < KKD; ++kk) {
            const int kc = 32 * kk + 8 * lg;
            const bf16x8 ah = ld8(&Ah[lr][kc]), al = ld8(&Al[lr][kc]);
            const bf16x8 bh = ld8(&sm.Rh[lr][kc]), bl = ld8(&sm.Rl[lr][kc]);
            t = mfma_bf16(ah, bh, t);
            a1 = mfma_bf16(ah, bl, a1);
            a2 = mfma_bf16(al, bh, a2);
          }
          t = t + a1 + a2;
        } else {
          // every decay formed directly: sum_c x_rc k_sc e^{G_rc - G_sc}
          const bf16(*X)[SM::LDB] = is_p ? sm.Q : sm.K;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * lg + e;
            float sum = 0.0f;
            if (s <= r) {
              for (int ch = 0; ch < DK; ++ch)
                sum += (float)X[r][ch] * (float)sm.K[s][ch] *
                       __builtin_amdgcn_exp2f(sm.G[r][ch] - sm.G[s][ch]);
            }
            t[e] = sum;
          }
        }
      }
      float(*dst)[SM::LDN] = is_p ? sm.P : sm.M;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        const bool keep = is_p ? s <= r : (ERASE && s < r);
        dst[r][s] = keep ? t[e] : 0.0f;
      }
    } else if (wave == 2) {
      // dA = -(dY U^T), strictly lower
      if constexpr (ERASE) {
#pragma unroll
        for (int kk = 0; kk < KKV; ++kk) {
          const int kc = 32 * kk + 8 * lg;
          const bf16x8 yh = ld8(&sm.Yh[lr][kc]), yl = ld8(&sm.Yl[lr][kc]);
          const bf16x8 uh = ld8(&sm.Uh[lr][kc]), ul = ld8(&sm.Ul[lr][kc]);
          t = mfma_bf16(yh, uh, t);
          t = mfma_bf16(yl, uh, t);
          t = mfma_bf16(yh, ul, t);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        sm.dA[r][s] = (ERASE && s < r) ? -t[e] : 0.0f;
      }
    } else {
      // dP = dO U^T, lower inclusive
#pragma unroll
      for (int kk = 0; kk < KKV; ++kk) {
        const int kc = 32 * kk + 8 * lg;
        const bf16x8 da = ld8(&sm.D[lr][kc]);
        const bf16x8 uh = ld8(&sm.Uh[lr][kc]), ul = ld8(&sm.Ul[lr][kc]);
        t = mfma_bf16(da, uh, t);
        t = mfma_bf16(da, ul, t);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        sm.dP[r][s] = (s <= r) ? t[e] : 0.0f;
      }
    }
  }
  __syncthreads();

  // ---- P1b: dM = diag(b) dA, sum_s dA M, the split gradient matrices ----
  {
    const int r = tid >> 4, s = tid & 15;   // the 16 lanes of a row group share r
    const float dA = sm.dA[r][s];
    const float dM = sm.beta[r] * dA;
    float hm = ERASE ? dA * sm.M[r][s] : 0.0f;
    hm = sum16(hm);
    if (s == 0) sm.dbm[r] = hm;
    sm.dA[r][s] = dM;
    bf16 h, l;
    split1(sm.dP[r][s], h, l);
    sm.dPh[r][s] = h;
    sm.dPl[r][s] = l;
    sm.dPTh[s][r] = h;
    sm.dPTl[s][r] = l;
    split1(dM, h, l);
    sm.dMh[r][s] = h;
    sm.dMl[r][s] = l;
    sm.dMTh[s][r] = h;
    sm.dMTl[s][r] = l;
  }
  __syncthreads();

  // ---- P2: dQ, dK and dG, this wave's channels, one 16-channel tile at a time ----
  {
    // dq and dk rows of this chunk: a buffer range that ends at the last valid
    // row, so stores to rows past the sequence's end are dropped (the host
    // bounds one chunk's rows below 4 GiB)
    const unsigned rows_bytes = (unsigned)sizeof(GT) * ((unsigned)(n - 1) * (unsigned)(H * DK) + DK);
    const rsrc_t rdq = make_rsrc32(dq + row0 * DK, rows_bytes);
    const rsrc_t rdk = make_rsrc32(dk + row0 * DK, rows_bytes);
    float dbpart[4] = {0.f, 0.f, 0.f, 0.f};
    auto rowx = [&](const bf16(*Xh)[SM::LDX], const bf16(*Xl)[SM::LDX]) {
      return cat(*reinterpret_cast<const bf16x4 *>(&Xh[lr][4 * lg]),
                 *reinterpret_cast<const bf16x4 *>(&Xl[lr][4 * lg]));
    };
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int c0 = 16 * (NTW * wave + nt), ch = c0 + lr;
      // h and dh rows ch (columns dv 32 kk + 8 lg .. +7) as B operands of
      // dO h^T, dY h^T and U dh^T
      f32x4 hf[KKV][2], gf[KKV][2];
#pragma unroll
      for (int kk = 0; kk < KKV; ++kk) {
        const long o = wsS + ws_state_off(DK, ch, 32 * kk + 8 * lg);   // 8 contiguous
        hf[kk][0] = *reinterpret_cast<const f32x4 *>(ws_h + o);
        hf[kk][1] = *reinterpret_cast<const f32x4 *>(ws_h + o + 4);
        gf[kk][0] = *reinterpret_cast<const f32x4 *>(ws_dh + o);
        gf[kk][1] = *reinterpret_cast<const f32x4 *>(ws_dh + o + 4);
      }
      f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ar = aq, au = aq;
      float hdh = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KKV; ++kk) {
        const int kc = 32 * kk + 8 * lg;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) hdh = fmaf(hf[kk][j][i], gf[kk][j][i], hdh);
        bf16x4 ah, al, bh, bl;
        split4(hf[kk][0], ah, al);
        split4(hf[kk][1], bh, bl);
        const bf16x8 hh = cat(ah, bh), hl = cat(al, bl);
        split4(gf[kk][0], ah, al);
        split4(gf[kk][1], bh, bl);
        const bf16x8 gh = cat(ah, bh), gl = cat(al, bl);
        const bf16x8 da = ld8(&sm.D[lr][kc]);
        aq = mfma_bf16(da, hh, aq);
        aq = mfma_bf16(da, hl, aq);
        if constexpr (ERASE) {
          const bf16x8 yh = ld8(&sm.Yh[lr][kc]), yl = ld8(&sm.Yl[lr][kc]);
          ar = mfma_bf16(yh, hh, ar);
          ar = mfma_bf16(yl, hh, ar);
          ar = mfma_bf16(yh, hl, ar);
        }
        const bf16x8 uh = ld8(&sm.Uh[lr][kc]), ul = ld8(&sm.Ul[lr][kc]);
        au = mfma_bf16(uh, gh, au);
        au = mfma_bf16(ul, gh, au);
        au = mfma_bf16(uh, gl, au);
      }
      // sum over dv: the four row groups hold the four 8-column parts
      hdh += __shfl_xor(hdh, 16);
      hdh += __shfl_xor(hdh, 32);

      // G of this lane's rows, and of the last row, before any dG is written
      // over them (only this wave touches these channels)
      float gv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gv[e] = sm.G[4 * lg + e][ch];
      const float glast = sm.G[C - 1][ch];

      // the decayed n x n x dk products: dP R^ and dM R^ (times e^G), and
      // dM^T K^ + dP^T Q^ (times e^{-G}); k = tokens 4 lg + j (hi | lo)
      f32x4 xp = {0.f, 0.f, 0.f, 0.f}, xm = xp, yf = xp;
      if (!exact) {
        const int tr = 4 * lg + (lr >> 2), tc = c0 + 4 * (lr & 3);
        const bf16x4 rth = ld_tr4(&sm.Rh[tr][tc]), rtl = ld_tr4(&sm.Rl[tr][tc]);
        const bf16x4 qth = ld_tr4(&sm.Qh[tr][tc]), qtl = ld_tr4(&sm.Ql[tr][tc]);
        const bf16x8 pA = rowx(sm.dPh, sm.dPl);
        xp = mfma_bf16(pA, cat(rth, rth), xp);
        xp = mfma_bf16(pA, cat(rtl, zero4), xp);
        const bf16x8 pT = rowx(sm.dPTh, sm.dPTl);
        yf = mfma_bf16(pT, cat(qth, qth), yf);
        yf = mfma_bf16(pT, cat(qtl, zero4), yf);
        if constexpr (ERASE) {
          const bf16x4 kth = ld_tr4(&sm.Kh[tr][tc]), ktl = ld_tr4(&sm.Kl[tr][tc]);
          const bf16x8 mA = rowx(sm.dMh, sm.dMl);
          xm = mfma_bf16(mA, cat(rth, rth), xm);
          xm = mfma_bf16(mA, cat(rtl, zero4), xm);
          const bf16x8 mT = rowx(sm.dMTh, sm.dMTl);
          yf = mfma_bf16(mT, cat(kth, kth), yf);
          yf = mfma_bf16(mT, cat(ktl, zero4), yf);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float eg = __builtin_amdgcn_exp2f(gv[e]);
          xp[e] *= eg;
          xm[e] *= eg;
          yf[e] *= __builtin_amdgcn_exp2f(-gv[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * lg + e;
          float sp = 0.0f, sx = 0.0f, sy = 0.0f;
          for (int s2 = 0; s2 < C; ++s2) {
            const float gs = sm.G[s2][ch];
            if (s2 <= r) {   // e^{G_r - G_s2}
              const float f = (float)sm.K[s2][ch] * __builtin_amdgcn_exp2f(gv[e] - gs);
              sp += sm.dP[r][s2] * f;
              if (ERASE && s2 < r) sx += sm.dA[r][s2] * f;
            }
            if (s2 >= r) {   // e^{G_s2 - G_r}
              const float f = __builtin_amdgcn_exp2f(gs - gv[e]);
              sy += sm.dP[s2][r] * (float)sm.Q[s2][ch] * f;
              if (ERASE && s2 > r) sy += sm.dA[s2][r] * (float)sm.K[s2][ch] * f;
            }
          }
          xp[e] = sp;
          xm[e] = sx;
          yf[e] = sy;
        }
      }

      // lane holds rows r = 4 lg + e of channel ch
      float tl = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        const float eg = __builtin_amdgcn_exp2f(gv[e]);
        const float ekb = __builtin_amdgcn_exp2f(glast - gv[e]);
        const float qv = (float)sm.Q[r][ch], kv = (float)sm.K[r][ch];
        const float dkh = ERASE ? -sm.beta[r] * ar[e] : 0.0f;   // -b (dY h^T), of dK^
        const float dqv = eg * aq[e] + xp[e];
        const float kpart = eg * dkh + xm[e];
        const float ku = ekb * au[e];
        const unsigned off = (unsigned)sizeof(GT) * ((unsigned)r * (unsigned)(H * DK) + (unsigned)ch);
        buf_st1(GT(dqv), rdq, off);
        buf_st1(GT(kpart + yf[e] + ku), rdk, off);
        sm.G[r][ch] = qv * dqv + kv * (kpart - yf[e] - ku);
        if constexpr (ERASE) dbpart[e] += kv * eg * ar[e];
        tl += kv * ku;
      }
      tl += __shfl_xor(tl, 16);
      tl += __shfl_xor(tl, 32);
      if (lg == 0) sm.dgl[ch] = tl + __builtin_amdgcn_exp2f(glast) * hdh;
    }
    if constexpr (ERASE) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = sum16(dbpart[e]);
        if (lr == 0) sm.dbp[wave][4 * lg + e] = p;
      }
    }
  }
  __syncthreads();

  // ---- P3: dlog a (suffix sums per channel) and db ----
  if (tid < DK) {
    const int ch = tid;
    float acc = sm.dgl[ch];   // the g_last terms sit on the last row
#pragma unroll
    for (int r = C - 1; r >= 0; --r) {
      acc += sm.G[r][ch];
      if (r < n) dlog_alpha[trow(r) * DK + ch] = acc;
    }
  } else if (tid < DK + C) {
    const int r = tid - DK;
    float db = sm.dba[r];
    if constexpr (ERASE) {
      db += sm.dbm[r];
#pragma unroll
      for (int w = 0; w < NW; ++w) db -= sm.dbp[w][r];
    }
    if (r < n) dbeta[trow(r)] = db;
  }
}

template <int DK, typename GT>
hipError_t launch_kda_grads(const BwdArgs &a) {
  const int nchunks = (a.T + C - 1) / C;
  dim3 grid((unsigned)((long)a.B * a.H * nchunks)), block(64 * NW);
#define GDR_LAUNCH(E)                                                                           \
  hipLaunchKernelGGL((chunk_bwd_kda_kernel<DK, E, GT>), grid, block, 0, a.stream,               \
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta,           \
                     a.log_alpha, (const bf16 *)a.d_o, a.ws_h, a.ws_u, a.ws_dh, a.ws_dy,         \
                     (GT *)a.dq, (GT *)a.dk, (GT *)a.dv, a.dbeta, a.dlog_alpha, a.B, a.T, a.H)
  if (a.erase) GDR_LAUNCH(true);
  else GDR_LAUNCH(false);
#undef GDR_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_bwd_kda_grads(const BwdArgs &a) {
  if (a.grad_bf16) return a.D == 128 ? launch_kda_grads<128, bf16>(a) : launch_kda_grads<64, bf16>(a);
  return a.D == 128 ? launch_kda_grads<128, float>(a) : launch_kda_grads<64, float>(a);
}

}  // namespace gdr
