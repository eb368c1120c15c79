// Chunk-parallel gradients of the chunkwise gated delta-rule forward
// (bf16 q/k/v/dO, fp32 state, MFMA, gfx950; dq, dk, dv written as fp32 or as
// bf16 rounded to nearest even, template argument GT).
//
// The forward evaluated per chunk (xhh.club digest "Transformer 入坑笔记（五）",
// chunked computation; page "NLP——线性注意力相关总结", sections "Gated DeltaNet
// (GDN)" and "DeltaNet") with entering state h, g the in-chunk cumulative log
// decay, gam = e^g, ec = e^{g_last - g}, Gam_rs = e^{g_r - g_s}:
//
//   M = strict_lower(K K^T o Gam),  A = diag(b) M,  T = (I + A)^{-1}
//   P = lower_incl(Q K^T o Gam)
//   R = V - diag(gam) K h,          U = T diag(b) R
//   O = diag(gam) Q h + P U,        h' = gam_last h + K^T diag(ec) U
//
// is differentiated in reverse.  Two sequential passes (the forward kernel in
// its recompute and reverse modes) leave in the workspace, per chunk, h and U
// and, from the reverse pass, dh (the gradient of the state leaving the
// chunk) and dY = T^T dU with dU = diag(ec) K dh + P^T dO.  Given those, every
// chunk's gradients are independent:
//
//   dR = diag(b) dY = dV          dA = -strict_lower(dY U^T)
//   dP = lower_incl(dO U^T)       dM = diag(b) dA
//   db_r  = sum_v dY_rv R_rv + sum_s dA_rs M_rs
//         = dY_r . v_r - gam_r k_r . (dY h^T)_r + sum_s dA_rs M_rs
//           (R = V - diag(gam) K h: the first sum needs no stored R)
//   dQ = diag(gam) dO h^T + (dP o Gam) K
//   dK = -diag(gam) dR h^T + diag(ec) U dh^T + (dM o Gam) K + (dM o Gam)^T K
//        + (dP o Gam)^T Q
//   dg_r  = gam_r q_r.(dO h^T)_r - gam_r k_r.(dR h^T)_r - ec_r k_r.(U dh^T)_r
//           + rowsum_r(E) - colsum_r(E),   E = dM o M + dP o P
//   dg_last += sum_r ec_r k_r.(U dh^T)_r + gam_last <h, dh>
//   dlog a_t = sum_{r >= t} dg_r           (g is a within-chunk cumsum)
//
// Without the erase term (S' = gam_last S + K^T diag(ec) U, U = diag(b) V)
// T = I and R = V: dY = dU, A and M vanish, and so do every dA / dM term and
// the dR h^T terms (R no longer depends on h): db_r = dY_r . v_r,
// dK = diag(ec) U dh^T + (dP o Gam)^T Q, E = dP o P (template flag ERASE).
//
// One workgroup of four waves per (chain, chunk).  q, k and dO are exact
// bf16 and enter MFMAs unsplit; every derived operand (h, dh, U, dR, dY,
// the n x n gradient matrices) is split into bf16 hi + lo, as in the forward
// kernels, so products carry ~16 significant bits with fp32 accumulation.
#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace gdr {
namespace {

constexpr int C = kBwdChunk;   // tokens per chunk (the forward kernel's)
constexpr int NW = 4;          // waves per workgroup

template <int DK>
struct __align__(16) BwdSmem {
  static constexpr int LDB = DK + 8;   // bf16 row stride of q, k, dO: 16-byte row reads of
                                       // 16 rows hit distinct banks
  static constexpr int LDN = C + 1;    // fp32 [C][C]
  static constexpr int LDX = C + 8;    // bf16 [C][C] hi / lo
  bf16 Q[C][LDB], K[C][LDB], D[C][LDB];
  bf16 Uh[C][LDB], Ul[C][LDB], Yh[C][LDB], Yl[C][LDB];   // U and dY split once
  float G[C][LDN];                     // dM o M + dP o P
  float Hm[C][LDN];                    // dA o M
  bf16 XPh[C][LDX], XPl[C][LDX];       // dP o Gam, lower inclusive
  bf16 XMh[C][LDX], XMl[C][LDX];       // dM o Gam, strictly lower
  float g[C], gam[C], ec[C], beta[C];
  float dba[C];                        // sum_v dY_rv V_rv
  float dbp[NW][C];                    // per-wave gam_r k_r . (dY h^T)_r
  float dg[C];
  float dgp[NW][C];                    // per-wave row terms of dg
  float tlast[NW], hdh[NW];            // per-wave sums for dg_last
};

// acc + sum_i a_i b_i over 8 values given as bf16 hi / lo parts, as
// hi.hi + hi.lo + lo.hi (the split products' precision), with packed bf16
// dot products: the fp32 values need not stay live after their split
__device__ __forceinline__ float dot8_split(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl,
                                            float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t a0 = {ah[2 * i], ah[2 * i + 1]}, a1 = {al[2 * i], al[2 * i + 1]};
    const bf16x2_t b0 = {bh[2 * i], bh[2 * i + 1]}, b1 = {bl[2 * i], bl[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(a0, b0, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(a0, b1, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(a1, b0, acc, false);
  }
  return acc;
}

template <int DK, int GATE, bool ERASE, typename GT>
__global__ void __launch_bounds__(64 * NW, 2)
chunk_bwd_grad_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                      const bf16 *__restrict__ v, const float *__restrict__ beta,
                      const float *__restrict__ log_alpha,
                      const bf16 *__restrict__ d_o, const float *__restrict__ ws_h,
                      const float *__restrict__ ws_u,
                      const float *__restrict__ ws_dh, const float *__restrict__ ws_dy,
                      GT *__restrict__ dq, GT *__restrict__ dk, GT *__restrict__ dv,
                      float *__restrict__ dbeta, float *__restrict__ dlog_alpha, int B, int T,
                      int H) {
  constexpr int DV = DK;
  constexpr int NTW = DK / 64;         // 16-column dk tiles per wave
  constexpr int KKV = DV / 32;         // 32-deep k steps over dv
  using SM = BwdSmem<DK>;
  static_assert(sizeof(SM) <= 80 * 1024, "two workgroups per CU");
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nchunks = (T + C - 1) / C;
  const int chain = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int bb = chain / H, hh = chain % H;
  const int n = min(C, T - c * C);                       // valid rows of this chunk
  const long row0 = ((long)bb * T + (long)c * C) * H + hh;   // token row of the chunk's row 0
  auto trow = [&](int r) { return row0 + (long)r * H; };
  const long wsS = ((long)chain * nchunks + c) * (DK * DV);   // h, dh of this chunk
  const long wsR = ((long)chain * nchunks + c) * (C * DV);    // U, dY of this chunk

  // h^T and dh^T of one of this wave's 16-column dk tiles as B operands:
  // column dk = dkt + lr, rows dv 32 kk + 8 lg .. +7.  The first tile's loads
  // are issued here, so their latency overlaps the input loads and the n x n
  // tiles; the second tile's before the first is used.
  struct Fetch {
    f32x4 h[KKV][2], g[KKV][2];
  };
  auto fetch = [&](int nt, Fetch &f) {
    const int dkt = 16 * (NTW * wave + nt);
#pragma unroll
    for (int kk = 0; kk < KKV; ++kk) {
      const long o = wsS + ws_state_off(DK, dkt + lr, 32 * kk + 8 * lg);   // 8 contiguous
      f.h[kk][0] = *reinterpret_cast<const f32x4 *>(ws_h + o);
      f.h[kk][1] = *reinterpret_cast<const f32x4 *>(ws_h + o + 4);
      f.g[kk][0] = *reinterpret_cast<const f32x4 *>(ws_dh + o);
      f.g[kk][1] = *reinterpret_cast<const f32x4 *>(ws_dh + o + 4);
    }
  };
  Fetch fa, fb;
  fetch(0, fa);

  // ---- P0: inputs into LDS; dV = b dY; sum_v dY V; decays ----
  for (int i = tid; i < C * SM::LDX; i += 64 * NW) {     // upper-right blocks stay zero
    (&sm.XPh[0][0])[i] = (bf16)0.0f;
    (&sm.XPl[0][0])[i] = (bf16)0.0f;
    (&sm.XMh[0][0])[i] = (bf16)0.0f;
    (&sm.XMl[0][0])[i] = (bf16)0.0f;
  }
  for (int i = tid; i < C * SM::LDN; i += 64 * NW) {
    (&sm.G[0][0])[i] = 0.0f;
    (&sm.Hm[0][0])[i] = 0.0f;
  }
  {
    // every load of this phase is issued before any of them is used: one
    // memory round trip
    constexpr int BPR = DK / 8;                          // 16-byte blocks per bf16 row
    constexpr int NB = C * BPR / (64 * NW);              // blocks per thread
    constexpr int F4 = DV / 32;                          // 8 threads per row, F4 float4 each
    const int r = tid >> 3, f0 = (tid & 7) * F4;
    u32x4 xq[NB], xk[NB], xd[NB];
    f32x4 u[F4], y[F4];
    bf16x4 vr[F4];                                       // v_r at the same columns as y
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = tid + 64 * NW * j, rj = i / BPR, blk = i % BPR;
      xq[j] = u32x4{0u, 0u, 0u, 0u};
      xk[j] = xq[j];
      xd[j] = xq[j];
      if (rj < n) {
        const long off = trow(rj) * DK + 8 * blk;
        xq[j] = *reinterpret_cast<const u32x4 *>(q + off);
        xk[j] = *reinterpret_cast<const u32x4 *>(k + off);
        xd[j] = *reinterpret_cast<const u32x4 *>(d_o + off);
      }
    }
#pragma unroll
    for (int j = 0; j < F4; ++j) {
      const long o = wsR + ws_tile_off(C, r, 4 * (f0 + j));
      u[j] = *reinterpret_cast<const f32x4 *>(ws_u + o);
      y[j] = *reinterpret_cast<const f32x4 *>(ws_dy + o);
      vr[j] = bf16x4{(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
      if (r < n) vr[j] = *reinterpret_cast<const bf16x4 *>(v + trow(r) * DV + 4 * (f0 + j));
    }
    const float b = r < n ? beta[trow(r)] : 0.0f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = tid + 64 * NW * j, rj = i / BPR, blk = i % BPR;
      *reinterpret_cast<u32x4 *>(&sm.Q[rj][8 * blk]) = xq[j];
      *reinterpret_cast<u32x4 *>(&sm.K[rj][8 * blk]) = xk[j];
      *reinterpret_cast<u32x4 *>(&sm.D[rj][8 * blk]) = xd[j];
    }
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < F4; ++j) {
      const int col = 4 * (f0 + j);
      bf16x4 h4, l4;
      split4(u[j], h4, l4);
      *reinterpret_cast<bf16x4 *>(&sm.Uh[r][col]) = h4;
      *reinterpret_cast<bf16x4 *>(&sm.Ul[r][col]) = l4;
      split4(y[j], h4, l4);
      *reinterpret_cast<bf16x4 *>(&sm.Yh[r][col]) = h4;
      *reinterpret_cast<bf16x4 *>(&sm.Yl[r][col]) = l4;
      dot += (y[j][0] * (float)vr[j][0] + y[j][1] * (float)vr[j][1]) +
             (y[j][2] * (float)vr[j][2] + y[j][3] * (float)vr[j][3]);
      if (r < n) st4(dv + trow(r) * DV + col, y[j] * b);
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
    if ((tid & 7) == 0) sm.dba[r] = dot;
  }
  if (wave == 0) {
    // in-chunk cumulative log decay (rows past the end carry log a = 0)
    const float la = (GATE == kGateScalar && lane < n) ? log_alpha[trow(lane)] : 0.0f;
    float gs = la;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const float y = __shfl_up(gs, d);
      if ((lane & 31) >= d) gs += y;
    }
    const float glast = __shfl(gs, C - 1);
    if (lane < C) {
      sm.g[lane] = gs;
      sm.gam[lane] = (GATE == kGateNone) ? 1.0f : __expf(gs);
      sm.ec[lane] = (GATE == kGateNone) ? 1.0f : __expf(glast - gs);
      sm.beta[lane] = lane < n ? beta[trow(lane)] : 0.0f;
    }
  }
  __syncthreads();

  // ---- P1: per 16x16 tile position (waves 0..2): P, M, dA, dP; the
  //      elementwise terms and the decayed gradient matrices ----
  if (wave < 3) {
    const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;
    f32x4 pt = {0.f, 0.f, 0.f, 0.f}, mt = pt, at = pt, dt = pt;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
      const int kc = 32 * kk + 8 * lg;
      const bf16x8 qa = ld8(&sm.Q[16 * ti + lr][kc]);
      const bf16x8 ka = ld8(&sm.K[16 * ti + lr][kc]);
      const bf16x8 kb = ld8(&sm.K[16 * tj + lr][kc]);
      const bf16x8 da = ld8(&sm.D[16 * ti + lr][kc]);
      const bf16x8 yh = ld8(&sm.Yh[16 * ti + lr][kc]), yl = ld8(&sm.Yl[16 * ti + lr][kc]);
      const bf16x8 uh = ld8(&sm.Uh[16 * tj + lr][kc]), ul = ld8(&sm.Ul[16 * tj + lr][kc]);
      pt = mfma_bf16(qa, kb, pt);
      if constexpr (ERASE) {
        mt = mfma_bf16(ka, kb, mt);
        at = mfma_bf16(yh, uh, at);
        at = mfma_bf16(yl, uh, at);
        at = mfma_bf16(yh, ul, at);
      }
      dt = mfma_bf16(da, uh, dt);
      dt = mfma_bf16(da, ul, dt);
    }
    // lane holds rows 16 ti + 4 lg + e of column s = 16 tj + lr
    const int s = 16 * tj + lr;
    const float gs = sm.g[s];
    f32x4 xp, xm;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * lg + e;
      const float gm = (GATE == kGateNone) ? 1.0f : __expf(sm.g[r] - gs);
      const float P = (s <= r) ? pt[e] * gm : 0.0f;
      const float M = (ERASE && s < r) ? mt[e] * gm : 0.0f;
      const float dA = (ERASE && s < r) ? -at[e] : 0.0f;
      const float dP = (s <= r) ? dt[e] : 0.0f;
      const float dM = sm.beta[r] * dA;
      sm.Hm[r][s] = dA * M;
      sm.G[r][s] = dM * M + dP * P;
      xp[e] = dP * gm;
      xm[e] = dM * gm;
    }
    bf16x4 h4, l4;
    split4(xp, h4, l4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.XPh[16 * ti + 4 * lg + e][s] = h4[e];
      sm.XPl[16 * ti + 4 * lg + e][s] = l4[e];
    }
    split4(xm, h4, l4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.XMh[16 * ti + 4 * lg + e][s] = h4[e];
      sm.XMl[16 * ti + 4 * lg + e][s] = l4[e];
    }
  }
  __syncthreads();

  // ---- P2: dQ and dK, this wave's dk columns, one 16-column tile at a time ----
  {
    float hdh = 0.0f, tl = 0.0f;
    struct Acc {
      f32x4 q[2], r[2], u[2];
    };
    // dO h^T, dR h^T and U dh^T for one tile
    auto tile_mm = [&](const Fetch &f, Acc &acc) {
      f32x4(&aq)[2] = acc.q;
      f32x4(&ar)[2] = acc.r;
      f32x4(&au)[2] = acc.u;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        aq[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        ar[rb] = aq[rb];
        au[rb] = aq[rb];
      }
#pragma unroll
      for (int kk = 0; kk < KKV; ++kk) {
        const int kc = 32 * kk + 8 * lg;
        bf16x8 hh, hl, gh, gl;
        {
          const f32x4 a = f.h[kk][0], b = f.h[kk][1], c2 = f.g[kk][0], d = f.g[kk][1];
          bf16x4 ah, al, bh, bl;
          split4(a, ah, al);
          split4(b, bh, bl);
          hh = cat(ah, bh);
          hl = cat(al, bl);
          split4(c2, ah, al);
          split4(d, bh, bl);
          gh = cat(ah, bh);
          gl = cat(al, bl);
        }
        if constexpr (GATE == kGateScalar) hdh = dot8_split(hh, hl, gh, gl, hdh);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const bf16x8 da = ld8(&sm.D[16 * rb + lr][kc]);
          // dY h^T here; the row factor b (dR = diag(b) dY) is applied after
          const bf16x8 rh = ld8(&sm.Yh[16 * rb + lr][kc]), rl = ld8(&sm.Yl[16 * rb + lr][kc]);
          const bf16x8 uh = ld8(&sm.Uh[16 * rb + lr][kc]), ul = ld8(&sm.Ul[16 * rb + lr][kc]);
          aq[rb] = mfma_bf16(da, hh, aq[rb]);
          aq[rb] = mfma_bf16(da, hl, aq[rb]);
          if constexpr (ERASE) {
            ar[rb] = mfma_bf16(rh, hh, ar[rb]);
            ar[rb] = mfma_bf16(rl, hh, ar[rb]);
            ar[rb] = mfma_bf16(rh, hl, ar[rb]);
          }
          au[rb] = mfma_bf16(uh, gh, au[rb]);
          au[rb] = mfma_bf16(ul, gh, au[rb]);
          au[rb] = mfma_bf16(uh, gl, au[rb]);
        }
        // keep the LDS operand reads of at most two k steps in flight: hoisting
        // all of them ahead of the products runs the registers out
        if (kk & 1) __builtin_amdgcn_sched_barrier(0);
      }
    };
    // dq and dk rows of this chunk: a buffer range that ends at the last valid
    // row, so stores to rows past the sequence's end are dropped (the host
    // bounds one chunk's rows below 4 GiB)
    const unsigned rows_bytes = (unsigned)sizeof(GT) * ((unsigned)(n - 1) * (unsigned)(H * DK) + DK);
    const rsrc_t rdq = make_rsrc32(dq + row0 * DK, rows_bytes);
    const rsrc_t rdk = make_rsrc32(dk + row0 * DK, rows_bytes);
    // the n x n x dk products, then dQ, dK and the dg terms of one tile
    auto tile_out = [&](int nt, const Acc &acc) {
      const int dkt = 16 * (NTW * wave + nt);   // first dk column of this tile
      const f32x4(&aq)[2] = acc.q;
      const f32x4(&ar)[2] = acc.r;
      const f32x4(&au)[2] = acc.u;
      // the n x n x dk products: k = tokens {4 lg + j} u {16 + 4 lg + j};
      // K and Q columns dkt + lr as B operands (transposing reads)
      const int c0 = dkt + 4 * (lr & 3);
      const bf16x8 kb = cat(ld_tr4(&sm.K[4 * lg + (lr >> 2)][c0]),
                            ld_tr4(&sm.K[16 + 4 * lg + (lr >> 2)][c0]));
      const bf16x8 qb = cat(ld_tr4(&sm.Q[4 * lg + (lr >> 2)][c0]),
                            ld_tr4(&sm.Q[16 + 4 * lg + (lr >> 2)][c0]));
      // per-row sums of this tile, added into this wave's LDS rows at its end
      float part[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      float partb[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (rb == 1) __builtin_amdgcn_sched_barrier(0);   // one row block's operands at a time
        const int ra = 16 * rb + lr;
        auto row8 = [&](const bf16(*X)[SM::LDX]) {
          return cat(*reinterpret_cast<const bf16x4 *>(&X[ra][4 * lg]),
                     *reinterpret_cast<const bf16x4 *>(&X[ra][16 + 4 * lg]));
        };
        // transposed: row ra of X^T = column ra of X, k rows 4 lg + j (+16)
        auto col8 = [&](const bf16(*X)[SM::LDX]) {
          const int cc = 16 * rb + 4 * (lr & 3);
          return cat(ld_tr4(&X[4 * lg + (lr >> 2)][cc]), ld_tr4(&X[16 + 4 * lg + (lr >> 2)][cc]));
        };
        f32x4 xq = {0.f, 0.f, 0.f, 0.f}, xk = xq;
        xq = mfma_bf16(row8(sm.XPh), kb, xq);
        xq = mfma_bf16(row8(sm.XPl), kb, xq);
        if constexpr (ERASE) {
          xk = mfma_bf16(row8(sm.XMh), kb, xk);
          xk = mfma_bf16(row8(sm.XMl), kb, xk);
          xk = mfma_bf16(col8(sm.XMh), kb, xk);
          xk = mfma_bf16(col8(sm.XMl), kb, xk);
        }
        xk = mfma_bf16(col8(sm.XPh), qb, xk);
        xk = mfma_bf16(col8(sm.XPl), qb, xk);
        // lane holds rows r0 + e of column dkt + lr
        const int r0 = 16 * rb + 4 * lg, col = dkt + lr;
        const f32x4 gm4 = *reinterpret_cast<const f32x4 *>(&sm.gam[r0]);
        const f32x4 ec4 = *reinterpret_cast<const f32x4 *>(&sm.ec[r0]);
        const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sm.beta[r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r0 + e;
          const float gq = gm4[e] * aq[rb][e];
          const float gr = ERASE ? gm4[e] * b4[e] * ar[rb][e] : 0.0f;
          const float gu = ec4[e] * au[rb][e];
          const unsigned off = (unsigned)sizeof(GT) * ((unsigned)r * (unsigned)(H * DK) + (unsigned)col);
          buf_st1(GT(gq + xq[e]), rdq, off);
          buf_st1(GT(gu - gr + xk[e]), rdk, off);
          const float kv = (float)sm.K[r][col];
          if constexpr (ERASE) partb[rb][e] += kv * (gm4[e] * ar[rb][e]);
          if constexpr (GATE == kGateScalar) {
            const float qv = (float)sm.Q[r][col];
            part[rb][e] += qv * gq - kv * gr - kv * gu;
            tl += kv * gu;
          }
        }
      }
      // lane lr = 0 of each row group owns rows 16 rb + 4 lg + e of this wave's
      // slots: the first tile writes them, the second adds (same lane, in order)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * lg + e;
          if constexpr (ERASE) {
            const float pb = sum16(partb[rb][e]);
            if (lr == 0) sm.dbp[wave][r] = (nt == 0 ? 0.0f : sm.dbp[wave][r]) + pb;
          }
          if constexpr (GATE == kGateScalar) {
            const float p = sum16(part[rb][e]);
            if (lr == 0) sm.dgp[wave][r] = (nt == 0 ? 0.0f : sm.dgp[wave][r]) + p;
          }
        }
    };
    Acc acc;
    tile_mm(fa, acc);
    tile_out(0, acc);
    if constexpr (NTW == 2) {
      // the second tile after the first: both tiles' operands live at once
      // would not fit the registers (the other workgroup on the CU covers
      // this fetch's latency)
      __builtin_amdgcn_sched_barrier(0);
      fetch(1, fb);
      tile_mm(fb, acc);
      tile_out(1, acc);
    }
    if constexpr (GATE == kGateScalar) {
      tl = sum64(tl);
      hdh = sum64(hdh);
      if (lane == 0) {
        sm.tlast[wave] = tl;
        sm.hdh[wave] = hdh;
      }
    }
  }
  __syncthreads();

  // ---- P3: db, dg and its suffix sums (one lane per row) ----
  if (wave == 0) {
    const int r = lane & 31;
    float db = sm.dba[r], gsum = 0.0f;
    if constexpr (ERASE) {
#pragma unroll
      for (int w = 0; w < NW; ++w) db -= sm.dbp[w][r];
    }
#pragma unroll 8
    for (int s2 = 0; s2 < C; ++s2) {
      if constexpr (ERASE) db += sm.Hm[r][s2];
      gsum += sm.G[r][s2] - sm.G[s2][r];
    }
    if (lane < C && r < n) dbeta[trow(r)] = db;
    if constexpr (GATE == kGateScalar) {
      float dg = gsum;
#pragma unroll
      for (int w = 0; w < NW; ++w) dg += sm.dgp[w][r];
      if (r == C - 1) {
        float tsum = 0.0f, hsum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          tsum += sm.tlast[w];
          hsum += sm.hdh[w];
        }
        dg += tsum + sm.gam[C - 1] * hsum;
      }
      if (lane < C) sm.dg[r] = dg;
      wave_lds_sync();
      float acc = 0.0f;
      for (int s2 = r; s2 < C; ++s2) acc += sm.dg[s2];
      if (lane < C && r < n) dlog_alpha[trow(r)] = acc;
    }
  }
}

template <int DK, typename GT>
hipError_t launch_dk(const BwdArgs &a) {
  const int nchunks = (a.T + C - 1) / C;
  dim3 grid((unsigned)((long)a.B * a.H * nchunks)), block(64 * NW);
#define GDR_LAUNCH(G, E)                                                                        \
  hipLaunchKernelGGL((chunk_bwd_grad_kernel<DK, G, E, GT>), grid, block, 0, a.stream,           \
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta,          \
                     a.log_alpha, (const bf16 *)a.d_o, a.ws_h, a.ws_u, a.ws_dh, a.ws_dy,        \
                     (GT *)a.dq, (GT *)a.dk, (GT *)a.dv, a.dbeta, a.dlog_alpha, a.B, a.T, a.H)
  if (a.erase) {
    if (a.gate == kGateNone) GDR_LAUNCH(kGateNone, true);
    else GDR_LAUNCH(kGateScalar, true);
  } else {
    if (a.gate == kGateNone) GDR_LAUNCH(kGateNone, false);
    else GDR_LAUNCH(kGateScalar, false);
  }
#undef GDR_LAUNCH
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk_by_grad(const BwdArgs &a) {
  return a.grad_bf16 ? launch_dk<DK, bf16>(a) : launch_dk<DK, float>(a);
}

}  // namespace

hipError_t launch_chunk_bwd_grads(const BwdArgs &a) {
  return a.D == 128 ? launch_dk_by_grad<128>(a) : launch_dk_by_grad<64>(a);
}

}  // namespace gdr
