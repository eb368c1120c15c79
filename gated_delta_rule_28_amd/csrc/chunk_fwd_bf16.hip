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
//   A   = strict_lower(diag(b) (K K^T o Gam))         (a2)
//   T'  = (I + A)^{-1} diag(b)                         (a3, unit lower solve)
//   P   = lower_incl(Q K^T o Gam)                      (a5)
//   U   = T' (V - diag(gam) K S)                       (a4, written residuals)
//   O   = diag(gam) Q S + P U                          (a6/a7)
//   S  <- gam_last S + K^T diag(e^{g_last - g}) U      (a6, carried state)
//
// Mapping.  One workgroup per (batch, head, Dv-slice of DVS columns); the
// Dv columns of S, U and O are independent given K, b and g, so slices of a
// chain never talk.  The workgroup walks the chunks in order.  Each of its
// DVS/16 waves owns 16 state columns and keeps them in MFMA accumulators for
// the whole sequence: every state-dependent product (K S, Q S, T'R, P U,
// K^T U') takes its right operand straight from those accumulator registers
// (an accumulator tile holds rows 4g..4g+3 of column l&15, which is exactly
// what a 16x16x32 B operand needs if the k order inside each 32-block is
// permuted; the left operands in LDS are stored with the same permutation).
// So the serial state chain never round-trips through LDS.  The per-chunk
// key-only work (decay cumsum, K K^T, Q K^T, the solve) is shared by the
// waves through LDS.
//
// Precision.  q, k, v are exact bf16 and enter MFMAs unsplit; every derived
// operand (S, R, U, T', P) is split into bf16 hi + lo and multiplied as
// hi*hi + hi*lo + lo*hi (two products when the other side is exact), so the
// products carry ~16 significant bits and accumulate in fp32.
#include "common.h"
#include "internal.h"

namespace gdr {
namespace {

// k order inside each 32-wide block: natural index 32kk + 16h + 4g + j lives
// at 32kk + 8g + 4h + j, so one 16-byte LDS read returns the eight k values a
// lane needs for an operand that pairs with accumulator rows 4g..4g+3 of two
// adjacent 16-row tiles.
__device__ __forceinline__ int perm32(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void split4(const f32x4 x, bf16x4 &hi, bf16x4 &lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bf16 h, l;
    split_bf16(x[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// acc += L (16x16, fp32, row-major at L[m*ldl + k]) * R (16x16, fp32, given
// transposed: R[k][n] = RT[n*ldr + k]) to ~fp32 accuracy with two MFMAs: the
// 32-deep k axis carries [L_hi | L_lo] against [R_hi ; R_hi], then
// [L_hi | L_lo] against [R_lo ; 0].
__device__ __forceinline__ f32x4 mm16_split(const float *L, int ldl, const float *RT, int ldr,
                                            f32x4 acc, int lane) {
  const int m = lane & 15, g = lane >> 4, k0 = 8 * (g & 1);
  bf16x8 a, b1, b2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bf16 lh, ll, rh, rl;
    split_bf16(L[m * ldl + k0 + j], lh, ll);
    split_bf16(RT[m * ldr + k0 + j], rh, rl);
    a[j] = g < 2 ? lh : ll;
    b1[j] = rh;
    b2[j] = g < 2 ? rl : (bf16)0.0f;
  }
  acc = mfma_bf16(a, b1, acc);
  return mfma_bf16(a, b2, acc);
}

template <int C, int DK, int DVS>
struct __align__(16) Smem {
  static constexpr int LDK = DK + 8;   // bf16 stride of [C][DK] rows (pads banks)
  static constexpr int LDC = C + 8;    // bf16 stride of [*][C] rows
  static constexpr int LDA = C + 4;    // fp32 stride of [C][C] rows
  bf16 Q[C][LDK];                      // q rows, dk permuted
  bf16 K[C][LDK];                      // k rows, dk permuted
  bf16 KT[DK][LDC];                    // k^T: row = dk, tokens permuted
  bf16 VT[DVS][LDC];                   // v^T slice: row = value column, tokens natural
  bf16 Th[C][LDC], Tl[C][LDC];         // T' = (I+A)^{-1} diag(b), cols permuted
  bf16 Ph[C][LDC], Pl[C][LDC];         // P, cols permuted
  float gam[C], ec[C], beta[C], g[C];  // e^g, e^{g_last-g}, b, g
  float A[C][LDA];                     // A (strict lower), natural
  float TT[C][LDA];                    // T^T: TT[s][r] = T[r][s]
  float Td[C / 16][16][20];            // diagonal blocks of T, row-major
  float X[DVS / 16][16][20];           // per-wave transposed scratch
};

template <int C, int DK, int DVS, typename OutT, int GATE>
__global__ void __launch_bounds__(4 * DVS, 1)
chunk_fwd_bf16_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                      const bf16 *__restrict__ v, const float *__restrict__ beta,
                      const float *__restrict__ log_alpha, const float *initial_state,
                      OutT *__restrict__ o, float *final_state, int B, int T, int H) {
  constexpr int NW = DVS / 16;         // waves; wave w owns value columns 16w..16w+15
  constexpr int NT = 64 * NW;
  constexpr int DV = DK;               // full value width (Dk == Dv)
  constexpr int NSLICE = DV / DVS;
  constexpr int NB = C / 16;           // 16-row blocks per chunk
  constexpr int KKD = DK / 32;         // 32-deep k steps over dk
  constexpr int KKC = C / 32;          // 32-deep k steps over tokens
  static_assert(C == 64 && (DK == 64 || DK == 128) && (DVS == 32 || DVS == 64), "tile config");
  using S_t = Smem<C, DK, DVS>;
  __shared__ S_t sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int col0 = slice * DVS + 16 * wave;   // first value column of this wave
  const long tok_stride = (long)H;            // rows of one head are H apart

  // zero the triangular operands once: their upper blocks are never written
  for (int i = tid; i < C * S_t::LDC; i += NT) {
    (&sm.Th[0][0])[i] = (bf16)0.0f;
    (&sm.Tl[0][0])[i] = (bf16)0.0f;
    (&sm.Ph[0][0])[i] = (bf16)0.0f;
    (&sm.Pl[0][0])[i] = (bf16)0.0f;
  }

  // state columns col0 + lr, rows 16mb + 4lg + e, in accumulators
  f32x4 Sacc[DK / 16];
  {
    const float *S0 = initial_state ? initial_state + (long)chain * DK * DV : nullptr;
#pragma unroll
    for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Sacc[mb][e] = S0 ? S0[(long)(16 * mb + 4 * lg + e) * DV + col0 + lr] : 0.0f;
  }

  const int nchunks = (T + C - 1) / C;
  for (int ci = 0; ci < nchunks; ++ci) {
    const int t0 = ci * C;
    const int n = min(C, T - t0);
    __syncthreads();   // previous chunk's readers are done with the shared tiles

    // ---- load q, k (row-major, dk permuted) and k^T; v^T slice; b; log a ----
    for (int it = tid; it < C / 4 * (DK / 8); it += NT) {
      const int cs = it % (DK / 8), rgp = it / (DK / 8);
      const int c0 = 8 * cs, r0 = 4 * rgp;
      bf16x8 qv[4], kv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        if (r < n) {
          const long off = (((long)bb * T + t0 + r) * tok_stride + hh) * DK + c0;
          qv[i] = ld8(q + off);
          kv[i] = ld8(k + off);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) { qv[i][j] = (bf16)0.0f; kv[i][j] = (bf16)0.0f; }
        }
        const int p0 = perm32(c0), p1 = perm32(c0 + 4);
        *reinterpret_cast<bf16x4 *>(&sm.Q[r][p0]) = bf16x4{qv[i][0], qv[i][1], qv[i][2], qv[i][3]};
        *reinterpret_cast<bf16x4 *>(&sm.Q[r][p1]) = bf16x4{qv[i][4], qv[i][5], qv[i][6], qv[i][7]};
        *reinterpret_cast<bf16x4 *>(&sm.K[r][p0]) = bf16x4{kv[i][0], kv[i][1], kv[i][2], kv[i][3]};
        *reinterpret_cast<bf16x4 *>(&sm.K[r][p1]) = bf16x4{kv[i][4], kv[i][5], kv[i][6], kv[i][7]};
      }
      const int pr = perm32(r0);   // 4 consecutive tokens stay consecutive
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<bf16x4 *>(&sm.KT[c0 + j][pr]) = bf16x4{kv[0][j], kv[1][j], kv[2][j], kv[3][j]};
    }
    for (int it = tid; it < C / 4 * (DVS / 8); it += NT) {
      const int cs = it % (DVS / 8), rgp = it / (DVS / 8);
      const int c0 = 8 * cs, r0 = 4 * rgp;
      bf16x8 vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        if (r < n) {
          vv[i] = ld8(v + (((long)bb * T + t0 + r) * tok_stride + hh) * DV + slice * DVS + c0);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) vv[i][j] = (bf16)0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<bf16x4 *>(&sm.VT[c0 + j][r0]) = bf16x4{vv[0][j], vv[1][j], vv[2][j], vv[3][j]};
    }
    if (wave == 0) {
      // in-chunk cumulative log decay (a1): inclusive scan over the wave
      const int r = lane;   // C == 64 == wavefront
      const long gi = ((long)bb * T + t0 + r) * tok_stride + hh;
      float la = 0.0f, bt = 0.0f;
      if (r < n) {
        bt = beta[gi];
        if (GATE == kGateScalar) la = log_alpha[gi];
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off, 64);
        if (lane >= off) la += y;
      }
      const float glast = __shfl(la, 63, 64);
      sm.g[r] = la;
      sm.gam[r] = __expf(la);
      sm.ec[r] = __expf(glast - la);
      sm.beta[r] = bt;
    }
    __syncthreads();

    // ---- a2 / a5: K K^T and Q K^T, lower tiles only, with the decay ----
    {
      constexpr int NTILE = NB * (NB + 1) / 2;
      for (int tt = wave; tt < 2 * NTILE; tt += NW) {
        const bool isq = tt >= NTILE;
        int x = isq ? tt - NTILE : tt, i = 0;
        while (x > i) { x -= i + 1; ++i; }
        const int j = x;   // tile (i, j), j <= i
        const bf16(*Xr)[S_t::LDK] = isq ? sm.Q : sm.K;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KKD; ++kk)
          acc = mfma_bf16(ld8(&Xr[16 * i + lr][32 * kk + 8 * lg]), ld8(&sm.K[16 * j + lr][32 * kk + 8 * lg]), acc);
        const int s = 16 * j + lr;
        const float gs = sm.g[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * lg + e;
          const float dec = (GATE == kGateNone) ? 1.0f : __expf(sm.g[r] - gs);
          if (!isq) {
            sm.A[r][s] = (s < r) ? sm.beta[r] * acc[e] * dec : 0.0f;
          } else {
            const float pv = (s <= r) ? acc[e] * dec : 0.0f;
            bf16 h, l;
            split_bf16(pv, h, l);
            sm.Ph[r][perm32(s)] = h;
            sm.Pl[r][perm32(s)] = l;
          }
        }
      }
    }
    __syncthreads();

    // ---- a3: T = (I + A)^{-1}; diagonal 16x16 blocks by forward substitution ----
    for (int bk = wave; bk < NB; bk += NW) {
      const int j = lr;                 // column of the block inverse
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == j) ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= sm.A[16 * bk + r][16 * bk + s] * x[s];
        x[r] = acc;
      }
      // lane group lg writes rows 4lg..4lg+3 of column j
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        sm.Td[bk][r][j] = x[r];
        const float tp = x[r] * sm.beta[16 * bk + j];
        bf16 h, l;
        split_bf16(tp, h, l);
        sm.Th[16 * bk + r][perm32(16 * bk + j)] = h;
        sm.Tl[16 * bk + r][perm32(16 * bk + j)] = l;
      }
      *reinterpret_cast<f32x4 *>(&sm.TT[16 * bk + j][16 * bk + 4 * lg]) =
          f32x4{x[4 * lg], x[4 * lg + 1], x[4 * lg + 2], x[4 * lg + 3]};
    }
    __syncthreads();
    // off-diagonal blocks by distance d = i - j:  T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
    for (int d = 1; d < NB; ++d) {
      for (int jb = wave; jb < NB - d; jb += NW) {
        const int ib = jb + d;
        f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = jb; kb < ib; ++kb)
          xacc = mm16_split(&sm.A[16 * ib][16 * kb], S_t::LDA, &sm.TT[16 * jb][16 * kb], S_t::LDA, xacc, lane);
        // X^T into this wave's scratch, then T_ij = -T_ii X
        *reinterpret_cast<f32x4 *>(&sm.X[wave][lr][4 * lg]) = xacc;
        __builtin_amdgcn_wave_barrier();
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mm16_split(&sm.Td[ib][0][0], 20, &sm.X[wave][0][0], 20, z, lane);
        __builtin_amdgcn_wave_barrier();
        const int s = 16 * jb + lr;
        const float bs = sm.beta[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * ib + 4 * lg + e;
          z[e] = -z[e];
          bf16 h, l;
          split_bf16(z[e] * bs, h, l);
          sm.Th[r][perm32(s)] = h;
          sm.Tl[r][perm32(s)] = l;
        }
        *reinterpret_cast<f32x4 *>(&sm.TT[s][16 * ib + 4 * lg]) = z;
      }
      __syncthreads();
    }

    // ---- serial state pass (a4, a6, a7): wave-local, state in registers ----
    {
      // B operands from the state accumulators (k = dk, permuted order)
      bf16x8 Sh[KKD], Sl[KKD];
#pragma unroll
      for (int kk = 0; kk < KKD; ++kk) {
        bf16x4 h0, l0, h1, l1;
        split4(Sacc[2 * kk], h0, l0);
        split4(Sacc[2 * kk + 1], h1, l1);
        Sh[kk] = cat(h0, h1);
        Sl[kk] = cat(l0, l1);
      }
      // K S and Q S  (rows = tokens of the chunk, cols = this wave's 16 columns)
      f32x4 KS[NB], QS[NB];
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KKD; ++kk) {
          const bf16x8 ak = ld8(&sm.K[16 * rb + lr][32 * kk + 8 * lg]);
          const bf16x8 aq = ld8(&sm.Q[16 * rb + lr][32 * kk + 8 * lg]);
          a1 = mfma_bf16(ak, Sh[kk], a1);
          a1 = mfma_bf16(ak, Sl[kk], a1);
          a2 = mfma_bf16(aq, Sh[kk], a2);
          a2 = mfma_bf16(aq, Sl[kk], a2);
        }
        KS[rb] = a1;
        QS[rb] = a2;
      }
      // R = V - diag(gam) K S, as split B operands over tokens
      bf16x8 Rh[KKC], Rl[KKC];
#pragma unroll
      for (int kk = 0; kk < KKC; ++kk) {
        bf16x4 hh2[2], ll2[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int rb = 2 * kk + hf;
          const int r0 = 16 * rb + 4 * lg;
          const bf16x4 vv = *reinterpret_cast<const bf16x4 *>(&sm.VT[16 * wave + lr][r0]);
          f32x4 rr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gm = (GATE == kGateNone) ? 1.0f : sm.gam[r0 + e];
            rr[e] = (float)vv[e] - gm * KS[rb][e];
          }
          split4(rr, hh2[hf], ll2[hf]);
        }
        Rh[kk] = cat(hh2[0], hh2[1]);
        Rl[kk] = cat(ll2[0], ll2[1]);
      }
      // U = T' R  (T' lower triangular: row block rb needs token blocks <= rb)
      f32x4 U[NB];
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk <= rb / 2; ++kk) {
          const bf16x8 th = ld8(&sm.Th[16 * rb + lr][32 * kk + 8 * lg]);
          const bf16x8 tl = ld8(&sm.Tl[16 * rb + lr][32 * kk + 8 * lg]);
          acc = mfma_bf16(th, Rh[kk], acc);
          acc = mfma_bf16(th, Rl[kk], acc);
          acc = mfma_bf16(tl, Rh[kk], acc);
        }
        U[rb] = acc;
      }
      // split U (for P U) and U' = diag(e^{g_last - g}) U (for the state update)
      bf16x8 Uh[KKC], Ul[KKC], Wh[KKC], Wl[KKC];
#pragma unroll
      for (int kk = 0; kk < KKC; ++kk) {
        bf16x4 uh[2], ul[2], wh[2], wl[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int rb = 2 * kk + hf;
          split4(U[rb], uh[hf], ul[hf]);
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (GATE == kGateNone) ? U[rb][e] : sm.ec[16 * rb + 4 * lg + e] * U[rb][e];
          split4(w, wh[hf], wl[hf]);
        }
        Uh[kk] = cat(uh[0], uh[1]);
        Ul[kk] = cat(ul[0], ul[1]);
        Wh[kk] = cat(wh[0], wh[1]);
        Wl[kk] = cat(wl[0], wl[1]);
      }
      // O = diag(gam) Q S + P U, written straight from the accumulators
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gm = (GATE == kGateNone) ? 1.0f : sm.gam[16 * rb + 4 * lg + e];
          acc[e] = gm * QS[rb][e];
        }
#pragma unroll
        for (int kk = 0; kk <= rb / 2; ++kk) {
          const bf16x8 ph = ld8(&sm.Ph[16 * rb + lr][32 * kk + 8 * lg]);
          const bf16x8 pl = ld8(&sm.Pl[16 * rb + lr][32 * kk + 8 * lg]);
          acc = mfma_bf16(ph, Uh[kk], acc);
          acc = mfma_bf16(ph, Ul[kk], acc);
          acc = mfma_bf16(pl, Uh[kk], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * lg + e;
          if (r < n) o[(((long)bb * T + t0 + r) * tok_stride + hh) * DV + col0 + lr] = from_f32<OutT>(acc[e]);
        }
      }
      // S <- gam_last S + K^T U'
      const float glast = (GATE == kGateNone) ? 1.0f : sm.gam[C - 1];
#pragma unroll
      for (int mb = 0; mb < DK / 16; ++mb) {
        f32x4 acc = Sacc[mb] * glast;
#pragma unroll
        for (int kk = 0; kk < KKC; ++kk) {
          const bf16x8 a = ld8(&sm.KT[16 * mb + lr][32 * kk + 8 * lg]);
          acc = mfma_bf16(a, Wh[kk], acc);
          acc = mfma_bf16(a, Wl[kk], acc);
        }
        Sacc[mb] = acc;
      }
    }
  }

  if (final_state) {
    float *SF = final_state + (long)chain * DK * DV;
#pragma unroll
    for (int mb = 0; mb < DK / 16; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) SF[(long)(16 * mb + 4 * lg + e) * DV + col0 + lr] = Sacc[mb][e];
  }
}

template <int DK, int DVS, typename OutT, int GATE>
hipError_t launch_cfg(const ChunkArgs &a) {
  constexpr int C = 64;
  const int nslice = DK / DVS;
  dim3 grid((unsigned)(a.B * a.H * nslice)), block(4 * DVS);
  hipLaunchKernelGGL((chunk_fwd_bf16_kernel<C, DK, DVS, OutT, GATE>), grid, block, 0, a.stream,
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
  return a.in_bf16 && (a.D == 128 || a.D == 64) && (a.chunk == 0 || a.chunk == 64) &&
         a.gate != kGateChannel;
}

hipError_t launch_chunk_fwd_bf16(const ChunkArgs &a) {
  // 64 value columns per workgroup fills the chip once there are >= 256
  // (chain, slice) pairs; fewer chains use 32-column slices for more workgroups.
  const long chains = (long)a.B * a.H;
  if (a.D == 128) {
    if (chains * 2 >= 256) return by_out<128, 64>(a);
    return by_out<128, 32>(a);
  }
  if (chains >= 256) return by_out<64, 64>(a);
  return by_out<64, 32>(a);
}

}  // namespace gdr
