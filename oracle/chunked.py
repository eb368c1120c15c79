"""Plain fp64 chunkwise evaluation of the gated delta rule (test oracle only).

The pages name the method -- split the sequence into chunks, use matrix
products inside a chunk, pass the recurrent state from chunk to chunk, and
turn the in-chunk recurrence into products through the WY representation and
a triangular solve (xhh.club digest "Transformer 入坑笔记（五）", sections
"分块计算" and the Q&A on Gated DeltaNet and KDA; diosapp tutorial, section
五) -- but they do not print the block equations.  This module writes out the
derivation below; it is pinned against the token recurrence on many chunk
sizes and ragged tails, and nothing else depends on it.

Derivation (one chain, one chunk of n tokens r = 0..n-1, S_0 = the state
entering the chunk, g_r = cumulative sum of log alpha inside the chunk):

  Write each step as S_r = (decayed S_{r-1}) + k_r u_r^T with the written
  residual u_r = beta_r (v_r - (decayed S_{r-1})^T k_r).  By induction

    GDN:  S_r = e^{g_r} S_0 + sum_{s<=r} e^{g_r-g_s} k_s u_s^T
    KDA:  S_r = Diag(e^{g_r}) S_0 + sum_{s<=r} Diag(e^{g_r-g_s}) k_s u_s^T

  Substituting the decayed state into u_r gives a unit lower-triangular
  system for the stacked residuals U [n, d_v]:

    (I + A) U = diag(beta) (V - X S_0),
      GDN: A_rs = beta_r e^{g_r-g_s} (k_r . k_s),  X = diag(e^{g}) K
      KDA: A_rs = beta_r sum_c k_rc k_sc e^{g_rc-g_sc},  X = K * e^{G}
    (A strictly lower triangular),

  and the outputs and the state leaving the chunk are

    O   = X_q S_0 + P U,   P_rs = e^{g_r-g_s}(q_r . k_s)  (KDA: per channel), s <= r
    S_n = e^{g_last} S_0 + (K * e^{g_last-g})^T U   (KDA: Diag(e^{g_last}) S_0 ...)

  where X_q is X with Q in place of K.  A library triangular solve does the
  solve step.  Results must not depend on the chunk size beyond rounding.
"""

import numpy as np
from scipy.linalg import solve_triangular


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def chunked_gated_delta(q, k, v, beta, log_alpha=None, initial_state=None,
                        chunk=64):
    """Chunkwise evaluation; same arguments and results as the recurrence."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    la = _f64(log_alpha)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    gate = "none" if la is None else ("scalar" if la.ndim == 3 else "channel")
    S_all = (np.zeros((B, H, Dk, Dv)) if initial_state is None
             else _f64(initial_state).copy())
    o = np.zeros((B, T, H, Dv))
    for b in range(B):
        for h in range(H):
            S = S_all[b, h]
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                Q, K, V = q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h]
                bet = beta[b, c0:c1, h]
                n = c1 - c0
                if gate == "none":
                    g = np.zeros(n)
                elif gate == "scalar":
                    g = np.cumsum(la[b, c0:c1, h])
                else:
                    g = np.cumsum(la[b, c0:c1, h], axis=0)          # [n, Dk]
                if gate == "channel":
                    # pairwise decay e^{g_r - g_s} per channel, for s <= r only
                    diff = g[:, None, :] - g[None, :, :]             # [r, s, Dk]
                    lower = np.tril(np.ones((n, n), dtype=bool))
                    dec = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                    KK = np.einsum("rc,sc,rsc->rs", K, K, dec)
                    QK = np.einsum("rc,sc,rsc->rs", Q, K, dec)
                    Xk = K * np.exp(g)
                    Xq = Q * np.exp(g)
                    tail = np.exp(g[-1][None, :] - g)                 # [n, Dk]
                    Kt = K * tail
                    S_decay = np.diag(np.exp(g[-1])) @ S
                else:
                    diff = g[:, None] - g[None, :]
                    lower = np.tril(np.ones((n, n), dtype=bool))
                    dec = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
                    KK = (K @ K.T) * dec
                    QK = (Q @ K.T) * dec
                    Xk = np.exp(g)[:, None] * K
                    Xq = np.exp(g)[:, None] * Q
                    Kt = np.exp(g[-1] - g)[:, None] * K
                    S_decay = np.exp(g[-1]) * S
                A = np.tril(bet[:, None] * KK, k=-1)
                rhs = bet[:, None] * (V - Xk @ S)
                U = solve_triangular(np.eye(n) + A, rhs, lower=True,
                                     unit_diagonal=True)
                P = np.tril(QK)
                o[b, c0:c1, h] = Xq @ S + P @ U
                S = S_decay + Kt.T @ U
            S_all[b, h] = S
    return o, S_all
