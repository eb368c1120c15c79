"""Reverse-mode gradients of the token recurrence, in fp64 -- TEST
INFRASTRUCTURE ONLY (see the package docstring).

The recurrence differentiated is the one in recurrence.py (page
"NLP——线性注意力相关总结", sections on Gated DeltaNet, DeltaNet and KDA; order
decay -> predict -> write -> read).  Per chain and token t, with S [d_k, d_v]:

    S~  = D_t S_{t-1}             D_t = a_t I (scalar gate), Diag(a_t) (per
                                  channel), I (no gate); a_t = e^{log a_t}
    p   = S~^T k_t                the prediction (0 without the erase term)
    u   = b_t (v_t - p)
    S_t = S~ + k_t u^T
    o_t = S_t^T q_t

Given the loss gradients dO = dL/do_t and dS_T = dL/dS_T, the reverse sweep
carries G = dL/dS_t from t = T down to 1:

    G    += q_t dO_t^T;        dq_t = S_t dO_t
    dk_t  = G u;               du = G^T k_t
    dv_t  = b_t du;            db_t = du . (v_t - p)
    dp    = -b_t du;           G += k_t dp^T;   dk_t += S~ dp   (erase term only)
    dlog a_t = sum over the decayed entries of G o S~ (per row for the
               channel gate, over all entries for the scalar gate)
    G     = D_t G              (the gradient reaching S_{t-1})

and dS_0 = G at the end.  The states are recomputed forward first and kept
for the sweep (the oracle runs on small inputs).  Pinned against central
finite differences of recurrence.gated_delta_recurrence in
tests/test_oracle_backward.py.
"""

import numpy as np

from .recurrence import infer_gate


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def gated_delta_backward(q, k, v, beta, log_alpha=None, initial_state=None, d_o=None,
                         d_final=None, erase=True):
    """Gradients of L with dL/do = d_o [B, T, H, Dv] and dL/dS_T = d_final
    [B, H, Dk, Dv] (either may be None for zero).

    Returns a dict with dq, dk [B, T, H, Dk], dv [B, T, H, Dv], dbeta
    [B, T, H], dlog_alpha (None, [B, T, H] or [B, T, H, Dk], like log_alpha)
    and dS0 [B, H, Dk, Dv], all float64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    log_alpha = _f64(log_alpha)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    gate = infer_gate(log_alpha, q.shape)
    S0 = np.zeros((B, H, Dk, Dv)) if initial_state is None else _f64(initial_state)
    dO = np.zeros((B, T, H, Dv)) if d_o is None else _f64(d_o)
    dST = np.zeros((B, H, Dk, Dv)) if d_final is None else _f64(d_final)

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    db = np.zeros_like(beta)
    dla = None if log_alpha is None else np.zeros_like(log_alpha)
    dS0 = np.zeros((B, H, Dk, Dv))

    for b_ in range(B):
        for h in range(H):
            # forward, keeping the decayed state, the prediction, the written
            # residual and the state of every token
            S = S0[b_, h].copy()
            St_all, p_all, u_all, S_all, a_all = [], [], [], [], []
            for t in range(T):
                if gate == "none":
                    a = np.ones(Dk)
                elif gate == "scalar":
                    a = np.full(Dk, np.exp(log_alpha[b_, t, h]))
                else:
                    a = np.exp(log_alpha[b_, t, h])
                St = a[:, None] * S
                kt = k[b_, t, h]
                p = St.T @ kt if erase else np.zeros(Dv)
                u = beta[b_, t, h] * (v[b_, t, h] - p)
                S = St + np.outer(kt, u)
                St_all.append(St)
                p_all.append(p)
                u_all.append(u)
                S_all.append(S)
                a_all.append(a)
            # reverse sweep
            G = dST[b_, h].copy()
            for t in range(T - 1, -1, -1):
                qt, kt, vt = q[b_, t, h], k[b_, t, h], v[b_, t, h]
                bt = beta[b_, t, h]
                St, p, u, St_full, a = St_all[t], p_all[t], u_all[t], S_all[t], a_all[t]
                do = dO[b_, t, h]
                G = G + np.outer(qt, do)
                dq[b_, t, h] = St_full @ do
                dkt = G @ u
                du = G.T @ kt
                dv[b_, t, h] = bt * du
                db[b_, t, h] = du @ (vt - p)
                if erase:
                    dp = -bt * du
                    G = G + np.outer(kt, dp)
                    dkt = dkt + St @ dp
                dk[b_, t, h] = dkt
                if gate == "scalar":
                    dla[b_, t, h] = np.sum(G * St)
                elif gate == "channel":
                    dla[b_, t, h] = np.sum(G * St, axis=1)
                G = a[:, None] * G
            dS0[b_, h] = G
    return {"dq": dq, "dk": dk, "dv": dv, "dbeta": db, "dlog_alpha": dla, "dS0": dS0}
