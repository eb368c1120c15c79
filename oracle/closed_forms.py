"""Independent formulations that pin the recurrence (test oracle only).

None of these shares code with recurrence.py: each evaluates the same object
by a different route, so a dropped term, a wrong sign or a transposed operand
in either one shows up as a disagreement.

* ``additive_closed_form`` -- the attention-style double sum of linear
  attention.  Page "NLP——线性注意力相关总结", section "补充2", equation (2):
  unrolling the rank-1 writes gives o_t = sum_{s<=t} (k_s . q_t) v_s; the
  bittide rendering of arXiv 2607.07953, section 2, equations (3)-(5), is
  the same identity.  With a decay (Mamba-2 style scalar, or GLA style
  per-key-channel, xhh.club digest Q&A) every write is scaled by the product
  of the decays applied after it.
* ``unrolled_transition_sum`` -- the gated delta rule written as a sum over
  writes, each carried forward by an explicit d_k x d_k transition matrix.
  Page "NLP——线性注意力相关总结", section KDA, item 3 prints this unrolled
  form with the write strength beta_i missing and an ambiguous factor order;
  the version here is the one that follows from the KDA recurrence itself:
      o_t = sum_{i<=t} beta_i (q_t^T M_t ... M_{i+1} k_i) v_i
            + (M_t ... M_1 S_0)^T q_t,
      M_j = (I - beta_j k_j k_j^T) Diag(alpha_j)   (KDA)
      M_j = alpha_j (I - beta_j k_j k_j^T)          (GDN; alpha_j = 1: DeltaNet)
* ``scalar_recurrence_d1`` -- the d_k = d_v = 1 case in plain Python floats,
  where every matrix is a number and the update can be checked by hand.
"""

import math

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def additive_closed_form(q, k, v, beta=None, log_alpha=None):
    """Brute-force O(T^2 d) output of (decayed) additive linear attention.

    o_t = sum_{s<=t} beta_s * (q_t^T D_{t,s} k_s) * v_s, where D_{t,s} is the
    product of the decays of tokens s+1..t (identity without a gate), a
    scalar for a per-head gate or a diagonal for a per-channel gate.  Zero
    initial state.  Shapes as in the recurrence; returns o [B, T, H, Dv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, Dk = q.shape
    beta = np.ones((B, T, H)) if beta is None else _f64(beta)
    la = _f64(log_alpha)
    o = np.zeros(v.shape)
    for t in range(T):
        for s in range(t + 1):
            if la is None:
                w = np.einsum("bhk,bhk->bh", q[:, t], k[:, s])
            elif la.ndim == 3:
                # decays applied after token s: tokens s+1 .. t
                decay = np.exp(la[:, s + 1:t + 1].sum(axis=1))      # [B, H]
                w = decay * np.einsum("bhk,bhk->bh", q[:, t], k[:, s])
            else:
                decay = np.exp(la[:, s + 1:t + 1].sum(axis=1))      # [B, H, Dk]
                w = np.einsum("bhk,bhk->bh", q[:, t] * decay, k[:, s])
            o[:, t] += (beta[:, s] * w)[:, :, None] * v[:, s]
    return o


def _transition(k_j, beta_j, la_j, gate):
    """The d_k x d_k matrix M_j that carries the memory across token j."""
    Dk = k_j.shape[0]
    erase = np.eye(Dk) - beta_j * np.outer(k_j, k_j)
    if gate == "none":
        return erase
    if gate == "scalar":
        return math.exp(la_j) * erase
    return erase @ np.diag(np.exp(la_j))


def unrolled_transition_sum(q, k, v, beta, log_alpha=None, initial_state=None):
    """Outputs and final state from explicit transition-matrix products.

    Evaluates every chain separately with dense d_k x d_k matrices, so it is
    meant for tiny T and d.  Returns (o [B, T, H, Dv], S_T [B, H, Dk, Dv]).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    la = _f64(log_alpha)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    gate = "none" if la is None else ("scalar" if la.ndim == 3 else "channel")
    S0 = np.zeros((B, H, Dk, Dv)) if initial_state is None else _f64(initial_state)
    o = np.zeros((B, T, H, Dv))
    S_T = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            M = [_transition(k[b, j, h], beta[b, j, h],
                             None if la is None else la[b, j, h], gate)
                 for j in range(T)]
            for t in range(T):
                # carry[i] = M_t M_{t-1} ... M_{i+1}  (identity for i = t)
                carry = np.eye(Dk)
                acc = np.zeros(Dv)
                for i in range(t, -1, -1):
                    acc += beta[b, i, h] * (q[b, t, h] @ carry @ k[b, i, h]) * v[b, i, h]
                    carry = carry @ M[i]
                # after the loop carry = M_t ... M_1 (all transitions)
                acc += (carry @ S0[b, h]).T @ q[b, t, h]
                o[b, t, h] = acc
            full = np.eye(Dk)
            write_sum = np.zeros((Dk, Dv))
            for i in range(T - 1, -1, -1):
                write_sum += beta[b, i, h] * np.outer(full @ k[b, i, h], v[b, i, h])
                full = full @ M[i]
            S_T[b, h] = full @ S0[b, h] + write_sum
    return o, S_T


def scalar_recurrence_d1(q, k, v, beta, alpha, s0=0.0):
    """d_k = d_v = 1: s_t = alpha_t (1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t,
    o_t = s_t q_t, in plain Python floats.  Sequences are 1-D lists."""
    s = float(s0)
    out = []
    for qt, kt, vt, bt, at in zip(q, k, v, beta, alpha):
        s = at * (1.0 - bt * kt * kt) * s + bt * kt * vt
        out.append(s * qt)
    return out, s
