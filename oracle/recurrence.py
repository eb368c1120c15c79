"""Token-by-token fp64 recurrence of the gated delta rule (test oracle only).

Definitions followed
--------------------
* DeltaNet (page "NLP——线性注意力相关总结", section "DeltaNet，引入误差修正的
  Delta Rule"): one online gradient step of rate beta_t on the reconstruction
  loss 1/2 |S^T k_t - v_t|^2 gives
      S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.
* Gated DeltaNet (same page, section "Gated DeltaNet (GDN)，引入标量遗忘门"):
      S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
      o_t = S_t^T q_t,
  with one scalar alpha_t in [0, 1] per head.
* KDA (same page, section "Kimi Delta Attention (KDA)，细粒度通道级门控"):
      S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
  with alpha_t in [0, 1]^{d_k}, one decay per key channel.

Each token applies the equation of its gate as written there, a transition
of the old state plus a rank-one write:
      S_t = M_t S_{t-1} + beta_t k_t v_t^T,
      M_t = alpha_t (I - beta_t k_t k_t^T)          (GDN; alpha_t = 1: DeltaNet)
      M_t = (I - beta_t k_t k_t^T) Diag(alpha_t)    (KDA: the channel decay is
                                                     the right-hand factor)
M_t is applied to S without forming it, as (I - beta k k^T) X = X - beta
k (k^T X), which is the same product regrouped.  For KDA, X = Diag(alpha) S:
the decay acts on the old state before the erase, which is also the order
the xhh.club digest "Transformer 入坑笔记（五）" gives in its Q&A on Gated
DeltaNet (decay the old state first, then predict from it).

Readings adopted where the pages leave a step open:
* The gate enters as log alpha (alpha = exp(log alpha)); the DeltaNet case
  is "no gate" (alpha = 1).
* No 1/sqrt(d_k) query scale, no normaliser Z and no feature map: the delta
  rule forms on the pages read the memory with the raw query.
* The state is stored [d_k, d_v] (S); p3's memory W in R^{d_v x d_phi} is S^T.
* ``erase=False`` drops the erase term -beta k k^T S and leaves the additive
  write S = alpha S + beta k v^T (plain linear attention when alpha = beta = 1,
  page "NLP——线性注意力相关总结", section "Linear Attention，线性复杂度的代价").

Layouts: q, k [B, T, H, Dk]; v [B, T, H, Dv]; beta [B, T, H];
log_alpha None | [B, T, H] (scalar gate) | [B, T, H, Dk] (channel gate);
state [B, H, Dk, Dv].  All arithmetic is float64.
"""

import numpy as np

GATES = ("none", "scalar", "channel")


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def infer_gate(log_alpha, q_shape):
    """Gate kind implied by the shape of log_alpha."""
    if log_alpha is None:
        return "none"
    if log_alpha.ndim == 3:
        return "scalar"
    if log_alpha.ndim == 4 and log_alpha.shape[-1] == q_shape[-1]:
        return "channel"
    raise ValueError(f"log_alpha shape {log_alpha.shape} matches no gate")


def gated_delta_recurrence(q, k, v, beta, log_alpha=None, initial_state=None,
                           erase=True):
    """Run the recurrence over T tokens for every (batch, head) chain.

    Returns (o [B, T, H, Dv], S_T [B, H, Dk, Dv]) in float64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    log_alpha = _f64(log_alpha)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != (B, T, H, Dk) or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("inconsistent q/k/v/beta shapes")
    gate = infer_gate(log_alpha, q.shape)

    if initial_state is None:
        S = np.zeros((B, H, Dk, Dv))
    else:
        S = _f64(initial_state).copy()
        if S.shape != (B, H, Dk, Dv):
            raise ValueError("initial_state must be [B, H, Dk, Dv]")

    o = np.empty((B, T, H, Dv))
    for t in range(T):
        kt = k[:, t]                                     # [B, H, Dk]
        bt = beta[:, t][:, :, None, None]                # [B, H, 1, 1]
        # the channel decay Diag(alpha_t) is the right-hand factor of M_t
        if gate == "channel":
            S = np.exp(log_alpha[:, t])[:, :, :, None] * S
        if erase:
            # (I - beta k k^T) S = S - beta k (k^T S)
            ktS = np.einsum("bhk,bhkv->bhv", kt, S)
            S = S - bt * np.einsum("bhk,bhv->bhkv", kt, ktS)
        # the scalar decay alpha_t multiplies the whole transition
        if gate == "scalar":
            S = np.exp(log_alpha[:, t])[:, :, None, None] * S
        S = S + bt * np.einsum("bhk,bhv->bhkv", kt, v[:, t])
        # o_t = S_t^T q_t: the read sees this token's own write
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


def recurrent_step(q, k, v, beta, log_alpha, state, erase=True):
    """One decode step for N independent sequences (a single token each).

    q, k [N, H, Dk]; v [N, H, Dv]; beta [N, H]; log_alpha None | [N, H] |
    [N, H, Dk]; state [N, H, Dk, Dv].  Returns (o [N, H, Dv], new_state).
    This is the recurrence above with T = 1 (``erase`` as there); the state
    is carried from call to call (the constant-size memory that replaces a
    KV cache, diosapp tutorial, section 一).
    """
    la = None if log_alpha is None else _f64(log_alpha)[:, None]
    o, S = gated_delta_recurrence(
        _f64(q)[:, None], _f64(k)[:, None], _f64(v)[:, None],
        _f64(beta)[:, None], la, state, erase=erase)
    return o[:, 0], S
