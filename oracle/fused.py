"""Prologue and epilogue activations around the recurrence, in fp64 --
TEST INFRASTRUCTURE ONLY (see the package docstring).

These are the per-token transforms a layer applies to its projections
before the recurrence and to the read-out after it.  What the pages fix:
  - q and k pass through a feature map before the recurrence
    ("线性注意力架构：机制、权衡与跨层路由", section 3, eqs. (7)-(8));
  - a and b lie in (0, 1) (xhh.club digest, Q&A on Gated DeltaNet;
    page "NLP——线性注意力相关总结", KDA section);
  - GLA's gate is sigmoid(.)^{1/tau} with tau = 16 (xhh.club digest, Q&A on
    GLA's gate);
  - the read-out passes an output gate with a SiLU activation (diosapp
    tutorial, section 四, the table of Gated DeltaNet's three gates).
Each function is the plain definition; the GPU path fuses them into its
kernels (gdr_fuse flags).

Readings adopted: the feature map is the L2
normalisation x / sqrt(sum x^2 + 1e-6) per (token, head) over d_k (unit keys
make the erase an orthogonal projection, diosapp tutorial, section 三); b
from a logit is the logistic sigmoid; a from an unconstrained x is
exp(-softplus(x)); the SiLU gate is o * g * sigmoid(g).
"""

import numpy as np

L2_EPS = 1e-6
GLA_TAU = 16.0


def l2_normalize(x, eps=L2_EPS):
    """x / sqrt(sum_i x_i^2 + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    """1 / (1 + e^{-x})."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), written so that large x does not overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def log_decay(x, kind):
    """log a from the decay pre-activation x: kind None returns x itself,
    "softplus" gives -softplus(x), "gla" gives log(sigmoid(x)^{1/16})."""
    if kind is None or x is None:
        return None if x is None else np.asarray(x, dtype=np.float64)
    if kind == "softplus":
        return -softplus(x)
    if kind == "gla":
        return np.log(sigmoid(x)) / GLA_TAU
    raise ValueError(f"unknown decay transform {kind!r}")


def prologue(q, k, beta, log_alpha, *, qk_l2norm=False, beta_sigmoid=False, decay=None):
    """The recurrence's inputs from the layer's pre-activations."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    beta = sigmoid(beta) if beta_sigmoid else np.asarray(beta, dtype=np.float64)
    return q, k, beta, log_decay(log_alpha, decay)


def silu_gate(o, g):
    """The SiLU output gate: o * g * sigmoid(g)."""
    g = np.asarray(g, dtype=np.float64)
    return np.asarray(o, dtype=np.float64) * g * sigmoid(g)
