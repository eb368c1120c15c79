"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.

This module only draws random inputs and names the workload shapes; it holds
none of the gated-delta arithmetic.  Both the fp64 oracle and the GPU path
read the tensors it returns (the oracle after an exact upcast of the rounded
values), so they always see bit-identical inputs.

Input recipe (identical for every workload, only the shapes and the gate
parameters change):
  q, k ~ N(0, 1), each L2-normalised over d_k per (token, head)
  v    ~ N(0, 1)
  beta = sigmoid(N(0, 1))                       one per (token, head)
  log alpha = -softplus(N(mu, sigma))           one per (token, head), or one
                                                per (token, head, key channel)
  initial state (decode) ~ N(0, state_std^2), fp32
The draws are float32 from a torch.Generator on the target device, in the
fixed order q, k, v, beta, alpha, state; q, k, v are then rounded to the
workload's input dtype (round-to-nearest-even for bf16).
"""

from dataclasses import dataclass, field
import hashlib

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class ChunkWorkload:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    chunk: int
    gate: str                 # "none" | "scalar" | "channel"
    in_dtype: str             # "f32" | "bf16"
    alpha_mu: float = -2.0
    alpha_sigma: float = 0.5
    description: str = ""

    @property
    def tokens(self):
        return self.B * self.T


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    Dk: int
    Dv: int
    steps: int
    gate: str
    in_dtype: str
    alpha_mu: float = -2.0
    alpha_sigma: float = 0.5
    state_std: float = 0.02
    description: str = ""


# The five synthetic workloads, in order.  Sizes and distributions are the
# ones the gated-delta pages' layer shapes suggest (d_k = d_v = 128 heads,
# hybrid-LLM-like head counts) plus one tiny fp32 case.
WORKLOADS = [
    ChunkWorkload("gdn_f32_tiny", B=1, T=64, H=1, Dk=16, Dv=16, chunk=16,
                  gate="scalar", in_dtype="f32",
                  description="Gated DeltaNet, fp32 throughout, one head, d=16"),
    ChunkWorkload("deltanet_bf16_b4h8t2048", B=4, T=2048, H=8, Dk=128, Dv=128,
                  chunk=64, gate="none", in_dtype="bf16",
                  description="DeltaNet (alpha = 1), bf16 inputs, fp32 state"),
    ChunkWorkload("gdn_bf16_b8h16t4096", B=8, T=4096, H=16, Dk=128, Dv=128,
                  chunk=64, gate="scalar", in_dtype="bf16",
                  description="Gated DeltaNet layer shape, bf16 inputs, fp32 state"),
    ChunkWorkload("kda_bf16_b2h32t8192", B=2, T=8192, H=32, Dk=128, Dv=128,
                  chunk=64, gate="channel", in_dtype="bf16",
                  alpha_mu=-3.0, alpha_sigma=1.0,
                  description="KDA per-channel decay, bf16 inputs, fp32 state"),
    DecodeWorkload("decode_gdn_n256h32", N=256, H=32, Dk=128, Dv=128,
                   steps=128, gate="scalar", in_dtype="bf16",
                   description="batched single-token decode, fp32 state in HBM"),
]
# the Gated DeltaNet variant of the b4h8t2048 shape
GDN_B4H8 = ChunkWorkload("gdn_bf16_b4h8t2048", B=4, T=2048, H=8, Dk=128, Dv=128,
                         chunk=64, gate="scalar", in_dtype="bf16",
                         description="Gated DeltaNet, bf16 inputs, fp32 state")
HEADLINE = WORKLOADS[2]
DECODE = WORKLOADS[4]


def by_name(name):
    for w in WORKLOADS + [GDN_B4H8]:
        if w.name == name:
            return w
    raise KeyError(name)


_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(tag):
    return _DTYPES[tag]


def _generator(seed_parts, device):
    digest = hashlib.sha256(repr(tuple(seed_parts)).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(digest[:8], "little") & ((1 << 63) - 1))
    return g


def _unit_rows(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def make_chunk_inputs(B, T, H, Dk, Dv, gate="scalar", in_dtype="bf16", *,
                      seed=0, device="cpu", alpha_mu=-2.0, alpha_sigma=0.5,
                      initial_state_std=None):
    """Seeded inputs for one chunkwise forward call.

    Returns a dict with q, k [B, T, H, Dk] and v [B, T, H, Dv] in the input
    dtype, beta [B, T, H] fp32, log_alpha (None, [B, T, H] or [B, T, H, Dk])
    fp32 and initial_state (None or [B, H, Dk, Dv] fp32).
    """
    if gate not in ("none", "scalar", "channel"):
        raise ValueError(gate)
    g = _generator(("chunk", B, T, H, Dk, Dv, gate, in_dtype, seed), device)
    dt = _DTYPES[in_dtype]
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q = _unit_rows(torch.randn(B, T, H, Dk, **kw)).to(dt)
    k = _unit_rows(torch.randn(B, T, H, Dk, **kw)).to(dt)
    v = torch.randn(B, T, H, Dv, **kw).to(dt)
    beta = torch.sigmoid(torch.randn(B, T, H, **kw))
    if gate == "none":
        log_alpha = None
    else:
        shape = (B, T, H) if gate == "scalar" else (B, T, H, Dk)
        log_alpha = -F.softplus(alpha_mu + alpha_sigma * torch.randn(*shape, **kw))
    s0 = None
    if initial_state_std is not None:
        s0 = initial_state_std * torch.randn(B, H, Dk, Dv, **kw)
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=log_alpha, initial_state=s0)


def make_workload_inputs(w, *, seed=0, device="cpu", T=None, B=None, H=None):
    """Inputs of a named chunk workload, optionally with a smaller B, T or H."""
    return make_chunk_inputs(B or w.B, T or w.T, H or w.H, w.Dk, w.Dv, w.gate,
                             w.in_dtype, seed=seed, device=device,
                             alpha_mu=w.alpha_mu, alpha_sigma=w.alpha_sigma)


def make_decode_inputs(N, H, Dk, Dv, steps, gate="scalar", in_dtype="bf16", *,
                       seed=0, device="cpu", alpha_mu=-2.0, alpha_sigma=0.5,
                       state_std=0.02):
    """Seeded inputs for `steps` consecutive decode steps of N sequences.

    Returns q, k [steps, N, H, Dk], v [steps, N, H, Dv] (input dtype),
    beta [steps, N, H], log_alpha (None / [steps, N, H] / [steps, N, H, Dk])
    and the fp32 starting state [N, H, Dk, Dv].
    """
    g = _generator(("decode", N, H, Dk, Dv, steps, gate, in_dtype, seed), device)
    dt = _DTYPES[in_dtype]
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q = _unit_rows(torch.randn(steps, N, H, Dk, **kw)).to(dt)
    k = _unit_rows(torch.randn(steps, N, H, Dk, **kw)).to(dt)
    v = torch.randn(steps, N, H, Dv, **kw).to(dt)
    beta = torch.sigmoid(torch.randn(steps, N, H, **kw))
    if gate == "none":
        log_alpha = None
    else:
        shape = (steps, N, H) if gate == "scalar" else (steps, N, H, Dk)
        log_alpha = -F.softplus(alpha_mu + alpha_sigma * torch.randn(*shape, **kw))
    state = state_std * torch.randn(N, H, Dk, Dv, **kw)
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=log_alpha, state=state)


def to_f64(t):
    """Exact float64 numpy copy of a tensor (None passes through)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
