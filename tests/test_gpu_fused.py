"""GPU parity of the fused prologue / epilogue (gdr_chunk_fwd_ex and
gdr_recurrent_step_ex): the kernels take pre-activations (q, k not
normalised, beta logits, decay pre-activations) and an output gate, and
must match the fp64 oracle applied to the transformed inputs (oracle.fused,
pinned in test_oracle_fused.py) followed by the SiLU gate.

Bars as in test_gpu_parity: 2e-3 max|err|/RMS for bf16 q/k/v, 1e-5 for
fp32 q/k/v and for the decode step.
"""

import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from oracle import gated_delta_recurrence, recurrent_step as oracle_step
from oracle import fused as F

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
F32_TOL = 1e-5
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


np64 = W.to_f64


def raw_inputs(B, T, H, D, gate, in_dtype, seed, decay):
    """Pre-activations: q, k with row norms spread over [0.3, 3], beta
    logits, decay pre-activations, an output gate; plus a starting state."""
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, in_dtype, seed=seed, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1000)
    dt = inp["q"].dtype
    kw = dict(device=DEV, generator=g)
    for name in ("q", "k"):
        scale = 0.3 + 2.7 * torch.rand(B, T, H, 1, **kw)
        inp[name] = (inp[name].float() * scale).to(dt)
    inp["beta"] = torch.randn(B, T, H, **kw)
    if gate != "none":
        shape = (B, T, H) if gate == "scalar" else (B, T, H, D)
        # softplus: log a = -softplus(x) near -0.1; GLA: sigmoid(x)^(1/16)
        mu = -2.0 if decay == "softplus" else 1.0
        inp["log_alpha"] = mu + 0.5 * torch.randn(*shape, **kw)
    inp["out_gate"] = torch.randn(B, T, H, D, **kw).to(dt)
    inp["initial_state"] = 0.3 * torch.randn(B, H, D, D, **kw)
    return inp


def oracle_fused(inp, *, qk_l2norm, beta_sigmoid, decay, gated, erase=True):
    q, k, b, la = F.prologue(np64(inp["q"]), np64(inp["k"]), np64(inp["beta"]),
                             np64(inp["log_alpha"]), qk_l2norm=qk_l2norm,
                             beta_sigmoid=beta_sigmoid, decay=decay)
    o, S = gated_delta_recurrence(q, k, np64(inp["v"]), b, la, np64(inp["initial_state"]),
                                  erase=erase)
    if gated:
        o = F.silu_gate(o, np64(inp["out_gate"]))
    return o, S


def check(inp, tol, *, qk_l2norm=True, beta_sigmoid=True, decay=None, gated=True, erase=True,
          **kw):
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"], qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid,
                         decay=decay, out_gate=inp["out_gate"] if gated else None, erase=erase,
                         **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_fused(inp, qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid,
                                decay=decay, gated=gated, erase=erase)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gate,decay", [("none", None), ("scalar", "softplus"), ("scalar", "gla"),
                                        ("channel", "softplus"), ("channel", "gla")])
def test_chunk_fused_all(D, gate, decay):
    say("chunk fused", D, gate, decay)
    inp = raw_inputs(2, 70, 3, D, gate, "bf16", seed=D + len(gate), decay=decay)
    check(inp, BF16_TOL, decay=decay)


@pytest.mark.parametrize("opts", [dict(qk_l2norm=True, beta_sigmoid=False, gated=False),
                                  dict(qk_l2norm=False, beta_sigmoid=True, gated=False),
                                  dict(qk_l2norm=False, beta_sigmoid=False, gated=True)])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_chunk_fused_one_at_a_time(opts, gate):
    say("chunk fused subset", opts, gate)
    inp = raw_inputs(2, 45, 2, 128, gate, "bf16", seed=31, decay=None)
    if not opts["qk_l2norm"]:
        for name in ("q", "k"):   # keep the unnormalised inputs in a sane range
            x = inp[name].float()
            inp[name] = (x / x.norm(dim=-1, keepdim=True)).to(inp[name].dtype)
    if not opts["beta_sigmoid"]:
        inp["beta"] = torch.sigmoid(inp["beta"])
    if gate != "none":
        inp["log_alpha"] = -torch.nn.functional.softplus(inp["log_alpha"] - 3.0)
    check(inp, BF16_TOL, decay=None, **opts)


@pytest.mark.parametrize("gate,decay", [("scalar", "softplus"), ("channel", "gla")])
def test_chunk_fused_many_chains(gate, decay):
    # 128 chains at d = 128: the 64-column slice configurations
    say("chunk fused many chains", gate, decay)
    inp = raw_inputs(8, 50, 16, 128, gate, "bf16", seed=41, decay=decay)
    check(inp, BF16_TOL, decay=decay)


def test_chunk_fused_gla_without_erase():
    # GLA proper: per-channel sigmoid^(1/16) decay and the additive write
    say("chunk fused GLA erase-free")
    inp = raw_inputs(2, 80, 3, 128, "channel", "bf16", seed=43, decay="gla")
    check(inp, BF16_TOL, decay="gla", erase=False)


def test_chunk_fused_bf16_output():
    say("chunk fused bf16 out")
    inp = raw_inputs(2, 60, 2, 128, "scalar", "bf16", seed=47, decay="softplus")
    o, _ = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"], qk_l2norm=True, beta_sigmoid=True,
                         decay="softplus", out_gate=inp["out_gate"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, _ = oracle_fused(inp, qk_l2norm=True, beta_sigmoid=True, decay="softplus", gated=True)
    rms = math.sqrt(float(np.mean(o_ref ** 2)))
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-38))) - 8.0)
    assert np.all(np.abs(np64(o) - o_ref) <= BF16_TOL * rms + half_ulp)


@pytest.mark.parametrize("gate,decay", [("none", None), ("scalar", "softplus"),
                                        ("channel", "gla")])
@pytest.mark.parametrize("D", [16, 64])
def test_chunk_fused_fp32(gate, decay, D):
    say("chunk fused fp32", gate, decay, D)
    inp = raw_inputs(2, 40, 2, D, gate, "f32", seed=D + 5, decay=decay)
    check(inp, F32_TOL, decay=decay)


@pytest.mark.parametrize("gate,decay", [("none", None), ("scalar", "softplus"),
                                        ("channel", "gla")])
@pytest.mark.parametrize("in_dtype,D", [("bf16", 128), ("f32", 32), ("f32", 16)])
def test_recurrent_step_fused(gate, decay, in_dtype, D):
    say("recurrent_step fused", gate, decay, in_dtype, D)
    N, H, steps = 4, 3, 4
    inp = W.make_decode_inputs(N, H, D, D, steps, gate, in_dtype, seed=D + 9, device=DEV,
                               state_std=0.3)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    kw = dict(device=DEV, generator=g)
    dt = inp["q"].dtype
    q = (inp["q"].float() * (0.3 + 2.7 * torch.rand(steps, N, H, 1, **kw))).to(dt)
    k = (inp["k"].float() * (0.3 + 2.7 * torch.rand(steps, N, H, 1, **kw))).to(dt)
    beta = torch.randn(steps, N, H, **kw)
    la = None
    if gate != "none":
        shape = (steps, N, H) if gate == "scalar" else (steps, N, H, D)
        la = (-2.0 if decay == "softplus" else 1.0) + 0.5 * torch.randn(*shape, **kw)
    og = torch.randn(steps, N, H, D, **kw).to(dt)
    state = inp["state"].clone()
    S_ref = np64(state)
    for t in range(steps):
        lt = None if la is None else la[t]
        o = gdr.recurrent_step(q[t], k[t], inp["v"][t], beta[t], lt, state, qk_l2norm=True,
                               beta_sigmoid=True, decay=decay, out_gate=og[t])
        torch.cuda.synchronize()
        qq, kk, bb, ll = F.prologue(np64(q[t]), np64(k[t]), np64(beta[t]),
                                    None if lt is None else np64(lt), qk_l2norm=True,
                                    beta_sigmoid=True, decay=decay)
        o_ref, S_ref = oracle_step(qq, kk, np64(inp["v"][t]), bb, ll, S_ref)
        o_ref = F.silu_gate(o_ref, np64(og[t]))
        assert rel_err(np64(o), o_ref) <= F32_TOL, t
    assert rel_err(np64(state), S_ref) <= F32_TOL


@pytest.mark.parametrize("T", [1, 17, 33])
@pytest.mark.parametrize("D,gate,decay", [(128, "none", None), (128, "scalar", "softplus"),
                                          (64, "scalar", "gla"), (128, "channel", "softplus"),
                                          (64, "channel", "gla")])
def test_chunk_fused_ragged_tails(T, D, gate, decay):
    # a single partial chunk, and a last chunk of one token: the padded
    # tokens' transformed beta and decay (nonzero for a zero input) must not
    # leak into the state; no initial state
    say("chunk fused ragged", T, D, gate, decay)
    inp = raw_inputs(2, T, 3, D, gate, "bf16", seed=T + D, decay=decay)
    inp["initial_state"] = None
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None,
                         qk_l2norm=True, beta_sigmoid=True, decay=decay, out_gate=inp["out_gate"])
    torch.cuda.synchronize()
    q, k, b, la = F.prologue(np64(inp["q"]), np64(inp["k"]), np64(inp["beta"]),
                             np64(inp["log_alpha"]), qk_l2norm=True, beta_sigmoid=True,
                             decay=decay)
    o_ref, S_ref = gated_delta_recurrence(q, k, np64(inp["v"]), b, la, None)
    o_ref = F.silu_gate(o_ref, np64(inp["out_gate"]))
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_chunk_fused_empty_sequence_keeps_the_state():
    # T = 0 with every option: the final state is the initial state
    inp = raw_inputs(1, 1, 2, 128, "scalar", "bf16", seed=5, decay="softplus")
    empty = {k2: (v2[:, :0] if k2 in ("q", "k", "v", "beta", "log_alpha", "out_gate") else v2)
             for k2, v2 in inp.items()}
    o, S = gdr.chunk_fwd(empty["q"], empty["k"], empty["v"], empty["beta"], empty["log_alpha"],
                         inp["initial_state"], qk_l2norm=True, beta_sigmoid=True,
                         decay="softplus", out_gate=empty["out_gate"])
    torch.cuda.synchronize()
    assert o.shape[1] == 0
    assert torch.equal(S, inp["initial_state"])


@pytest.mark.parametrize("D,B,H", [(128, 2, 3), (128, 8, 16), (64, 4, 64)])
@pytest.mark.parametrize("decay", ["softplus", "gla"])
def test_chunk_fused_kda_strong_decay(D, B, H, decay):
    # per-token log decays down to about -15 after the fused transform, so
    # that some chunks take the exact in-chunk path; the decay sums are
    # shared by several waves (six prep waves at d=128 B=2 H=3, four at
    # d=128 B=8 H=16 and at d=64 with 256 chains), each flagging its own
    # channels
    say("chunk fused kda strong decay", B, H, decay)
    inp = raw_inputs(B, 70, H, D, "channel", "bf16", seed=B + H, decay=decay)
    g = torch.Generator(device=DEV)
    g.manual_seed(B * H)
    x = torch.randn(B, 70, H, D, device=DEV, generator=g)
    # softplus: log a = -softplus(x), x ~ N(3, 5); GLA: log a = -softplus(-x)/16
    inp["log_alpha"] = 3.0 + 5.0 * x if decay == "softplus" else -40.0 + 60.0 * x
    check(inp, BF16_TOL, decay=decay)
    la = F.log_decay(np64(inp["log_alpha"]), decay)
    # the case is only meaningful if some chunk crosses the exact-path bound
    sums = np.add.reduceat(la, np.arange(0, 70, 16), axis=1)
    assert sums.min() < -64.0


@pytest.mark.parametrize("gate,decay", [("scalar", "softplus"), ("channel", "softplus"),
                                        ("channel", "gla")])
def test_chunk_fused_d64_many_chains(gate, decay):
    # 256 chains at d = 64: the 64-column slice configurations (four prep
    # waves in the KDA kernel: two waves share the decay sums and the norms,
    # 16 channel pairs each)
    say("chunk fused d64 many chains", gate, decay)
    inp = raw_inputs(4, 45, 64, 64, gate, "bf16", seed=53, decay=decay)
    check(inp, BF16_TOL, decay=decay)


@pytest.mark.parametrize("gate,decay", [("scalar", "softplus"), ("channel", "gla")])
def test_chunk_fused_graph_replays_match_eager(gate, decay):
    # a fused chunk forward captured once as a HIP graph: every replay, with
    # eager work and synchronisations in between, equals the eager call bit
    # for bit
    say("chunk fused graph replay", gate, decay)
    inp = raw_inputs(2, 70, 3, 128, gate, "bf16", seed=61, decay=decay)
    o = torch.empty(2, 70, 3, 128, device=DEV)
    S = torch.empty(2, 3, 128, 128, device=DEV)
    s0 = inp["initial_state"].clone()

    def call():
        gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], s0,
                      qk_l2norm=True, beta_sigmoid=True, decay=decay,
                      out_gate=inp["out_gate"], o=o, final_state=S)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    for rep in range(3):
        s0.copy_(0.1 * (rep + 1) * torch.randn(2, 3, 128, 128, device=DEV, generator=gen))
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_s = o.clone(), S.clone()
        o.zero_()
        S.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(got_o, o) and torch.equal(got_s, S), rep
