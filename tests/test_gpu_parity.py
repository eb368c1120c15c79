"""GPU parity: the HIP kernels behind the C ABI against the fp64 oracle.

Both sides read the same seeded inputs (the oracle an exact fp64 upcast of
the rounded values).  Error measure: max |got - ref| / RMS(ref) over every
compared element, for the outputs and for the final state.  Bars:
  * bf16 q/k/v with fp32 state and fp32 output: 2e-3
  * fp32 q/k/v (and every decode step, which is plain fp32 arithmetic): 1e-5
  * bf16 output: |got - ref| <= 2e-3 * RMS(ref) + half a bf16 ulp of ref
"""

import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from oracle import gated_delta_recurrence, recurrent_step as oracle_step

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


def bf16_half_ulp(x):
    ax = np.maximum(np.abs(x), 1e-38)
    return np.exp2(np.floor(np.log2(ax)) - 8.0)


def np64(t):
    return W.to_f64(t)


def oracle_on(inp, chains=None):
    """Oracle over all chains, or over a list of (b, h) chains."""
    q, k, v, beta = (np64(inp[n]) for n in ("q", "k", "v", "beta"))
    la = np64(inp["log_alpha"])
    s0 = np64(inp["initial_state"])
    if chains is None:
        return gated_delta_recurrence(q, k, v, beta, la, s0)
    outs = []
    for b, h in chains:
        sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
        o, S = gated_delta_recurrence(sl(q), sl(k), sl(v), sl(beta), sl(la),
                                      None if s0 is None else s0[b:b + 1, h:h + 1])
        outs.append((o[0, :, 0], S[0, 0]))
    return outs


def run_chunk(inp, **kw):
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"], **kw)
    torch.cuda.synchronize()
    return o, S


def with_state(inp, std=0.3, seed=99):
    B, T, H, Dk = inp["q"].shape
    Dv = inp["v"].shape[-1]
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    inp = dict(inp)
    inp["initial_state"] = std * torch.randn(B, H, Dk, Dv, device=DEV, generator=g)
    return inp


def test_library_is_the_hip_build():
    assert gdr.abi_version() == gdr._abi.ABI_VERSION == 4
    assert gdr.library_loaded()


# ---------------------------------------------------------------------------
# decode step


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_recurrent_step_parity(D, gate, in_dtype):
    say("recurrent_step", D, gate, in_dtype)
    N, H, steps = 5, 3, 6
    inp = W.make_decode_inputs(N, H, D, D, steps, gate, in_dtype, seed=D, device=DEV,
                               state_std=0.3)
    state = inp["state"].clone()
    S_ref = np64(state)
    for t in range(steps):
        la = None if inp["log_alpha"] is None else inp["log_alpha"][t]
        o = gdr.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["beta"][t], la, state)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_step(np64(inp["q"][t]), np64(inp["k"][t]), np64(inp["v"][t]),
                                   np64(inp["beta"][t]), None if la is None else np64(la), S_ref)
        assert rel_err(np64(o), o_ref) <= F32_TOL, t
    assert rel_err(np64(state), S_ref) <= F32_TOL


def test_recurrent_step_bf16_output():
    say("recurrent_step bf16 out")
    inp = W.make_decode_inputs(7, 4, 128, 128, 1, "scalar", "bf16", seed=3, device=DEV)
    state = inp["state"].clone()
    o = gdr.recurrent_step(inp["q"][0], inp["k"][0], inp["v"][0], inp["beta"][0],
                           inp["log_alpha"][0], state, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, _ = oracle_step(np64(inp["q"][0]), np64(inp["k"][0]), np64(inp["v"][0]),
                           np64(inp["beta"][0]), np64(inp["log_alpha"][0]), np64(inp["state"]))
    rms = math.sqrt(float(np.mean(o_ref ** 2)))
    assert np.all(np.abs(np64(o) - o_ref) <= BF16_TOL * rms + bf16_half_ulp(o_ref))


# ---------------------------------------------------------------------------
# chunk forward, plain-fp32 path (small heads)


def test_tiny_fp32_workload():
    w = W.WORKLOADS[0]
    say("workload", w.name)
    inp = W.make_workload_inputs(w, seed=0, device=DEV)
    o, S = run_chunk(inp, chunk=w.chunk)
    o_ref, S_ref = oracle_on(inp)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= F32_TOL and es <= F32_TOL


@pytest.mark.parametrize("D,chunk", [(16, 16), (16, 0), (32, 32), (64, 64), (64, 16)])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_chunk_small_fp32(D, chunk, gate, T):
    say("chunk small f32", D, chunk, gate, T)
    inp = with_state(W.make_chunk_inputs(2, T, 2, D, D, gate, "f32", seed=T, device=DEV))
    o, S = run_chunk(inp, chunk=chunk)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= F32_TOL
    assert rel_err(np64(S), S_ref) <= F32_TOL


@pytest.mark.parametrize("chunk", [0, 64])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_chunk_fp32_d128(chunk, gate, T):
    """fp32 q/k/v at d = 128 (16-token chunks whatever `chunk` asks), with an
    initial state and ragged tails, to the fp32 bar."""
    say("chunk f32 d128", chunk, gate, T)
    inp = with_state(W.make_chunk_inputs(2, T, 3, 128, 128, gate, "f32", seed=T + 1,
                                         device=DEV))
    o, S = run_chunk(inp, chunk=chunk)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= F32_TOL
    assert rel_err(np64(S), S_ref) <= F32_TOL


def test_chunk_fp32_d128_erase_free_and_fused():
    say("chunk f32 d128 erase-free / fused")
    from oracle import fused as F
    inp = with_state(W.make_chunk_inputs(2, 45, 2, 128, 128, "channel", "f32", seed=8,
                                         device=DEV))
    o, S = run_chunk(inp, erase=False)
    a = {k: np64(v) for k, v in inp.items()}
    o_ref, S_ref = gated_delta_recurrence(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"],
                                          a["initial_state"], erase=False)
    assert rel_err(np64(o), o_ref) <= F32_TOL and rel_err(np64(S), S_ref) <= F32_TOL
    g = torch.Generator(device=DEV)
    g.manual_seed(4)
    xb = torch.randn(2, 45, 2, device=DEV, generator=g)
    xd = -3.0 + torch.randn(2, 45, 2, 128, device=DEV, generator=g)
    gate = torch.randn(2, 45, 2, 128, device=DEV, generator=g)
    q2 = inp["q"] * 3.0
    o, S = gdr.chunk_fwd(q2, inp["k"], inp["v"], xb, xd, inp["initial_state"], qk_l2norm=True,
                         beta_sigmoid=True, decay="softplus", out_gate=gate)
    torch.cuda.synchronize()
    qf, kf, bf, lf = F.prologue(np64(q2), a["k"], np64(xb), np64(xd), qk_l2norm=True,
                                beta_sigmoid=True, decay="softplus")
    o_ref, S_ref = gated_delta_recurrence(qf, kf, a["v"], bf, lf, a["initial_state"])
    o_ref = F.silu_gate(o_ref, np64(gate))
    assert rel_err(np64(o), o_ref) <= F32_TOL and rel_err(np64(S), S_ref) <= F32_TOL


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_chunk_small_bf16_inputs(gate):
    say("chunk small bf16", gate)
    inp = with_state(W.make_chunk_inputs(3, 77, 2, 32, 32, gate, "bf16", seed=5, device=DEV))
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= F32_TOL
    assert rel_err(np64(S), S_ref) <= F32_TOL


def test_decode_graph_replays_match_eager():
    # the decode loop captured once as a HIP graph: every replay, with eager
    # work and synchronisations in between, equals the eager loop bit for bit
    say("decode graph replay")
    N, H, D, steps = 8, 4, 128, 6
    inp = W.make_decode_inputs(N, H, D, D, steps, "scalar", "bf16", seed=21, device=DEV)
    state = inp["state"].clone()
    o = torch.empty(steps, N, H, D, device=DEV)

    def one_pass():
        for t in range(steps):
            gdr.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["beta"][t],
                               inp["log_alpha"][t], state, o=o[t])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    for rep in range(3):
        start = 0.02 * (rep + 1) * torch.randn(N, H, D, D, device=DEV, generator=gen)
        state.copy_(start)
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_s = o.clone(), state.clone()
        state.copy_(start)
        one_pass()
        torch.cuda.synchronize()
        assert torch.equal(got_o, o) and torch.equal(got_s, state), rep


# ---------------------------------------------------------------------------
# chunk forward, MFMA path (bf16 q/k/v, Dk = Dv in {64, 128})


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
@pytest.mark.parametrize("s0", [False, True])
def test_chunk_mfma_small_batch(D, gate, T, s0):
    say("chunk mfma", D, gate, T, s0)
    inp = W.make_chunk_inputs(2, T, 3, D, D, gate, "bf16", seed=T + D, device=DEV)
    if s0:
        inp = with_state(inp)
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_chunk_mfma_many_chains(gate):
    # 128 chains: the 64-column slice configuration, 8-way XCD chain mapping
    say("chunk mfma many chains", gate)
    inp = with_state(W.make_chunk_inputs(8, 130, 16, 128, 128, gate, "bf16", seed=4, device=DEV))
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= BF16_TOL
    assert rel_err(np64(S), S_ref) <= BF16_TOL


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_chunk_mfma_d64_many_chains(gate):
    # 256 chains at d = 64: the 64-column (whole-width) slice configuration
    say("chunk mfma d64 many chains", gate)
    inp = with_state(W.make_chunk_inputs(4, 70, 64, 64, 64, gate, "bf16", seed=6, device=DEV))
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= BF16_TOL
    assert rel_err(np64(S), S_ref) <= BF16_TOL


def test_chunk_mfma_bf16_output():
    say("chunk mfma bf16 out")
    inp = W.make_chunk_inputs(2, 150, 2, 128, 128, "scalar", "bf16", seed=8, device=DEV)
    o, _ = run_chunk(inp, out_dtype=torch.bfloat16)
    o_ref, _ = oracle_on(inp)
    rms = math.sqrt(float(np.mean(o_ref ** 2)))
    assert np.all(np.abs(np64(o) - o_ref) <= BF16_TOL * rms + bf16_half_ulp(o_ref))


def test_chunk_mfma_deterministic():
    say("chunk mfma determinism")
    inp = with_state(W.make_chunk_inputs(4, 300, 8, 128, 128, "scalar", "bf16", seed=2, device=DEV))
    o1, S1 = run_chunk(inp)
    o2, S2 = run_chunk(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ---------------------------------------------------------------------------
# chunk forward, per-channel decay (KDA), MFMA path (bf16, Dk = Dv in {64, 128})


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 100])
@pytest.mark.parametrize("s0", [False, True])
def test_chunk_kda_small_batch(D, T, s0):
    say("chunk kda", D, T, s0)
    inp = W.make_chunk_inputs(2, T, 3, D, D, "channel", "bf16", seed=3 * T + D, device=DEV)
    if s0:
        inp = with_state(inp)
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("alpha_mu,alpha_sigma", [(-3.0, 1.0), (1.0, 1.0), (3.0, 2.5)])
def test_chunk_kda_decay_range(alpha_mu, alpha_sigma):
    # from weak decay to per-step log decays beyond -10 on some channels,
    # which sends those chunks down the exact (unfactored) in-chunk path
    say("chunk kda decay range", alpha_mu, alpha_sigma)
    inp = with_state(W.make_chunk_inputs(2, 97, 4, 128, 128, "channel", "bf16", seed=11,
                                         device=DEV, alpha_mu=alpha_mu, alpha_sigma=alpha_sigma))
    o, S = run_chunk(inp)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_on(inp)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("D,B,H", [(128, 8, 16), (64, 2, 3), (64, 4, 64)])
def test_chunk_kda_exact_path_configs(D, B, H):
    # strong per-channel decay (some chunks take the exact in-chunk path) in
    # the other launch configurations: 64-column slices with four prep waves
    # (128 chains at d = 128, 256 at d = 64) and d = 64 with 32-column slices
    say("chunk kda exact path", D, B, H)
    inp = with_state(W.make_chunk_inputs(B, 70, H, D, D, "channel", "bf16", seed=13 + D,
                                         device=DEV, alpha_mu=3.0, alpha_sigma=2.5))
    o, S = run_chunk(inp)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_on(inp)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_chunk_kda_many_chains():
    # 128 chains: the 64-column slice configuration
    say("chunk kda many chains")
    inp = with_state(W.make_chunk_inputs(8, 70, 16, 128, 128, "channel", "bf16", seed=5,
                                         device=DEV))
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= BF16_TOL
    assert rel_err(np64(S), S_ref) <= BF16_TOL


def test_chunk_kda_d64_many_chains():
    # 256 chains at d = 64: the whole-width slice configuration
    say("chunk kda d64 many chains")
    inp = with_state(W.make_chunk_inputs(4, 70, 64, 64, 64, "channel", "bf16", seed=7,
                                         device=DEV))
    o, S = run_chunk(inp)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(o), o_ref) <= BF16_TOL
    assert rel_err(np64(S), S_ref) <= BF16_TOL


def test_chunk_kda_bf16_output_and_determinism():
    say("chunk kda bf16 out")
    inp = with_state(W.make_chunk_inputs(2, 150, 2, 128, 128, "channel", "bf16", seed=9,
                                         device=DEV))
    o, _ = run_chunk(inp, out_dtype=torch.bfloat16)
    o2, _ = run_chunk(inp, out_dtype=torch.bfloat16)
    assert torch.equal(o, o2)
    o_ref, _ = oracle_on(inp)
    rms = math.sqrt(float(np.mean(o_ref ** 2)))
    assert np.all(np.abs(np64(o) - o_ref) <= BF16_TOL * rms + bf16_half_ulp(o_ref))


# ---------------------------------------------------------------------------
# state carry and special cases


@pytest.mark.parametrize("D,in_dtype,gate", [(128, "bf16", "scalar"), (32, "f32", "scalar"),
                                             (128, "bf16", "channel")])
def test_state_passing_split_and_decode(D, in_dtype, gate):
    say("state passing", D, in_dtype, gate)
    T = 150
    tol = BF16_TOL if in_dtype == "bf16" else F32_TOL
    inp = with_state(W.make_chunk_inputs(2, T, 3, D, D, gate, in_dtype, seed=6, device=DEV))
    o_all, S_all = run_chunk(inp)
    # split at 70: run [0, 70) then [70, T) from the carried state
    cut = lambda x, a, b: x[:, a:b].contiguous()
    first = {n: cut(inp[n], 0, 70) for n in ("q", "k", "v", "beta", "log_alpha")}
    first["initial_state"] = inp["initial_state"]
    o1, S1 = run_chunk(first)
    second = {n: cut(inp[n], 70, T) for n in ("q", "k", "v", "beta", "log_alpha")}
    second["initial_state"] = S1
    o2, S2 = run_chunk(second)
    o_ref, S_ref = oracle_on(inp)
    assert rel_err(np64(torch.cat([o1, o2], 1)), o_ref) <= tol
    assert rel_err(np64(S2), S_ref) <= tol
    # chunk_fwd over T-1 tokens, then one decode step on the last token
    head = {n: cut(inp[n], 0, T - 1) for n in ("q", "k", "v", "beta", "log_alpha")}
    head["initial_state"] = inp["initial_state"]
    _, S_head = run_chunk(head)
    state = S_head.clone()
    o_last = gdr.recurrent_step(inp["q"][:, T - 1].contiguous(), inp["k"][:, T - 1].contiguous(),
                                inp["v"][:, T - 1].contiguous(), inp["beta"][:, T - 1].contiguous(),
                                inp["log_alpha"][:, T - 1].contiguous(), state)
    torch.cuda.synchronize()
    assert rel_err(np64(o_last), o_ref[:, T - 1]) <= tol
    assert rel_err(np64(state), S_ref) <= tol


def test_in_place_state_carry():
    say("in-place carry")
    inp = with_state(W.make_chunk_inputs(2, 90, 2, 128, 128, "scalar", "bf16", seed=7, device=DEV))
    S0 = inp["initial_state"].clone()
    o_ref, S_ref = oracle_on(inp)
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"], final_state=inp["initial_state"])
    torch.cuda.synchronize()
    assert S.data_ptr() == inp["initial_state"].data_ptr()
    assert rel_err(np64(S), S_ref) <= BF16_TOL
    assert rel_err(np64(o), o_ref) <= BF16_TOL
    assert not torch.equal(S, S0)


def test_empty_sequence_passes_state_through():
    say("T = 0")
    B, H, D = 2, 3, 128
    q = torch.empty(B, 0, H, D, device=DEV, dtype=torch.bfloat16)
    beta = torch.empty(B, 0, H, device=DEV)
    la = torch.empty(B, 0, H, device=DEV)
    S0 = torch.randn(B, H, D, D, device=DEV)
    o, S = gdr.chunk_fwd(q, q, q, beta, la, S0)
    torch.cuda.synchronize()
    assert o.shape == (B, 0, H, D) and torch.equal(S, S0)
    o, S = gdr.chunk_fwd(q, q, q, beta, la, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


@pytest.mark.parametrize("D,in_dtype,gate", [(128, "bf16", "scalar"), (16, "f32", "scalar"),
                                             (128, "bf16", "channel")])
def test_hard_reset_gate_has_no_nan(D, in_dtype, gate):
    say("hard reset", D, in_dtype, gate)
    inp = with_state(W.make_chunk_inputs(1, 80, 2, D, D, gate, in_dtype, seed=1, device=DEV))
    inp["log_alpha"] = torch.full_like(inp["log_alpha"], -50.0)
    o, S = run_chunk(inp)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_on(inp)
    tol = BF16_TOL if in_dtype == "bf16" else F32_TOL
    assert rel_err(np64(o), o_ref) <= tol


def _chunk_decays(B, T, H, per_token, seed):
    """log a with a per-chunk decay regime: chunk c of every chain draws its
    mean per-token log decay from `per_token`, and each token varies by up to
    50% around it."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    nch = (T + 31) // 32
    pick = torch.randint(0, len(per_token), (B, nch, H), device=DEV, generator=g)
    mean = torch.tensor(per_token, device=DEV, dtype=torch.float32)[pick]
    mean = mean.repeat_interleave(32, dim=1)[:, :T]
    return mean * (0.5 + torch.rand(B, T, H, device=DEV, generator=g))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("regime", ["steady", "mixed", "hard_then_soft"])
def test_chunk_scalar_decay_regimes(D, regime):
    # long runs of decay (the total log decay of a chain reaches several
    # hundred), chunks whose own decay is beyond e^-40, and mixtures of both
    say("chunk scalar decay regime", D, regime)
    B, T, H = 2, 613, 4
    inp = with_state(W.make_chunk_inputs(B, T, H, D, D, "scalar", "bf16", seed=D + 7, device=DEV))
    if regime == "steady":
        la = _chunk_decays(B, T, H, [-0.6], seed=3)
    elif regime == "mixed":
        la = _chunk_decays(B, T, H, [-0.01, -0.3, -0.9, -2.5], seed=4)
    else:
        la = _chunk_decays(B, T, H, [-0.02], seed=5)
        la[:, :96] = -3.0
    inp["log_alpha"] = la.contiguous()
    o, S = run_chunk(inp)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_on(inp)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= BF16_TOL and es <= BF16_TOL


# ---------------------------------------------------------------------------
# the named workloads at full size, outputs of sampled chains against the
# oracle (every token and value column of each sampled chain)


def _sampled(w, chains, seed=0):
    say("workload", w.name, "chains", chains)
    inp = W.make_workload_inputs(w, seed=seed, device=DEV)
    o, S = run_chunk(inp, chunk=w.chunk)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    refs = oracle_on(inp, chains)
    for (b, h), (o_ref, S_ref) in zip(chains, refs):
        eo, es = rel_err(np64(o[b, :, h]), o_ref), rel_err(np64(S[b, h]), S_ref)
        say("chain", (b, h), "max|err|/rms o", eo, "state", es)
        assert eo <= BF16_TOL and es <= BF16_TOL, (b, h)


def test_workload_deltanet_b4h8_sampled():
    _sampled(W.WORKLOADS[1], [(0, 0), (3, 7), (2, 5)])


def test_workload_gdn_b4h8_sampled():
    _sampled(W.GDN_B4H8, [(0, 0), (1, 6), (3, 7)])


def test_workload_gdn_b8h16_sampled():
    _sampled(W.HEADLINE, [(0, 0), (5, 9), (7, 15)])


def test_workload_kda_b2h32_sampled():
    _sampled(W.by_name("kda_bf16_b2h32t8192"), [(0, 0), (1, 17), (1, 31)])
