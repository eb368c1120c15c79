"""GPU parity of the backward (gdr_chunk_bwd) against the fp64 oracle.

The oracle is oracle.backward.gated_delta_backward, the reverse sweep of the
token recurrence, itself pinned by finite differences (test_oracle_backward.py).
Both sides read the same seeded inputs; d_o is bf16 (exact for both), the
loss gradient on the final state fp32.  Every gradient tensor is compared
element by element at max |got - ref| / RMS(ref) <= 2e-3 (bf16 q/k/v with
fp32 state, as for the forward).
"""

import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from oracle import gated_delta_backward

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dS0")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def f64(t):
    return W.to_f64(t)


def make_case(B, T, H, D, gate, seed, s0=True, dst=True):
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=seed, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(1000 + seed)
    if s0:
        inp["initial_state"] = 0.3 * torch.randn(B, H, D, D, device=DEV, generator=g)
    inp["d_o"] = torch.randn(B, T, H, D, device=DEV, generator=g).to(torch.bfloat16)
    inp["d_final_state"] = (0.5 * torch.randn(B, H, D, D, device=DEV, generator=g)) if dst else None
    return inp


def run_gpu(inp, **kw):
    out = gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                        inp["initial_state"], inp["d_o"], inp["d_final_state"], **kw)
    torch.cuda.synchronize()
    out["dS0"] = out.pop("d_initial_state")
    return out


def oracle(inp, chains=None, erase=True):
    """Oracle gradients over all chains, or over a list of (b, h) chains
    (then a list of per-chain dicts)."""
    a = {k: f64(v) for k, v in inp.items()}
    if chains is None:
        return gated_delta_backward(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"],
                                    a["initial_state"], a["d_o"], a["d_final_state"],
                                    erase=erase)
    outs = []
    for b, h in chains:
        sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
        st = lambda x: None if x is None else x[b:b + 1, h:h + 1]
        outs.append(gated_delta_backward(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(a["beta"]),
                                         sl(a["log_alpha"]), st(a["initial_state"]),
                                         sl(a["d_o"]), st(a["d_final_state"]), erase=erase))
    return outs


def check_all(got, ref, gate):
    errs = {}
    for n in NAMES:
        if n == "dlog_alpha" and gate == "none":
            assert got[n] is None
            continue
        errs[n] = rel_err(f64(got[n]), ref[n])
    say("max|err|/rms", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("T", [1, 17, 32, 33, 100])
def test_backward_small_batch(D, gate, T):
    say("bwd", D, gate, T)
    inp = make_case(2, T, 2, D, gate, seed=T + D)
    check_all(run_gpu(inp), oracle(inp), gate)


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_backward_zero_initial_state_and_no_state_gradient(gate):
    say("bwd no S0 / no dS_T", gate)
    inp = make_case(2, 45, 3, 128, gate, seed=5, s0=False, dst=False)
    check_all(run_gpu(inp), oracle(inp), gate)


@pytest.mark.parametrize("D,B,H", [(128, 4, 32), (64, 8, 32)])
def test_backward_many_chains(D, B, H):
    """The wide launch (64-column slices of the state) of the two passes."""
    say("bwd many chains", D, B, H)
    inp = make_case(B, 40, H, D, "scalar", seed=9)
    check_all(run_gpu(inp), oracle(inp), "scalar")


def test_backward_decay_regimes():
    """Strong decays (g down to about -60 within a chunk) and a hard reset."""
    say("bwd decay regimes")
    inp = make_case(2, 70, 2, 128, "scalar", seed=21)
    la = inp["log_alpha"].clone()
    la[0] = -2.0          # strong, steady
    la[1, 30] = -50.0     # a hard reset mid-chunk
    inp["log_alpha"] = la
    check_all(run_gpu(inp), oracle(inp), "scalar")


def test_backward_deterministic_and_workspace_reuse():
    say("bwd determinism")
    inp = make_case(2, 77, 2, 128, "scalar", seed=31)
    need = gdr.chunk_bwd_workspace_bytes(inp["q"], inp["log_alpha"])
    ws = torch.full((need,), 0xAB, device=DEV, dtype=torch.uint8)   # stale contents are ignored
    a = run_gpu(inp, workspace=ws)
    b = run_gpu(inp, workspace=ws)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_backward_without_initial_state_gradient():
    say("bwd want_d_initial_state=False")
    inp = make_case(1, 20, 2, 64, "scalar", seed=2)
    out = gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                        inp["initial_state"], inp["d_o"], inp["d_final_state"],
                        want_d_initial_state=False)
    torch.cuda.synchronize()
    assert out["d_initial_state"] is None
    ref = oracle(inp)
    assert rel_err(f64(out["dq"]), ref["dq"]) <= TOL
    # a d_initial_state buffer in `out` is refused rather than written unchecked
    buf = {n: torch.empty_like(t) for n, t in out.items() if t is not None}
    buf["d_initial_state"] = torch.empty(1, device=DEV)
    with pytest.raises(ValueError):
        gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                      inp["initial_state"], inp["d_o"], inp["d_final_state"],
                      want_d_initial_state=False, out=buf)


def test_backward_headline_shape_sampled_chains():
    """The Gated DeltaNet layer shape B=8, H=16, T=4096, d=128 in the launch
    the benchmark times; the oracle checks three chains in full (every token's
    gradients and dS_0)."""
    w = W.HEADLINE
    say("bwd", w.name, "sampled")
    inp = make_case(w.B, w.T, w.H, w.Dk, w.gate, seed=0, s0=False)
    got = run_gpu(inp)
    chains = [(0, 0), (3, 7), (7, 15)]
    for (b, h), ref in zip(chains, oracle(inp, chains)):
        sub = {n: None if got[n] is None else
               (got[n][b:b + 1, h:h + 1] if n == "dS0" else got[n][b:b + 1, :, h:h + 1])
               for n in NAMES}
        check_all(sub, ref, w.gate)


# The erase-free forms (S_t = a_t S_{t-1} + b_t k_t v_t^T): linear attention
# without a gate, the Mamba-2 / SSD decay with the per-head gate.


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("T", [1, 33, 100])
def test_backward_erase_free(D, gate, T):
    say("bwd erase-free", D, gate, T)
    inp = make_case(2, T, 2, D, gate, seed=3 * T + D)
    check_all(run_gpu(inp, erase=False), oracle(inp, erase=False), gate)


def test_backward_erase_free_many_chains_and_strong_decay():
    """The wide launch, a strong steady decay and a hard reset mid-chunk."""
    say("bwd erase-free many chains")
    inp = make_case(4, 70, 32, 128, "scalar", seed=41, s0=True, dst=True)
    la = inp["log_alpha"].clone()
    la[0] = -2.0
    la[1, 30] = -50.0
    inp["log_alpha"] = la
    check_all(run_gpu(inp, erase=False), oracle(inp, erase=False), "scalar")


def test_backward_erase_free_differs_from_the_erase_form():
    """The erase flag reaches the kernels: the two forms give different dk."""
    say("bwd erase flag")
    inp = make_case(1, 40, 2, 64, "scalar", seed=7)
    a = run_gpu(inp, erase=False)
    b = run_gpu(inp, erase=True)
    ref = oracle(inp, erase=True)
    assert rel_err(f64(b["dk"]), ref["dk"]) <= TOL
    assert rel_err(f64(a["dk"]), ref["dk"]) > 0.05


# The per-channel gate (KDA; without the erase term GLA's decay): 16-token
# chunks through the KDA kernel's recompute and reverse passes and its own
# gradient kernel.


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 16, 17, 40, 100])
def test_backward_kda(D, T):
    say("bwd kda", D, T)
    inp = make_case(2, T, 2, D, "channel", seed=5 * T + D)
    check_all(run_gpu(inp), oracle(inp), "channel")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 33, 100])
def test_backward_kda_erase_free(D, T):
    say("bwd gla decay", D, T)
    inp = make_case(2, T, 2, D, "channel", seed=7 * T + D)
    check_all(run_gpu(inp, erase=False), oracle(inp, erase=False), "channel")


@pytest.mark.parametrize("erase", [True, False])
def test_backward_kda_exact_path(erase):
    """Chunks where some channel's in-chunk log decay falls below -64 (and a
    hard reset of one channel), which take the directly formed decays."""
    say("bwd kda exact path", erase)
    inp = make_case(2, 70, 2, 128, "channel", seed=23)
    la = inp["log_alpha"].clone()
    la[0, 16:32, :, :8] = -6.0     # a whole chunk 96 below on eight channels
    la[1, 40, 1, 5] = -80.0        # one channel reset mid-chunk
    la[1, 50:60, 0, 100:] = -9.0   # part of a chunk, strong
    inp["log_alpha"] = la
    check_all(run_gpu(inp, erase=erase), oracle(inp, erase=erase), "channel")


@pytest.mark.parametrize("D,B,H", [(128, 2, 32), (128, 4, 32), (64, 8, 32)])
def test_backward_kda_many_chains(D, B, H):
    """Both slice widths of the passes (32 columns below 128 chains at d = 128,
    64 above), sampled chains against the oracle."""
    say("bwd kda many chains", D, B, H)
    inp = make_case(B, 37, H, D, "channel", seed=11)
    got = run_gpu(inp)
    chains = [(0, 0), (B - 1, H - 1), (B // 2, 7)]
    refs = oracle(inp, chains=chains)
    for (b, h), ref in zip(chains, refs):
        sub = {n: (got[n][b:b + 1, :, h:h + 1] if n != "dS0" else got[n][b:b + 1, h:h + 1])
               for n in NAMES}
        check_all(sub, ref, "channel")


def test_backward_kda_full_shape_sampled_chains():
    """The KDA layer shape B=2, H=32, T=8192, d=128 with the workload's own
    decay distribution, in the launch the benchmark times (32-column slices);
    the oracle checks two chains in full, every token's gradients and dS_0."""
    w = W.by_name("kda_bf16_b2h32t8192")
    say("bwd", w.name, "sampled")
    inp = W.make_workload_inputs(w, seed=0, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    inp["d_o"] = torch.randn(w.B, w.T, w.H, w.Dv, device=DEV, generator=g).to(torch.bfloat16)
    inp["d_final_state"] = 0.5 * torch.randn(w.B, w.H, w.Dk, w.Dv, device=DEV, generator=g)
    got = run_gpu(inp)
    chains = [(0, 0), (1, 31)]
    for (b, h), ref in zip(chains, oracle(inp, chains)):
        sub = {n: (got[n][b:b + 1, h:h + 1] if n == "dS0" else got[n][b:b + 1, :, h:h + 1])
               for n in NAMES}
        check_all(sub, ref, "channel")


def test_backward_kda_no_state_gradients_and_determinism():
    say("bwd kda no S0 / no dS_T, determinism")
    inp = make_case(1, 50, 3, 64, "channel", seed=3, s0=False, dst=False)
    a = run_gpu(inp)
    check_all(a, oracle(inp), "channel")
    b = run_gpu(inp)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
