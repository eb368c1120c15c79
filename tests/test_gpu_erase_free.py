"""GPU parity of the erase-free variant (gate | GDR_NO_ERASE): the additive
write S_t = a_t S_{t-1} + b_t k_t v_t^T (linear attention with no gate, the
Mamba-2 / SSD decay with the scalar gate, GLA's with the channel gate), run
by the same kernels without the triangular solve, against the fp64 oracle's
erase=False recurrence (itself pinned to the additive closed forms).

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


def with_state(inp, std=0.3, seed=98):
    B, T, H, Dk = inp["q"].shape
    Dv = inp["v"].shape[-1]
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    inp = dict(inp)
    inp["initial_state"] = std * torch.randn(B, H, Dk, Dv, device=DEV, generator=g)
    return inp


def run_and_check(inp, tol, **kw):
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"], erase=False, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    s0 = inp["initial_state"]
    o_ref, S_ref = gated_delta_recurrence(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]),
                                          np64(inp["beta"]), np64(inp["log_alpha"]),
                                          None if s0 is None else np64(s0), erase=False)
    eo, es = rel_err(np64(o), o_ref), rel_err(np64(S), S_ref)
    say("max|err|/rms o", eo, "state", es)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("T", [1, 33, 130])
def test_chunk_erase_free_mfma(D, gate, T):
    # bf16 q/k/v: the MFMA kernels (scalar-gate kernel for none/scalar, the
    # per-channel kernel for channel), 32-column slices
    say("chunk erase-free", D, gate, T)
    inp = with_state(W.make_chunk_inputs(2, T, 3, D, D, gate, "bf16", seed=T + 2 * D, device=DEV))
    run_and_check(inp, BF16_TOL)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_chunk_erase_free_many_chains(gate):
    # 128 chains at d = 128: the 64-column slice configurations
    say("chunk erase-free many chains", gate)
    inp = with_state(W.make_chunk_inputs(8, 70, 16, 128, 128, gate, "bf16", seed=21, device=DEV))
    run_and_check(inp, BF16_TOL)


def test_chunk_erase_free_channel_exact_path():
    # strong per-channel decay: chunks on the exact in-chunk path
    say("chunk erase-free channel exact path")
    inp = with_state(W.make_chunk_inputs(2, 97, 4, 128, 128, "channel", "bf16", seed=23,
                                         device=DEV, alpha_mu=3.0, alpha_sigma=2.5))
    run_and_check(inp, BF16_TOL)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("D", [16, 64])
def test_chunk_erase_free_fp32(gate, D):
    # fp32 q/k/v: the fp32 kernel
    say("chunk erase-free fp32", gate, D)
    inp = with_state(W.make_chunk_inputs(2, 75, 2, D, D, gate, "f32", seed=D + 1, device=DEV))
    run_and_check(inp, F32_TOL)


def test_chunk_erase_free_bf16_output():
    say("chunk erase-free bf16 out")
    inp = with_state(W.make_chunk_inputs(2, 90, 2, 128, 128, "scalar", "bf16", seed=29, device=DEV))
    o, _ = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"], erase=False, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, _ = gated_delta_recurrence(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]),
                                      np64(inp["beta"]), np64(inp["log_alpha"]),
                                      np64(inp["initial_state"]), erase=False)
    rms = math.sqrt(float(np.mean(o_ref ** 2)))
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-38))) - 8.0)
    assert np.all(np.abs(np64(o) - o_ref) <= BF16_TOL * rms + half_ulp)


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_recurrent_step_erase_free(D, gate):
    say("recurrent_step erase-free", D, gate)
    N, H, steps = 4, 3, 5
    inp = W.make_decode_inputs(N, H, D, D, steps, gate, "bf16", seed=D + 7, device=DEV,
                               state_std=0.3)
    state = inp["state"].clone()
    S_ref = np64(state)
    for t in range(steps):
        la = None if inp["log_alpha"] is None else inp["log_alpha"][t]
        o = gdr.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["beta"][t], la, state,
                               erase=False)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_step(np64(inp["q"][t]), np64(inp["k"][t]), np64(inp["v"][t]),
                                   np64(inp["beta"][t]), None if la is None else np64(la), S_ref,
                                   erase=False)
        assert rel_err(np64(o), o_ref) <= F32_TOL, t
    assert rel_err(np64(state), S_ref) <= F32_TOL


def test_workload_additive_sampled():
    # the headline shape with the erase-free scalar gate, sampled chains
    w = W.HEADLINE
    say("workload erase-free", w.name)
    inp = W.make_workload_inputs(w, seed=0, device=DEV)
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None,
                         chunk=w.chunk, erase=False)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    for b, h in [(0, 0), (6, 11)]:
        sl = lambda x: np64(x[b:b + 1, :, h:h + 1])
        o_ref, S_ref = gated_delta_recurrence(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                              sl(inp["beta"]), sl(inp["log_alpha"]), erase=False)
        eo = rel_err(np64(o[b, :, h]), o_ref[0, :, 0])
        es = rel_err(np64(S[b, h]), S_ref[0, 0])
        say("chain", (b, h), "max|err|/rms o", eo, "state", es)
        assert eo <= BF16_TOL and es <= BF16_TOL
