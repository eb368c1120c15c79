"""GPU parity on the degenerate inputs of the delta rule, against the fp64
oracle (page "NLP——线性注意力相关总结", sections "Gated DeltaNet (GDN)" and
"Kimi Delta Attention (KDA)": the write strength b in [0, 1] and unit keys):

  beta0      b = 0 everywhere: nothing is written or erased, the state only
             decays and every output reads the decayed initial state;
  beta1      b = 1 everywhere: each erase is a full projection (the state
             loses the key's direction before the write);
  same_key   one unit key for the whole sequence with b = 1: every pair of
             tokens is coupled in the key Gram (all its strict-lower entries
             are 1 up to decay), and the last write to the key wins;
  zero_keys  k = 0 over tokens 10..59 (whole chunks and partial ones): those
             tokens neither write nor erase, while q still reads.

Forward, backward and decode, every gate, at the bars of the other parity
tests (2e-3 of RMS for bf16 q/k/v, 1e-5 for decode).  A reference that is
exactly zero (dv and dk with b = 0, whose every term carries a factor b)
must come out zero.
"""

import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from oracle import gated_delta_backward, gated_delta_recurrence, recurrent_step

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"
CASES = ("beta0", "beta1", "same_key", "zero_keys")
GATES = ("none", "scalar", "channel")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def check(got, ref, tol, name):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), name
    rms = math.sqrt(float(np.mean(ref * ref)))
    if rms == 0.0:
        err = float(np.max(np.abs(got)))
        assert err <= 1e-6, (name, err)
        return err
    err = float(np.max(np.abs(got - ref))) / rms
    assert err <= tol, (name, err)
    return err


def degenerate(inp, case):
    """The inputs of `case`, from seeded generic ones (q, k unit rows)."""
    inp = dict(inp)
    if case == "beta0":
        inp["beta"] = torch.zeros_like(inp["beta"])
    elif case == "beta1":
        inp["beta"] = torch.ones_like(inp["beta"])
    elif case == "same_key":
        inp["beta"] = torch.ones_like(inp["beta"])
        inp["k"] = inp["k"][:, :1].expand_as(inp["k"]).contiguous()
    elif case == "zero_keys":
        k = inp["k"].clone()
        k[:, 10:60] = 0
        inp["k"] = k
    else:
        raise ValueError(case)
    return inp


def make(B, T, H, D, gate, seed):
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=seed, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(700 + seed)
    inp["initial_state"] = 0.3 * torch.randn(B, H, D, D, device=DEV, generator=g)
    inp["d_o"] = torch.randn(B, T, H, D, device=DEV, generator=g).to(torch.bfloat16)
    inp["d_final_state"] = 0.5 * torch.randn(B, H, D, D, device=DEV, generator=g)
    return inp


def f64(x):
    return None if x is None else W.to_f64(x)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("D", [64, 128])
def test_forward_degenerate(case, gate, D):
    say("forward", case, gate, D)
    inp = degenerate(make(2, 100, 2, D, gate, seed=D + len(gate)), case)
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         inp["initial_state"])
    torch.cuda.synchronize()
    o_ref, S_ref = gated_delta_recurrence(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                                          f64(inp["beta"]), f64(inp["log_alpha"]),
                                          f64(inp["initial_state"]))
    e_o = check(W.to_f64(o), o_ref, TOL, "o")
    e_s = check(W.to_f64(S), S_ref, TOL, "S")
    say(f"o {e_o:.2e}  S {e_s:.2e}")


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("gate", GATES)
def test_backward_degenerate(case, gate):
    say("backward", case, gate)
    inp = degenerate(make(2, 100, 2, 128, gate, seed=11 + len(gate)), case)
    got = gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                        inp["initial_state"], inp["d_o"], inp["d_final_state"])
    torch.cuda.synchronize()
    ref = gated_delta_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["beta"]),
                               f64(inp["log_alpha"]), f64(inp["initial_state"]),
                               f64(inp["d_o"]), f64(inp["d_final_state"]))
    errs = {}
    for n, r in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"),
                 ("dlog_alpha", "dlog_alpha"), ("d_initial_state", "dS0")):
        if gate == "none" and n == "dlog_alpha":
            assert got[n] is None
            continue
        errs[n] = check(W.to_f64(got[n]), ref[r], TOL, n)
    say({k: f"{v:.1e}" for k, v in errs.items()})


@pytest.mark.parametrize("case", ["beta0", "beta1", "zero_keys"])
@pytest.mark.parametrize("gate", GATES)
def test_decode_degenerate(case, gate):
    """One decode step: b = 0 or 1, or a zero key for every sequence."""
    say("decode", case, gate)
    d = W.make_decode_inputs(4, 3, 128, 128, 1, gate, "bf16", seed=21, device=DEV)
    q, k, v, beta = d["q"][0], d["k"][0], d["v"][0], d["beta"][0]
    la = None if d["log_alpha"] is None else d["log_alpha"][0]
    if case == "beta0":
        beta = torch.zeros_like(beta)
    elif case == "beta1":
        beta = torch.ones_like(beta)
    else:
        k = torch.zeros_like(k)
    s_in = W.to_f64(d["state"])
    o = gdr.recurrent_step(q, k, v, beta, la, d["state"])
    torch.cuda.synchronize()
    o_ref, S_ref = recurrent_step(f64(q), f64(k), f64(v), f64(beta), f64(la), s_in)
    e_o = check(W.to_f64(o), o_ref, 1e-5, "o")
    e_s = check(W.to_f64(d["state"]), S_ref, 1e-5, "S")
    say(f"o {e_o:.2e}  S {e_s:.2e}")
