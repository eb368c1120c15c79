"""Parity at the largest sizes: tensors past 2^31 elements (and fp32 tensors
past 4 GiB), where every chain's and chunk's base offset must be formed in
64-bit arithmetic, and head counts at the documented H * Dk bounds of the
forward kernels (one chunk's rows then span close to 4 GiB, the reach of
their 32-bit per-chunk offsets).

The kernels run over the whole tensors; the fp64 oracle checks whole
sequences of sampled chains: the first and the last, and the two on either
side of the 2^31-element (or 4 GiB) boundary.  Inputs are sliced on the
device before they reach the host.  Each test holds up to ~125 GB of device
memory (the KDA backward's workspace is ~79 GB) and releases it at its end.
"""

import gc
import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from oracle import gated_delta_backward, gated_delta_recurrence, recurrent_step
from oracle import fused as F

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


@pytest.fixture(autouse=True)
def release_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def seq(x, b, h):
    """Whole sequence of chain (b, h) of a [B, T, H, ...] tensor, fp64 on the host."""
    return None if x is None else W.to_f64(x[b:b + 1, :, h:h + 1])


def st(x, b, h):
    """State of chain (b, h) of a [B, H, Dk, Dv] tensor, fp64 on the host."""
    return None if x is None else W.to_f64(x[b:b + 1, h:h + 1])


def boundary_chains(B, H, T, D, elems):
    """(b, h) of the first and last chains and of the two chains whose rows
    meet at element offset `elems` of a [B, T, H, D] tensor (a multiple of
    T * H * D, so the boundary falls between two sequences)."""
    b = elems // (T * H * D)
    assert b * T * H * D == elems and 0 < b < B
    return [(0, 0), (b - 1, H - 1), (b, 0), (B - 1, H - 1)]


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_forward_past_2g_elements(gate):
    """q, k, v of 2.2e9 elements (8.8 GB fp32 o): B = 4200, T = 256, H = 16,
    d = 128, in the wide launch (64-column slices)."""
    B, T, H, D = 4200, 256, 16, 128
    say("forward past 2^31 elements", gate, B, T, H, D)
    assert B * T * H * D > 2 ** 31
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=5, device=DEV)
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"])
    torch.cuda.synchronize()
    for b, h in boundary_chains(B, H, T, D, 2 ** 31):
        o_ref, S_ref = gated_delta_recurrence(seq(inp["q"], b, h), seq(inp["k"], b, h),
                                              seq(inp["v"], b, h), seq(inp["beta"], b, h),
                                              seq(inp["log_alpha"], b, h))
        e_o, e_s = rel_err(seq(o, b, h), o_ref), rel_err(st(S, b, h), S_ref)
        say(f"chain ({b}, {h}): o {e_o:.2e}  S {e_s:.2e}")
        assert e_o <= TOL and e_s <= TOL


@pytest.mark.parametrize("gate,H,T,fused", [("scalar", 265000, 64, False),
                                            ("scalar", 265000, 64, True),
                                            ("channel", 554000, 32, False)])
def test_forward_at_the_head_count_bound(gate, H, T, fused):
    """H * Dk just below the documented bounds (34,000,000 without the
    per-channel gate, 71,000,000 with it) at B = 1, d = 128: a chunk's rows of
    the fp32 output (and of the per-channel log decays) span up to 4.2 GB.
    With `fused`, the SiLU output gate is read at the same offsets."""
    B, D = 1, 128
    bound = 71_000_000 if gate == "channel" else 34_000_000
    assert 0.99 * bound < H * D < bound
    say("forward at the H * Dk bound", gate, H, T, "fused gate" if fused else "")
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=6, device=DEV)
    og = None
    if fused:
        g = torch.Generator(device=DEV)
        g.manual_seed(61)
        og = torch.randn(B, T, H, D, device=DEV, generator=g).to(torch.bfloat16)
    o, S = gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                         output_final_state=False, out_gate=og)
    torch.cuda.synchronize()
    assert S is None
    for h in (0, 1, H // 2, H - 2, H - 1):
        o_ref, _ = gated_delta_recurrence(seq(inp["q"], 0, h), seq(inp["k"], 0, h),
                                          seq(inp["v"], 0, h), seq(inp["beta"], 0, h),
                                          seq(inp["log_alpha"], 0, h))
        if fused:
            o_ref = F.silu_gate(o_ref, seq(og, 0, h))
        e_o = rel_err(seq(o, 0, h), o_ref)
        say(f"head {h}: o {e_o:.2e}")
        assert e_o <= TOL


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_decode_past_2g_state_elements(gate):
    """A state of 2.15e9 fp32 elements (N = 8200, H = 16, d = 128), one step,
    bf16 q/k/v."""
    N, H, D = 8200, 16, 128
    say("decode past 2^31 state elements", gate, N, H, D)
    assert N * H * D * D > 2 ** 31
    d = W.make_decode_inputs(N, H, D, D, 1, gate, "bf16", seed=7, device=DEV)
    n0 = 2 ** 31 // (H * D * D)                  # first sequence past the boundary
    picks = [(0, 0), (n0 - 1, H - 1), (n0, 0), (N - 1, H - 1)]
    before = {p: W.to_f64(d["state"][p[0], p[1]]) for p in picks}
    la = d["log_alpha"][0] if d["log_alpha"] is not None else None
    o = gdr.recurrent_step(d["q"][0], d["k"][0], d["v"][0], d["beta"][0], la, d["state"])
    torch.cuda.synchronize()
    for n, h in picks:
        sl = lambda x: None if x is None else W.to_f64(x[n:n + 1, h:h + 1])
        o_ref, S_ref = recurrent_step(sl(d["q"][0]), sl(d["k"][0]), sl(d["v"][0]),
                                      sl(d["beta"][0]), sl(la), before[(n, h)][None, None])
        e_o = rel_err(sl(o), o_ref)
        e_s = rel_err(W.to_f64(d["state"][n:n + 1, h:h + 1]), S_ref)
        say(f"sequence ({n}, {h}): o {e_o:.2e}  S {e_s:.2e}")
        assert e_o <= 1e-5 and e_s <= 1e-5


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_backward_past_4g_bytes(gate):
    """B = 4200, T = 128, H = 16, d = 128: fp32 gradients of 1.1e9 elements
    (4.4 GB) and a workspace of 44 GB (79 GB with the per-channel gate), with
    an initial state and a final-state gradient."""
    B, T, H, D = 4200, 128, 16, 128
    say("backward past 4 GiB", gate, B, T, H, D)
    assert 4 * B * T * H * D > 2 ** 32
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=8, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(81)
    s0 = 0.3 * torch.randn(B, H, D, D, device=DEV, generator=g)
    d_o = torch.randn(B, T, H, D, device=DEV, generator=g).to(torch.bfloat16)
    d_st = 0.5 * torch.randn(B, H, D, D, device=DEV, generator=g)
    got = gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], s0, d_o,
                        d_st)
    torch.cuda.synchronize()
    for b, h in boundary_chains(B, H, T, D, 2 ** 30):
        ref = gated_delta_backward(seq(inp["q"], b, h), seq(inp["k"], b, h),
                                   seq(inp["v"], b, h), seq(inp["beta"], b, h),
                                   seq(inp["log_alpha"], b, h), st(s0, b, h), seq(d_o, b, h),
                                   st(d_st, b, h))
        errs = {n: rel_err(seq(got[n], b, h), ref[n])
                for n in ("dq", "dk", "dv", "dbeta", "dlog_alpha")}
        errs["dS0"] = rel_err(st(got["d_initial_state"], b, h), ref["dS0"])
        say(f"chain ({b}, {h}):", {k: f"{v:.1e}" for k, v in errs.items()})
        assert all(v <= TOL for v in errs.values()), errs
