"""GPU parity of the training pair: gdr_chunk_fwd_train (the forward that also
fills the backward's workspace) and gdr_chunk_bwd_saved (the backward that
reads it instead of recomputing the forward).

The forward's o and S_T are compared with the fp64 oracle recurrence at the
2e-3 bar of the bf16 path, and with chunk_fwd; the saved backward's gradients
with the fp64 oracle's reverse sweep at 2e-3 and with the backward that
recomputes the forward itself, which computes the same stored values.
"""

import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from oracle import gated_delta_backward, gated_delta_recurrence

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "d_initial_state")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = W.to_f64(got) if torch.is_tensor(got) else np.asarray(got, np.float64)
    ref = W.to_f64(ref) if torch.is_tensor(ref) else np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place of x (8 significant bits)."""
    ax = np.maximum(np.abs(x), 1e-38)
    return np.exp2(np.floor(np.log2(ax)) - 8.0)


def make_case(B, T, H, D, gate, seed):
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=seed, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(500 + seed)
    inp["initial_state"] = 0.3 * torch.randn(B, H, D, D, device=DEV, generator=g)
    inp["d_o"] = torch.randn(B, T, H, D, device=DEV, generator=g).to(torch.bfloat16)
    inp["d_final_state"] = 0.5 * torch.randn(B, H, D, D, device=DEV, generator=g)
    return inp


def args(inp):
    return (inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["initial_state"])


def oracle_fwd(inp, erase):
    f = lambda x: None if x is None else W.to_f64(x)
    return gated_delta_recurrence(*(f(x) for x in args(inp)), erase=erase)


def oracle_bwd(inp, erase):
    f = lambda x: None if x is None else W.to_f64(x)
    return gated_delta_backward(*(f(x) for x in args(inp)), f(inp["d_o"]),
                                f(inp["d_final_state"]), erase=erase)


@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("D,T", [(64, 1), (128, 40), (64, 100), (128, 100)])
def test_train_pair_matches_the_oracle(D, T, gate, erase):
    say("train pair", D, T, gate, erase)
    inp = make_case(2, T, 2, D, gate, seed=T + D + len(gate))
    o, S, ws = gdr.chunk_fwd_train(*args(inp), erase=erase)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_fwd(inp, erase)
    e_o, e_s = rel_err(o, o_ref), rel_err(S, S_ref)
    o2, S2 = gdr.chunk_fwd(*args(inp), erase=erase)
    torch.cuda.synchronize()
    e_o2 = rel_err(o, o2)
    say(f"o {e_o:.2e}  S {e_s:.2e}  o vs chunk_fwd {e_o2:.2e}")
    assert e_o <= TOL and e_s <= TOL
    assert e_o2 <= 1e-4

    got = gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"], erase=erase,
                        workspace=ws, saved=True)
    plain = gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"], erase=erase)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp, erase)
    ref["d_initial_state"] = ref.pop("dS0")
    errs, diffs = {}, {}
    for n in NAMES:
        if gate == "none" and n == "dlog_alpha":
            assert got[n] is None
            continue
        errs[n] = rel_err(got[n], ref[n])
        diffs[n] = rel_err(got[n], plain[n])
    say("vs oracle", {k: f"{v:.2e}" for k, v in errs.items()},
        "vs recomputing backward", {k: f"{v:.1e}" for k, v in diffs.items()})
    assert all(v <= TOL for v in errs.values()), errs
    assert all(v <= 1e-5 for v in diffs.values()), diffs


def test_train_pair_bf16_output_and_in_place_state():
    """bf16 o, and the final state written over the initial one (the saved
    backward reads the entering states from its workspace, not S_0)."""
    say("train pair bf16 o, in-place carry")
    inp = make_case(2, 77, 3, 128, "scalar", seed=3)
    s0 = inp["initial_state"].clone()
    ref_in = dict(inp, initial_state=s0)
    o, S, ws = gdr.chunk_fwd_train(*args(inp), out_dtype=torch.bfloat16,
                                   final_state=inp["initial_state"])
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and S.data_ptr() == inp["initial_state"].data_ptr()
    o_ref, S_ref = oracle_fwd(ref_in, True)
    # the 2e-3 bar plus the rounding of each value to bf16
    rms = math.sqrt(float(np.mean(o_ref ** 2)))
    assert np.all(np.abs(W.to_f64(o) - o_ref) <= TOL * rms + bf16_half_ulp(o_ref))
    assert rel_err(S, S_ref) <= TOL
    got = gdr.chunk_bwd(*args(ref_in), inp["d_o"], inp["d_final_state"], workspace=ws,
                        saved=True)
    torch.cuda.synchronize()
    ref = oracle_bwd(ref_in, True)
    for n, rn in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"),
                  ("dlog_alpha", "dlog_alpha"), ("d_initial_state", "dS0")):
        assert rel_err(got[n], ref[rn]) <= TOL, n


def test_train_pair_many_chains_sampled():
    """Both slice widths of the launches (64-column slices at 256 chains)."""
    for gate, B, H, D in (("scalar", 8, 32, 128), ("channel", 4, 32, 128), ("none", 8, 32, 64)):
        say("train pair many chains", gate, B, H, D)
        inp = make_case(B, 50, H, D, gate, seed=9)
        o, S, ws = gdr.chunk_fwd_train(*args(inp))
        got = gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"], workspace=ws,
                            saved=True)
        plain = gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"])
        torch.cuda.synchronize()
        for n in NAMES:
            if gate == "none" and n == "dlog_alpha":
                assert got[n] is None and plain[n] is None
                continue
            assert rel_err(got[n], plain[n]) <= 1e-5, n
        for b, h in ((0, 0), (B - 1, H - 1)):
            sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
            st = lambda x: None if x is None else x[b:b + 1, h:h + 1]
            sub = {"q": sl(inp["q"]), "k": sl(inp["k"]), "v": sl(inp["v"]),
                   "beta": sl(inp["beta"]), "log_alpha": sl(inp["log_alpha"]),
                   "initial_state": st(inp["initial_state"]), "d_o": sl(inp["d_o"]),
                   "d_final_state": st(inp["d_final_state"])}
            o_ref, _ = oracle_fwd(sub, True)
            assert rel_err(o[b:b + 1, :, h:h + 1], o_ref) <= TOL
            ref = oracle_bwd(sub, True)
            assert rel_err(got["dk"][b:b + 1, :, h:h + 1], ref["dk"]) <= TOL
            if gate != "none":
                assert rel_err(got["dlog_alpha"][b:b + 1, :, h:h + 1], ref["dlog_alpha"]) <= TOL


@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("D,T", [(64, 33), (128, 100)])
def test_bf16_gradients_are_the_fp32_ones_rounded(D, T, gate, erase):
    """grad_dtype=bf16 (gdr_chunk_bwd_ex): dq, dk, dv are the fp32 gradients
    rounded to nearest even, bit for bit, and the other outputs those of the
    fp32 call; so within the 2e-3 bar plus half a bf16 ulp of the oracle.
    Likewise after the training forward (saved), and gdr_chunk_bwd_ex with
    fp32 gradients is gdr_chunk_bwd bit for bit."""
    say("bf16 gradients", D, T, gate, erase)
    inp = make_case(2, T, 2, D, gate, seed=7 * T + D + len(gate))
    bw = lambda **kw: gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"], erase=erase,
                                    **kw)
    f32 = bw()
    b16 = bw(grad_dtype=torch.bfloat16)
    _, _, ws = gdr.chunk_fwd_train(*args(inp), erase=erase)
    f32s = bw(workspace=ws, saved=True)
    b16s = bw(workspace=ws, saved=True, grad_dtype=torch.bfloat16)
    # the fp32 form of the extended entry point, called directly
    ex = {n: torch.full_like(t, float("nan")) for n, t in f32.items() if t is not None}
    B, T_, H, Dk = inp["q"].shape
    gate_flags = gdr._gate_of(inp["log_alpha"], (B, T_, H), Dk) | (0 if erase else gdr._abi.GDR_NO_ERASE)
    need = gdr.chunk_bwd_workspace_bytes(inp["q"], inp["log_alpha"], erase=erase)
    ws2 = torch.empty(need, device=DEV, dtype=torch.uint8)
    p = lambda t: None if t is None else t.data_ptr()
    st = gdr._abi.gdr_chunk_bwd_ex(
        B, T_, H, Dk, Dk, 0, gdr._abi.GDR_BF16, gdr._abi.GDR_F32, gate_flags,
        *(p(t) for t in args(inp)), p(inp["d_o"]), p(inp["d_final_state"]), p(ex["dq"]),
        p(ex["dk"]), p(ex["dv"]), p(ex["dbeta"]), p(ex.get("dlog_alpha")),
        p(ex["d_initial_state"]), ws2.data_ptr(), need, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == gdr._abi.GDR_OK
    for n in NAMES:
        if f32[n] is None:
            assert b16[n] is None and b16s[n] is None
            continue
        assert torch.equal(ex[n], f32[n]), n
        if n in ("dq", "dk", "dv"):
            assert b16[n].dtype == torch.bfloat16 and b16s[n].dtype == torch.bfloat16
            assert torch.equal(b16[n], f32[n].to(torch.bfloat16)), n
            assert torch.equal(b16s[n], f32s[n].to(torch.bfloat16)), n
        else:
            assert b16[n].dtype == torch.float32
            assert torch.equal(b16[n], f32[n]) and torch.equal(b16s[n], f32s[n]), n
    ref = oracle_bwd(inp, erase)
    for n in ("dq", "dk", "dv"):
        r = ref[n]
        rms = math.sqrt(float(np.mean(r * r)))
        assert np.all(np.abs(W.to_f64(b16[n]) - r) <= TOL * rms + bf16_half_ulp(r)), n


def test_saved_backward_needs_the_workspace():
    inp = make_case(1, 8, 1, 64, "scalar", seed=1)
    with pytest.raises(ValueError):
        gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"], saved=True)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_autograd_function_gives_the_kernels_gradients(gate):
    """loss.backward() through chunk_gated_delta_rule: every input gradient is
    chunk_bwd's for the same upstream gradients (bitwise, cast to the input
    dtypes: the kernels write dq, dk, dv as bf16 directly, the fp32 values
    rounded to nearest even), and within the 2e-3 bar of the oracle."""
    say("autograd", gate)
    inp = make_case(2, 70, 2, 64, gate, seed=13)
    leaves = {n: inp[n].detach().clone().requires_grad_(True)
              for n in ("q", "k", "v", "beta", "log_alpha", "initial_state")
              if inp[n] is not None}
    get = lambda n: leaves.get(n)
    o, S = gdr.chunk_gated_delta_rule(get("q"), get("k"), get("v"), get("beta"),
                                      get("log_alpha"), get("initial_state"))
    w_o = inp["d_o"].float()
    w_s = inp["d_final_state"]
    ((o * w_o).sum() + (S * w_s).sum()).backward()
    torch.cuda.synchronize()
    ref = gdr.chunk_bwd(*args(inp), inp["d_o"], inp["d_final_state"])
    torch.cuda.synchronize()
    pairs = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"),
             ("initial_state", "d_initial_state")]
    if gate != "none":
        pairs.append(("log_alpha", "dlog_alpha"))
    orc = oracle_bwd(inp, True)
    orc["d_initial_state"] = orc.pop("dS0")
    for n, g in pairs:
        got = leaves[n].grad
        assert got is not None and got.dtype == leaves[n].dtype, n
        assert torch.equal(got, ref[g].to(got.dtype)), n
        assert rel_err(ref[g], orc[g]) <= TOL, n


def test_autograd_retained_graph_differentiates_twice():
    """The workspace lives on the autograd graph: with retain_graph=True a
    second backward reads it again and accumulates the same gradients (every
    leaf's gradient is exactly twice the first one's)."""
    say("autograd retain_graph")
    inp = make_case(1, 45, 2, 64, "channel", seed=17)
    leaves = {n: inp[n].detach().clone().requires_grad_(True)
              for n in ("q", "k", "v", "beta", "log_alpha", "initial_state")}
    o, S = gdr.chunk_gated_delta_rule(*(leaves[n] for n in ("q", "k", "v", "beta", "log_alpha",
                                                            "initial_state")))
    loss = (o * inp["d_o"].float()).sum() + (S * inp["d_final_state"]).sum()
    loss.backward(retain_graph=True)
    torch.cuda.synchronize()
    first = {n: t.grad.clone() for n, t in leaves.items()}
    loss.backward()
    torch.cuda.synchronize()
    for n, t in leaves.items():
        assert torch.equal(t.grad, 2 * first[n]), n
