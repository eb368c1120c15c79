"""The allocation-free backward entry point against the one with a workspace.

gdr_chunk_bwd_noalloc runs gdr_chunk_bwd's kernels on the library's static
device array instead of a caller's workspace.  Called through the C ABI
twice in a row, the second time on a smaller input (so the array holds the
first call's data when the second starts), its gradients must equal those of
gdr_chunk_bwd with a torch-allocated workspace: bit for bit (the same
deterministic kernels), hence also within the 2e-3 bar of the parity tests.
"""

import math
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_28_amd as gdr
import workloads as W
from gated_delta_rule_28_amd import _abi

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "d_initial_state")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = W.to_f64(got)
    ref = W.to_f64(ref)
    return float(np.max(np.abs(got - ref))) / max(math.sqrt(float(np.mean(ref * ref))), 1e-300)


def case(B, T, H, D, gate, seed):
    inp = W.make_chunk_inputs(B, T, H, D, D, gate, "bf16", seed=seed, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    inp["initial_state"] = 0.3 * torch.randn(B, H, D, D, device=DEV, generator=g)
    inp["d_o"] = torch.randn(B, T, H, D, device=DEV, generator=g).to(torch.bfloat16)
    inp["d_final_state"] = 0.5 * torch.randn(B, H, D, D, device=DEV, generator=g)
    return inp


def noalloc(inp):
    B, T, H, D = inp["q"].shape
    la = inp["log_alpha"]
    gate = (_abi.GDR_GATE_NONE if la is None else
            _abi.GDR_GATE_CHANNEL if la.dim() == 4 else _abi.GDR_GATE_SCALAR)
    f32 = dict(device=DEV, dtype=torch.float32)
    out = {"dq": torch.empty(B, T, H, D, **f32), "dk": torch.empty(B, T, H, D, **f32),
           "dv": torch.empty(B, T, H, D, **f32), "dbeta": torch.empty(B, T, H, **f32),
           "dlog_alpha": None if la is None else torch.empty(*la.shape, **f32),
           "d_initial_state": torch.empty(B, H, D, D, **f32)}
    ptr = lambda t: None if t is None else t.data_ptr()
    st = _abi.gdr_chunk_bwd_noalloc(
        B, T, H, D, D, 0, _abi.GDR_BF16, gate, inp["q"].data_ptr(), inp["k"].data_ptr(),
        inp["v"].data_ptr(), inp["beta"].data_ptr(), ptr(inp["log_alpha"]),
        inp["initial_state"].data_ptr(), inp["d_o"].data_ptr(), inp["d_final_state"].data_ptr(),
        out["dq"].data_ptr(), out["dk"].data_ptr(), out["dv"].data_ptr(),
        out["dbeta"].data_ptr(), ptr(out["dlog_alpha"]), out["d_initial_state"].data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _abi.GDR_OK, _abi.status_str(st)
    return out


def test_noalloc_backward_equals_the_workspace_entry_point():
    # the second call is smaller: it runs on what the first left in the array
    # (the per-channel gate's passes and gradient kernel too, on a third call)
    for B, T, H, D, gate, seed in ((2, 100, 3, 128, "scalar", 1), (1, 40, 2, 64, "none", 2),
                                   (1, 30, 2, 64, "channel", 3)):
        say("noalloc bwd", B, T, H, D, gate)
        inp = case(B, T, H, D, gate, seed)
        need = gdr.chunk_bwd_workspace_bytes(inp["q"], inp["log_alpha"])
        assert 0 < need <= _abi.NOALLOC_SCRATCH_BYTES
        got = noalloc(inp)
        ref = gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                            inp["initial_state"], inp["d_o"], inp["d_final_state"])
        torch.cuda.synchronize()
        for n in NAMES:
            if ref[n] is None:
                assert got[n] is None
                continue
            assert rel_err(got[n], ref[n]) <= 2e-3, n
            assert torch.equal(got[n], ref[n]), n
