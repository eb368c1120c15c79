"""Gated delta-rule forward pass for AMD MI355X (gfx950).

Thin Python layer over the C ABI in libgdr.so: it checks tensors, allocates
outputs with torch (device memory and streams only) and passes raw pointers.
All arithmetic runs in the HIP kernels.

    o, S_T = chunk_fwd(q, k, v, beta, log_alpha, initial_state)
    o      = recurrent_step(q, k, v, beta, log_alpha, state)   # state in place
    grads  = chunk_bwd(q, k, v, beta, log_alpha, initial_state, d_o, d_final_state)

For training, chunk_fwd_train returns the forward's outputs together with
the backward's workspace, which chunk_bwd(..., workspace=ws, saved=True)
reads instead of recomputing the forward:

    o, S_T, ws = chunk_fwd_train(q, k, v, beta, log_alpha, initial_state)
    grads = chunk_bwd(q, k, v, beta, log_alpha, initial_state, d_o, d_final_state,
                      workspace=ws, saved=True)

chunk_gated_delta_rule wraps that pair as a torch.autograd.Function, so that
o, S_T = chunk_gated_delta_rule(q, k, v, beta, log_alpha, initial_state)
takes part in loss.backward() (every gradient from the kernels above).

Gate kind follows log_alpha: None -> DeltaNet (alpha = 1); [B, T, H] ->
Gated DeltaNet (one decay per head); [B, T, H, Dk] -> KDA (one per channel).
erase=False drops the erase term (S = alpha S + beta k v^T): linear
attention, the Mamba-2 / SSD decay and GLA's, through the same kernels.

Fused prologue / epilogue (keyword options of both calls): qk_l2norm=True
normalises q and k per (token, head); beta_sigmoid=True takes beta as a
logit; decay="softplus" takes log_alpha as x with log a = -softplus(x),
decay="gla" as x with a = sigmoid(x)^(1/16); out_gate=g multiplies the
output by g * sigmoid(g) (SiLU gate, same shape as o, dtype of q).
"""

import torch

from . import _abi
from ._abi import GdrError, abi_version, status_str, LIB_PATH

__all__ = ["chunk_fwd", "chunk_fwd_train", "chunk_gated_delta_rule", "recurrent_step", "chunk_bwd",
           "chunk_bwd_workspace_bytes", "GdrError", "abi_version", "status_str", "LIB_PATH",
           "library_loaded"]

_DT = {torch.float32: _abi.GDR_F32, torch.bfloat16: _abi.GDR_BF16}


def library_loaded():
    return _abi._lib is not None


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_dev(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def _gate_of(log_alpha, lead_shape, Dk):
    if log_alpha is None:
        return _abi.GDR_GATE_NONE
    if tuple(log_alpha.shape) == tuple(lead_shape):
        return _abi.GDR_GATE_SCALAR
    if tuple(log_alpha.shape) == tuple(lead_shape) + (Dk,):
        return _abi.GDR_GATE_CHANNEL
    raise ValueError(f"log_alpha shape {tuple(log_alpha.shape)} fits neither "
                     f"{tuple(lead_shape)} (per head) nor {tuple(lead_shape) + (Dk,)} (per channel)")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


_DECAY = {None: 0, "log": 0, "softplus": _abi.GDR_FUSE_DECAY_SOFTPLUS, "gla": _abi.GDR_FUSE_DECAY_GLA}


def _fuse_flags(qk_l2norm, beta_sigmoid, decay):
    if decay not in _DECAY:
        raise ValueError(f"decay must be one of {sorted(k for k in _DECAY if k)} or None")
    return ((_abi.GDR_FUSE_QK_L2NORM if qk_l2norm else 0) |
            (_abi.GDR_FUSE_BETA_SIGMOID if beta_sigmoid else 0) | _DECAY[decay])


def _check_gate_tensor(out_gate, shape, dtype):
    if out_gate is None:
        return
    _check_dev("out_gate", out_gate, dtype)
    if tuple(out_gate.shape) != tuple(shape):
        raise ValueError(f"out_gate must be {tuple(shape)}")


def _fwd_args(q, k, v, beta, log_alpha, initial_state, out_dtype, output_final_state, o,
              final_state, erase):
    """Checks of a forward call's tensors; allocates o and the final state
    when not given.  Returns B, T, H, Dk, Dv, the gate flags, o, final_state."""
    _check_dev("q", q)
    if q.dtype not in _DT:
        raise TypeError("q/k/v must be bf16 or fp32")
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("beta", beta, torch.float32)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B, T, H, Dk] and v [B, T, H, Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if tuple(beta.shape) != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    gate = _gate_of(log_alpha, (B, T, H), Dk) | (0 if erase else _abi.GDR_NO_ERASE)
    if log_alpha is not None:
        _check_dev("log_alpha", log_alpha, torch.float32)
    if initial_state is not None:
        _check_dev("initial_state", initial_state, torch.float32)
        if tuple(initial_state.shape) != (B, H, Dk, Dv):
            raise ValueError("initial_state must be [B, H, Dk, Dv]")
    if out_dtype not in _DT:
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if o is None:
        o = torch.empty(B, T, H, Dv, device=q.device, dtype=out_dtype)
    else:
        _check_dev("o", o, out_dtype)
        if tuple(o.shape) != (B, T, H, Dv):
            raise ValueError("o must be [B, T, H, Dv]")
    if final_state is None and output_final_state:
        final_state = torch.empty(B, H, Dk, Dv, device=q.device, dtype=torch.float32)
    elif final_state is not None:
        _check_dev("final_state", final_state, torch.float32)
        if tuple(final_state.shape) != (B, H, Dk, Dv):
            raise ValueError("final_state must be [B, H, Dk, Dv]")
    return B, T, H, Dk, Dv, gate, o, final_state


def chunk_fwd(q, k, v, beta, log_alpha=None, initial_state=None, *, chunk=0,
              out_dtype=torch.float32, output_final_state=True, o=None, final_state=None,
              erase=True, qk_l2norm=False, beta_sigmoid=False, decay=None, out_gate=None):
    """Chunkwise forward over whole sequences.

    q, k [B, T, H, Dk] and v [B, T, H, Dv] (bf16 or fp32, same dtype);
    beta [B, T, H] fp32; log_alpha None | [B, T, H] | [B, T, H, Dk] fp32;
    initial_state None | [B, H, Dk, Dv] fp32.  Returns (o [B, T, H, Dv] in
    out_dtype, final state [B, H, Dk, Dv] fp32 or None).  `o` and
    `final_state` may be passed preallocated; final_state may be the
    initial_state tensor itself (in-place carry).

    erase=False drops the erase term (additive write).  Fused options
    (applied inside the kernels, see the module docstring): qk_l2norm,
    beta_sigmoid (beta holds logits), decay="softplus" | "gla" (log_alpha
    holds the pre-activation; needs a gate), out_gate [B, T, H, Dv] in the
    dtype of q (o <- o * g * sigmoid(g)).
    """
    B, T, H, Dk, Dv, gate, o, final_state = _fwd_args(
        q, k, v, beta, log_alpha, initial_state, out_dtype, output_final_state, o, final_state,
        erase)
    fuse = _fuse_flags(qk_l2norm, beta_sigmoid, decay)
    _check_gate_tensor(out_gate, (B, T, H, Dv), q.dtype)
    st = _abi.gdr_chunk_fwd_ex(B, T, H, Dk, Dv, int(chunk), _DT[q.dtype], _DT[out_dtype], gate,
                               fuse, q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                               _ptr(log_alpha), _ptr(out_gate), _ptr(initial_state),
                               o.data_ptr(), _ptr(final_state), _stream(q.device))
    if st != _abi.GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd_ex")
    return o, final_state


def recurrent_step(q, k, v, beta, log_alpha, state, *, out_dtype=torch.float32, o=None,
                   erase=True, qk_l2norm=False, beta_sigmoid=False, decay=None, out_gate=None):
    """One decode token for N sequences; `state` [N, H, Dk, Dv] fp32 is
    updated in place.  q, k [N, H, Dk]; v [N, H, Dv]; beta [N, H];
    log_alpha None | [N, H] | [N, H, Dk].  Returns o [N, H, Dv].  erase and
    the fused options are those of chunk_fwd (out_gate [N, H, Dv])."""
    _check_dev("q", q)
    if q.dtype not in _DT:
        raise TypeError("q/k/v must be bf16 or fp32")
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("beta", beta, torch.float32)
    _check_dev("state", state, torch.float32)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [N, H, Dk] and v [N, H, Dv]")
    N, H, Dk = q.shape
    Dv = v.shape[2]
    if tuple(beta.shape) != (N, H) or tuple(state.shape) != (N, H, Dk, Dv):
        raise ValueError("beta must be [N, H] and state [N, H, Dk, Dv]")
    gate = _gate_of(log_alpha, (N, H), Dk) | (0 if erase else _abi.GDR_NO_ERASE)
    if log_alpha is not None:
        _check_dev("log_alpha", log_alpha, torch.float32)
    if out_dtype not in _DT:
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if o is None:
        o = torch.empty(N, H, Dv, device=q.device, dtype=out_dtype)
    else:
        _check_dev("o", o, out_dtype)
        if tuple(o.shape) != (N, H, Dv):
            raise ValueError("o must be [N, H, Dv]")
    fuse = _fuse_flags(qk_l2norm, beta_sigmoid, decay)
    _check_gate_tensor(out_gate, (N, H, Dv), q.dtype)
    st = _abi.gdr_recurrent_step_ex(N, H, Dk, Dv, _DT[q.dtype], _DT[out_dtype], gate, fuse,
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                                    _ptr(log_alpha), _ptr(out_gate), state.data_ptr(),
                                    o.data_ptr(), _stream(q.device))
    if st != _abi.GDR_OK:
        raise GdrError(st, "gdr_recurrent_step_ex")
    return o


def chunk_fwd_train(q, k, v, beta, log_alpha=None, initial_state=None, *, chunk=0,
                    out_dtype=torch.float32, output_final_state=True, o=None, final_state=None,
                    erase=True, workspace=None):
    """chunk_fwd for training: the same (o, final state), and besides the
    backward's workspace holding what chunk_bwd(..., saved=True) reads in
    place of its recompute pass.  Returns (o, final_state, workspace).

    Inputs within chunk_bwd's supported set (bf16 q/k/v, Dk = Dv in {64,
    128}, every gate, with or without the erase term), no fused options.
    `workspace`, a uint8 GPU tensor of at least chunk_bwd_workspace_bytes,
    is allocated with torch when not given.  Pass the same inputs and this
    workspace, unchanged, to chunk_bwd(..., saved=True).
    """
    B, T, H, Dk, Dv, gate, o, final_state = _fwd_args(
        q, k, v, beta, log_alpha, initial_state, out_dtype, output_final_state, o, final_state,
        erase)
    need = int(_abi.gdr_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, int(chunk), _DT[q.dtype], gate))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    else:
        _check_dev("workspace", workspace, torch.uint8)
    st = _abi.gdr_chunk_fwd_train(B, T, H, Dk, Dv, int(chunk), _DT[q.dtype], _DT[out_dtype], gate,
                                  q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                                  _ptr(log_alpha), _ptr(initial_state), o.data_ptr(),
                                  _ptr(final_state), workspace.data_ptr(), workspace.numel(),
                                  _stream(q.device))
    if st != _abi.GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd_train")
    return o, final_state, workspace


def chunk_bwd_workspace_bytes(q, log_alpha=None, chunk=0, erase=True):
    """Bytes of device workspace chunk_bwd needs for inputs shaped like q
    ([B, T, H, Dk]) and this gate (0 when the call is not supported)."""
    B, T, H, Dk = q.shape
    gate = _gate_of(log_alpha, (B, T, H), Dk) | (0 if erase else _abi.GDR_NO_ERASE)
    return int(_abi.gdr_chunk_bwd_workspace_bytes(B, T, H, Dk, Dk, int(chunk), _DT[q.dtype], gate))


def chunk_bwd(q, k, v, beta, log_alpha=None, initial_state=None, d_o=None, d_final_state=None,
              *, chunk=0, erase=True, workspace=None, want_d_initial_state=True, out=None,
              saved=False, grad_dtype=torch.float32):
    """Gradients of chunk_fwd's o and final state.

    Inputs as for chunk_fwd (bf16 q/k/v, Dk = Dv in {64, 128}, every gate,
    with or without the erase term); d_o [B, T, H, Dv] in the dtype of q
    (None for zero) and d_final_state [B, H, Dk, Dv] fp32 (None for zero).
    Returns a dict with dq, dk, dv (grad_dtype: fp32 or bf16, each the fp32
    gradient rounded to nearest even; shaped like q, k, v), dbeta
    [B, T, H], dlog_alpha (None without a gate, else shaped like log_alpha)
    and d_initial_state
    [B, H, Dk, Dv] (None when want_d_initial_state is False).  `workspace`,
    a uint8 GPU tensor of at least chunk_bwd_workspace_bytes, is allocated
    with torch when not given; `out`, a dict of the same keys and shapes,
    receives the gradients when given (nothing is allocated then).
    saved=True: `workspace` is the one chunk_fwd_train filled for these same
    inputs; the recompute pass is skipped.
    """
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("grad_dtype must be torch.float32 or torch.bfloat16")
    _check_dev("q", q)
    if q.dtype not in _DT:
        raise TypeError("q/k/v must be bf16 or fp32")
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("beta", beta, torch.float32)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("expected q, k, v [B, T, H, D] (Dk = Dv)")
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if tuple(beta.shape) != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    gate = _gate_of(log_alpha, (B, T, H), Dk) | (0 if erase else _abi.GDR_NO_ERASE)
    if log_alpha is not None:
        _check_dev("log_alpha", log_alpha, torch.float32)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check_dev(name, t, torch.float32)
            if tuple(t.shape) != (B, H, Dk, Dv):
                raise ValueError(f"{name} must be [B, H, Dk, Dv]")
    if d_o is None:
        d_o = torch.zeros_like(v)
    _check_dev("d_o", d_o, q.dtype)
    if tuple(d_o.shape) != (B, T, H, Dv):
        raise ValueError("d_o must be [B, T, H, Dv]")
    shapes = {"dq": (B, T, H, Dk), "dk": (B, T, H, Dk), "dv": (B, T, H, Dv),
              "dbeta": (B, T, H),
              "dlog_alpha": None if log_alpha is None else tuple(log_alpha.shape),
              "d_initial_state": (B, H, Dk, Dv) if want_d_initial_state else None}
    dtypes = {n: grad_dtype if n in ("dq", "dk", "dv") else torch.float32 for n in shapes}
    if out is None:
        out = {n: None if shp is None else torch.empty(*shp, device=q.device, dtype=dtypes[n])
               for n, shp in shapes.items()}
    else:
        for n, shp in shapes.items():
            t = out.get(n)
            if shp is None:
                if t is not None:
                    raise ValueError("dlog_alpha must be None without a gate" if n == "dlog_alpha"
                                     else "d_initial_state must be None when "
                                          "want_d_initial_state is False")
                out[n] = None
                continue
            _check_dev(n, t, dtypes[n])
            if tuple(t.shape) != shp:
                raise ValueError(f"{n} must be {shp}")
    need = int(_abi.gdr_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, int(chunk), _DT[q.dtype], gate))
    if workspace is None:
        if saved:
            raise ValueError("saved=True needs the workspace chunk_fwd_train filled")
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    else:
        _check_dev("workspace", workspace, torch.uint8)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(), _ptr(log_alpha),
            _ptr(initial_state), d_o.data_ptr(), _ptr(d_final_state), out["dq"].data_ptr(),
            out["dk"].data_ptr(), out["dv"].data_ptr(), out["dbeta"].data_ptr(),
            _ptr(out["dlog_alpha"]), _ptr(out["d_initial_state"]), workspace.data_ptr(),
            workspace.numel())
    if grad_dtype == torch.float32:   # the fp32 entry points
        name = "gdr_chunk_bwd_saved" if saved else "gdr_chunk_bwd"
        st = getattr(_abi, name)(B, T, H, Dk, Dv, int(chunk), _DT[q.dtype], gate, *ptrs,
                                 _stream(q.device))
    else:
        name = "gdr_chunk_bwd_ex"
        st = _abi.gdr_chunk_bwd_ex(B, T, H, Dk, Dv, int(chunk), _DT[q.dtype], _DT[grad_dtype],
                                   gate, *ptrs, saved, _stream(q.device))
    if st != _abi.GDR_OK:
        raise GdrError(st, name)
    return out


class _ChunkRule(torch.autograd.Function):
    """chunk_fwd_train in the forward, chunk_bwd(saved=True) in the backward;
    the workspace lives on the autograd graph between the two (released with
    the graph, so a retained graph can be differentiated again)."""

    @staticmethod
    def forward(ctx, q, k, v, beta, log_alpha, initial_state, erase, chunk):
        o, S, ws = chunk_fwd_train(q, k, v, beta, log_alpha, initial_state, chunk=chunk,
                                   erase=erase)
        ctx.save_for_backward(q, k, v, beta, log_alpha, initial_state)
        ctx.ws, ctx.erase, ctx.chunk = ws, erase, chunk
        return o, S

    @staticmethod
    def backward(ctx, d_o, d_final):
        q, k, v, beta, log_alpha, initial_state = ctx.saved_tensors
        # the kernels take dL/do in the dtype of q (exact MFMA operands)
        d_o = torch.zeros_like(v) if d_o is None else d_o.to(q.dtype).contiguous()
        d_final = None if d_final is None else d_final.float().contiguous()
        # dq, dk, dv come out of the kernels in the dtype of q, k, v
        g = chunk_bwd(q, k, v, beta, log_alpha, initial_state, d_o, d_final, chunk=ctx.chunk,
                      erase=ctx.erase, workspace=ctx.ws, saved=True,
                      want_d_initial_state=initial_state is not None, grad_dtype=q.dtype)

        def like(x, t):
            return None if x is None or t is None else x.to(t.dtype)
        return (like(g["dq"], q), like(g["dk"], k), like(g["dv"], v), g["dbeta"],
                g["dlog_alpha"], g["d_initial_state"], None, None)


def chunk_gated_delta_rule(q, k, v, beta, log_alpha=None, initial_state=None, *, erase=True,
                           chunk=0):
    """Differentiable chunkwise forward: (o [B, T, H, Dv] fp32, final state
    [B, H, Dk, Dv] fp32), with gradients for q, k, v, beta, log_alpha and
    initial_state from chunk_bwd.  Inputs as for chunk_fwd_train (bf16
    q/k/v, Dk = Dv in {64, 128}, every gate, erase or not).  The upstream
    gradient of o is rounded to the dtype of q before the backward kernels
    read it; the backward's workspace (chunk_bwd_workspace_bytes) is held
    from the forward until the backward has run.
    """
    return _ChunkRule.apply(q, k, v, beta, log_alpha, initial_state, erase, int(chunk))
