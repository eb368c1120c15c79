"""ctypes binding of libgdr.so (the C ABI declared in include/gdr.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C entry points.  The library is loaded on first use; if
it is missing the call fails loudly (there is no fallback path).
"""

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_EINVAL, GDR_EUNSUPPORTED, GDR_EHIP, GDR_EWORKSPACE = 0, -1, -2, -3, -4
ABI_VERSION = 4
GDR_F32, GDR_BF16 = 0, 1
GDR_GATE_NONE, GDR_GATE_SCALAR, GDR_GATE_CHANNEL = 0, 1, 2
GDR_NO_ERASE = 0x100   # OR'd into a gate: additive write, no erase term
# fused prologue flags (gdr_fuse)
GDR_FUSE_QK_L2NORM, GDR_FUSE_BETA_SIGMOID, GDR_FUSE_DECAY_SOFTPLUS, GDR_FUSE_DECAY_GLA = 1, 2, 4, 8

# every function the header declares, with its ctypes signature
_c_int, _vp, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "gdr_abi_version": (_c_int, []),
    "gdr_status_str": (ctypes.c_char_p, [_c_int]),
    "gdr_chunk_fwd": (_c_int, [_c_int] * 9 + [_vp] * 9),
    "gdr_recurrent_step": (_c_int, [_c_int] * 7 + [_vp] * 8),
    "gdr_chunk_fwd_ex": (_c_int, [_c_int] * 10 + [_vp] * 10),
    "gdr_recurrent_step_ex": (_c_int, [_c_int] * 8 + [_vp] * 9),
    "gdr_chunk_fwd_workspace_bytes": (_sz, [_c_int] * 9),
    "gdr_chunk_bwd_workspace_bytes": (_sz, [_c_int] * 8),
    "gdr_chunk_bwd": (_c_int, [_c_int] * 8 + [_vp] * 15 + [_sz, _vp]),
    "gdr_chunk_bwd_noalloc": (_c_int, [_c_int] * 8 + [_vp] * 15),
    "gdr_chunk_fwd_train": (_c_int, [_c_int] * 9 + [_vp] * 9 + [_sz, _vp]),
    "gdr_chunk_bwd_saved": (_c_int, [_c_int] * 8 + [_vp] * 15 + [_sz, _vp]),
    "gdr_chunk_bwd_ex": (_c_int, [_c_int] * 9 + [_vp] * 15 + [_sz, _c_int, _vp]),
}
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None
_lock = threading.Lock()


class GdrError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


def load():
    """Load libgdr.so once and attach the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -c 'import __graft_entry__ as g; g.build()'` "
                    "or `python -m gated_delta_rule_28_amd.csrc.build`")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            if lib.gdr_abi_version() != ABI_VERSION:
                raise RuntimeError("libgdr.so ABI version mismatch")
            _lib = lib
    return _lib


def abi_version():
    return load().gdr_abi_version()


def status_str(status):
    return load().gdr_status_str(int(status)).decode()


def gdr_chunk_fwd(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, q, k, v, beta,
                  log_alpha, initial_state, o, final_state, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_fwd(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, q, k, v,
                                beta, log_alpha, initial_state, o, final_state, stream)


def gdr_recurrent_step(N, H, Dk, Dv, in_dtype, out_dtype, gate, q, k, v, beta, log_alpha,
                       state, o, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_recurrent_step(N, H, Dk, Dv, in_dtype, out_dtype, gate, q, k, v, beta,
                                     log_alpha, state, o, stream)


def gdr_chunk_fwd_ex(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, fuse, q, k, v, beta,
                     log_alpha, out_gate, initial_state, o, final_state, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_fwd_ex(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, fuse, q, k,
                                   v, beta, log_alpha, out_gate, initial_state, o, final_state,
                                   stream)


def gdr_recurrent_step_ex(N, H, Dk, Dv, in_dtype, out_dtype, gate, fuse, q, k, v, beta,
                          log_alpha, out_gate, state, o, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_recurrent_step_ex(N, H, Dk, Dv, in_dtype, out_dtype, gate, fuse, q, k, v,
                                        beta, log_alpha, out_gate, state, o, stream)


def gdr_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate):
    return load().gdr_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate)


def gdr_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, gate):
    return load().gdr_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, gate)


def gdr_chunk_bwd(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta, log_alpha,
                  initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                  d_initial_state, workspace, workspace_bytes, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_bwd(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta, log_alpha,
                                initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                                d_initial_state, workspace, workspace_bytes, stream)


def gdr_chunk_fwd_train(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, q, k, v, beta,
                        log_alpha, initial_state, o, final_state, workspace, workspace_bytes,
                        stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_fwd_train(B, T, H, Dk, Dv, chunk, in_dtype, out_dtype, gate, q, k, v,
                                      beta, log_alpha, initial_state, o, final_state, workspace,
                                      workspace_bytes, stream)


def gdr_chunk_bwd_saved(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta, log_alpha,
                        initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                        d_initial_state, workspace, workspace_bytes, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_bwd_saved(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta,
                                      log_alpha, initial_state, d_o, d_final_state, dq, dk, dv,
                                      dbeta, dlog_alpha, d_initial_state, workspace,
                                      workspace_bytes, stream)


def gdr_chunk_bwd_ex(B, T, H, Dk, Dv, chunk, in_dtype, grad_dtype, gate, q, k, v, beta,
                     log_alpha, initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                     d_initial_state, workspace, workspace_bytes, saved, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_bwd_ex(B, T, H, Dk, Dv, chunk, in_dtype, grad_dtype, gate, q, k, v,
                                   beta, log_alpha, initial_state, d_o, d_final_state, dq, dk,
                                   dv, dbeta, dlog_alpha, d_initial_state, workspace,
                                   workspace_bytes, int(saved), stream)


def gdr_chunk_bwd_noalloc(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta, log_alpha,
                          initial_state, d_o, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                          d_initial_state, stream):
    """Raw call of the C entry point with integer sizes and raw pointers."""
    return load().gdr_chunk_bwd_noalloc(B, T, H, Dk, Dv, chunk, in_dtype, gate, q, k, v, beta,
                                        log_alpha, initial_state, d_o, d_final_state, dq, dk, dv,
                                        dbeta, dlog_alpha, d_initial_state, stream)
