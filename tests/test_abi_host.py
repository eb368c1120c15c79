"""Host-side checks of the C ABI library (no GPU needed).

The library must load, export every function include/gdr.h declares, and
reject invalid calls on the host with the documented status codes before
anything is launched (these calls never reach the HIP runtime).
"""

import ctypes
import os
import re

import pytest

from gated_delta_rule_28_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == ["gdr_abi_version", "gdr_chunk_bwd", "gdr_chunk_bwd_ex", "gdr_chunk_bwd_noalloc",
                     "gdr_chunk_bwd_saved", "gdr_chunk_bwd_workspace_bytes",
                     "gdr_chunk_fwd", "gdr_chunk_fwd_ex", "gdr_chunk_fwd_train",
                     "gdr_chunk_fwd_workspace_bytes",
                     "gdr_recurrent_step", "gdr_recurrent_step_ex", "gdr_status_str"], names
    assert set(names) == set(_abi.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert _abi.abi_version() == _abi.ABI_VERSION == 4


def test_build_entry_accepts_the_built_library():
    """The check build() runs after compiling passes on the built library."""
    import __graft_entry__
    __graft_entry__.check_loaded()


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_compiles_as_c_and_cpp(tmp_path, lang, std):
    """include/gdr.h is a plain C interface: a C99 (and a C++) translation unit
    that includes it and calls an entry point compiles."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no host compiler or ROCm headers")
    src = tmp_path / "use_gdr.c"
    src.write_text('#include "gdr.h"\n'
                   "int main(void) { return gdr_abi_version() == GDR_ABI_VERSION ? 0 : 1; }\n")
    r = subprocess.run([cc, std, "-Wall", "-Werror", "-fsyntax-only", "-x", lang,
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises at once: the path
    has no other implementation to fall back on."""
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "libgdr.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _abi.abi_version()
    with pytest.raises(RuntimeError, match="missing"):
        _abi.gdr_chunk_bwd_workspace_bytes(1, 1, 1, 64, 64, 0, _abi.GDR_BF16,
                                           _abi.GDR_GATE_SCALAR)


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert _abi.status_str(st).startswith("GDR_")
    assert "unknown" in _abi.status_str(-99)


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced


def chunk(**kw):
    a = dict(B=1, T=8, H=1, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
             out_dtype=_abi.GDR_F32, gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE,
             beta=FAKE, log_alpha=FAKE, initial_state=None, o=FAKE, final_state=None,
             stream=None)
    a.update(kw)
    return _abi.gdr_chunk_fwd(**a)


def step(**kw):
    a = dict(N=1, H=1, Dk=128, Dv=128, in_dtype=_abi.GDR_BF16, out_dtype=_abi.GDR_F32,
             gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, log_alpha=FAKE,
             state=FAKE, o=FAKE, stream=None)
    a.update(kw)
    return _abi.gdr_recurrent_step(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), _abi.GDR_EINVAL),
    (dict(T=-5), _abi.GDR_EINVAL),
    (dict(Dk=0), _abi.GDR_EINVAL),
    (dict(q=None), _abi.GDR_EINVAL),
    (dict(o=None), _abi.GDR_EINVAL),
    (dict(beta=None), _abi.GDR_EINVAL),
    (dict(q=FAKE + 4), _abi.GDR_EINVAL),                      # misaligned
    (dict(beta=FAKE + 2), _abi.GDR_EINVAL),
    (dict(initial_state=FAKE + 8), _abi.GDR_EINVAL),
    (dict(gate=_abi.GDR_GATE_NONE), _abi.GDR_EINVAL),         # log_alpha given for no gate
    (dict(log_alpha=None), _abi.GDR_EINVAL),                  # gate without log_alpha
    (dict(gate=7), _abi.GDR_EINVAL),
    (dict(gate=_abi.GDR_GATE_SCALAR | 0x200), _abi.GDR_EINVAL),   # unknown flag bit
    (dict(gate=_abi.GDR_GATE_NONE | _abi.GDR_NO_ERASE), _abi.GDR_EINVAL),   # log_alpha given
    (dict(in_dtype=5), _abi.GDR_EINVAL),
    (dict(Dk=128, Dv=64), _abi.GDR_EUNSUPPORTED),
    (dict(Dk=96, Dv=96), _abi.GDR_EUNSUPPORTED),
    (dict(chunk=48), _abi.GDR_EUNSUPPORTED),
    (dict(in_dtype=_abi.GDR_F32, Dk=96, Dv=96), _abi.GDR_EUNSUPPORTED),
    (dict(in_dtype=_abi.GDR_F32, Dk=128, Dv=64), _abi.GDR_EUNSUPPORTED),
    (dict(in_dtype=_abi.GDR_F32, chunk=48), _abi.GDR_EUNSUPPORTED),
    # one chunk's rows of a [*, H, 128] tensor must span less than 4 GiB
    (dict(H=300000), _abi.GDR_EUNSUPPORTED),
    # per-channel gate: one chunk's rows of the [*, H, 128] fp32 log decays
    (dict(H=600000, gate=_abi.GDR_GATE_CHANNEL), _abi.GDR_EUNSUPPORTED),
    # per-channel log decays are read with 16-byte vectors
    (dict(gate=_abi.GDR_GATE_CHANNEL, log_alpha=FAKE + 4), _abi.GDR_EINVAL),
])
def test_chunk_fwd_rejects(kw, want):
    assert chunk(**kw) == want


def test_chunk_fwd_empty_batch_is_a_no_op():
    assert chunk(B=0, q=None, k=None, v=None, o=None) == _abi.GDR_OK
    assert chunk(H=0, q=None, k=None, v=None, o=None) == _abi.GDR_OK


@pytest.mark.parametrize("kw,want", [
    (dict(N=-1), _abi.GDR_EINVAL),
    (dict(state=None), _abi.GDR_EINVAL),
    (dict(state=FAKE + 4), _abi.GDR_EINVAL),
    (dict(v=None), _abi.GDR_EINVAL),
    (dict(gate=_abi.GDR_GATE_NONE), _abi.GDR_EINVAL),
    (dict(Dk=128, Dv=32), _abi.GDR_EUNSUPPORTED),
    (dict(Dk=256, Dv=256), _abi.GDR_EUNSUPPORTED),
])
def test_recurrent_step_rejects(kw, want):
    assert step(**kw) == want


def test_recurrent_step_empty_is_a_no_op():
    assert step(N=0, q=None, k=None, v=None, state=None, o=None) == _abi.GDR_OK


def chunk_ex(**kw):
    a = dict(B=1, T=8, H=1, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
             out_dtype=_abi.GDR_F32, gate=_abi.GDR_GATE_SCALAR, fuse=0, q=FAKE, k=FAKE, v=FAKE,
             beta=FAKE, log_alpha=FAKE, out_gate=None, initial_state=None, o=FAKE,
             final_state=None, stream=None)
    a.update(kw)
    return _abi.gdr_chunk_fwd_ex(**a)


def step_ex(**kw):
    a = dict(N=1, H=1, Dk=128, Dv=128, in_dtype=_abi.GDR_BF16, out_dtype=_abi.GDR_F32,
             gate=_abi.GDR_GATE_SCALAR, fuse=0, q=FAKE, k=FAKE, v=FAKE, beta=FAKE,
             log_alpha=FAKE, out_gate=None, state=FAKE, o=FAKE, stream=None)
    a.update(kw)
    return _abi.gdr_recurrent_step_ex(**a)


@pytest.mark.parametrize("kw", [
    dict(fuse=16),                                                     # unknown flag bit
    dict(fuse=_abi.GDR_FUSE_DECAY_SOFTPLUS | _abi.GDR_FUSE_DECAY_GLA), # two decay transforms
    dict(fuse=_abi.GDR_FUSE_DECAY_GLA, gate=_abi.GDR_GATE_NONE, log_alpha=None),  # no gate
    dict(out_gate=FAKE + 2),                                           # misaligned out_gate
])
def test_fused_prologue_validation(kw):
    assert chunk_ex(**kw) == _abi.GDR_EINVAL
    assert step_ex(**kw) == _abi.GDR_EINVAL


# one chunk's rows of the fp32 output, with the fused output gate read at the
# same element offsets: the size bounds hold for that form too
@pytest.mark.parametrize("gate,H", [(_abi.GDR_GATE_SCALAR, 271000),
                                    (_abi.GDR_GATE_CHANNEL, 560000)])
def test_chunk_fwd_size_bound_with_fused_gate(gate, H):
    assert chunk_ex(H=H, gate=gate, out_gate=FAKE, out_dtype=_abi.GDR_F32) == \
        _abi.GDR_EUNSUPPORTED


def test_chunk_bwd_refuses_an_unrequested_initial_state_buffer(monkeypatch):
    """With want_d_initial_state=False a d_initial_state buffer in `out` raises
    before any launch instead of being handed to the kernel unchecked (it
    would be written with B*H*Dk*Dv floats whatever its size)."""
    import torch
    import gated_delta_rule_28_amd as gdr

    def host_check(name, t, dtype=None):
        if dtype is not None and t.dtype != dtype:
            raise TypeError(name)

    called = []
    monkeypatch.setattr(gdr, "_check_dev", host_check)
    monkeypatch.setattr(_abi, "gdr_chunk_bwd", lambda *a: called.append(a) or 0)
    B, T, H, D = 1, 8, 2, 64
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16)
    beta = torch.zeros(B, T, H)
    out = {"dq": torch.zeros(B, T, H, D), "dk": torch.zeros(B, T, H, D),
           "dv": torch.zeros(B, T, H, D), "dbeta": torch.zeros(B, T, H),
           "dlog_alpha": None, "d_initial_state": torch.zeros(1)}
    with pytest.raises(ValueError, match="d_initial_state"):
        gdr.chunk_bwd(q, q, q, beta, None, None, q, None, want_d_initial_state=False, out=out)
    assert not called


def test_recurrent_step_checks_output_shape_before_launch(monkeypatch):
    """A preallocated o of the wrong shape raises in Python and the C entry
    point is never called (a smaller o would be written past its end)."""
    import torch
    import gated_delta_rule_28_amd as gdr

    def host_check(name, t, dtype=None):   # the device check, minus the device
        if dtype is not None and t.dtype != dtype:
            raise TypeError(name)

    called = []
    monkeypatch.setattr(gdr, "_check_dev", host_check)
    monkeypatch.setattr(_abi, "gdr_recurrent_step_ex", lambda *a: called.append(a) or 0)
    N, H, D = 2, 3, 16
    q = torch.zeros(N, H, D)
    beta = torch.zeros(N, H)
    state = torch.zeros(N, H, D, D)
    for bad in (torch.zeros(N, H, D - 1), torch.zeros(1, H, D), torch.zeros(N * H * D)):
        with pytest.raises(ValueError, match="o must be"):
            gdr.recurrent_step(q, q, q, beta, None, state, o=bad)
    assert not called



# ---------------------------------------------------------------------------
# workspace queries and the backward entry point


def test_forward_needs_no_workspace():
    for args in ((8, 4096, 16, 128, 128, 0, _abi.GDR_BF16, _abi.GDR_F32, _abi.GDR_GATE_SCALAR),
                 (2, 8192, 32, 128, 128, 64, _abi.GDR_BF16, _abi.GDR_F32, _abi.GDR_GATE_CHANNEL),
                 (1, 64, 1, 16, 16, 16, _abi.GDR_F32, _abi.GDR_F32, _abi.GDR_GATE_SCALAR)):
        assert _abi.gdr_chunk_fwd_workspace_bytes(*args) == 0


def bwd_ws(B=8, T=4096, H=16, D=128, chunk=0, in_dtype=_abi.GDR_BF16, gate=_abi.GDR_GATE_SCALAR):
    return _abi.gdr_chunk_bwd_workspace_bytes(B, T, H, D, D, chunk, in_dtype, gate)


def test_backward_workspace_size():
    # per chain and 32-token chunk: two D x D states and two 32 x D tiles, fp32
    per = 4 * (2 * 128 * 128 + 2 * 32 * 128)
    assert bwd_ws() == 8 * 16 * 128 * per
    assert bwd_ws(T=33) == 8 * 16 * 2 * per                 # a ragged tail is one more chunk
    assert bwd_ws(gate=_abi.GDR_GATE_NONE) == bwd_ws()
    # the erase-free forms keep the same partitions (U holds b o V there)
    assert bwd_ws(gate=_abi.GDR_GATE_SCALAR | _abi.GDR_NO_ERASE) == bwd_ws()
    assert bwd_ws(gate=_abi.GDR_GATE_NONE | _abi.GDR_NO_ERASE) == bwd_ws()
    # the per-channel gate: 16-token chunks, the same partitions per chunk
    per16 = 4 * (2 * 128 * 128 + 2 * 16 * 128)
    assert bwd_ws(gate=_abi.GDR_GATE_CHANNEL) == 8 * 16 * 256 * per16
    assert bwd_ws(gate=_abi.GDR_GATE_CHANNEL, T=17) == 8 * 16 * 2 * per16
    assert bwd_ws(gate=_abi.GDR_GATE_CHANNEL | _abi.GDR_NO_ERASE) == \
        bwd_ws(gate=_abi.GDR_GATE_CHANNEL)
    assert bwd_ws(D=64, T=64, B=1, H=1) == 2 * 4 * (2 * 64 * 64 + 2 * 32 * 64)
    # unsupported calls and empty inputs need none
    for kw in (dict(in_dtype=_abi.GDR_F32), dict(D=32), dict(T=0), dict(B=0),
               dict(chunk=48), dict(gate=9)):
        assert bwd_ws(**kw) == 0, kw


def bwd(**kw):
    a = dict(B=1, T=8, H=1, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
             gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, log_alpha=FAKE,
             initial_state=None, d_o=FAKE, d_final_state=None, dq=FAKE, dk=FAKE, dv=FAKE,
             dbeta=FAKE, dlog_alpha=FAKE, d_initial_state=None, workspace=FAKE,
             workspace_bytes=1 << 40, stream=None)
    a.update(kw)
    return _abi.gdr_chunk_bwd(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), _abi.GDR_EINVAL),
    (dict(q=None), _abi.GDR_EINVAL),
    (dict(d_o=None), _abi.GDR_EINVAL),
    (dict(dq=None), _abi.GDR_EINVAL),
    (dict(dbeta=None), _abi.GDR_EINVAL),
    (dict(dlog_alpha=None), _abi.GDR_EINVAL),                  # a gate needs its gradient
    (dict(gate=_abi.GDR_GATE_NONE, log_alpha=None), _abi.GDR_EINVAL),   # and none without
    (dict(log_alpha=None), _abi.GDR_EINVAL),
    (dict(dk=FAKE + 4), _abi.GDR_EINVAL),
    (dict(d_initial_state=FAKE + 8), _abi.GDR_EINVAL),
    (dict(in_dtype=_abi.GDR_F32), _abi.GDR_EUNSUPPORTED),
    (dict(Dk=32, Dv=32), _abi.GDR_EUNSUPPORTED),
    (dict(Dk=128, Dv=64), _abi.GDR_EUNSUPPORTED),
    (dict(H=300000), _abi.GDR_EUNSUPPORTED),
    (dict(workspace=None), _abi.GDR_EWORKSPACE),
    (dict(workspace=FAKE + 16), _abi.GDR_EWORKSPACE),          # not 256-byte aligned
    (dict(workspace_bytes=4 * (2 * 128 * 128 + 2 * 32 * 128) - 1), _abi.GDR_EWORKSPACE),
])
def test_chunk_bwd_rejects(kw, want):
    assert bwd(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), _abi.GDR_EINVAL),
    (dict(dq=None), _abi.GDR_EINVAL),
    (dict(in_dtype=_abi.GDR_F32), _abi.GDR_EUNSUPPORTED),
    (dict(workspace=None), _abi.GDR_EWORKSPACE),
])
def test_chunk_bwd_saved_validates_like_chunk_bwd(kw, want):
    a = dict(B=1, T=8, H=1, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
             gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, log_alpha=FAKE,
             initial_state=None, d_o=FAKE, d_final_state=None, dq=FAKE, dk=FAKE, dv=FAKE,
             dbeta=FAKE, dlog_alpha=FAKE, d_initial_state=None, workspace=FAKE,
             workspace_bytes=1 << 40, stream=None)
    a.update(kw)
    assert _abi.gdr_chunk_bwd_saved(**a) == want
    assert _abi.gdr_chunk_bwd(**a) == want


@pytest.mark.parametrize("saved", [0, 1])
@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), _abi.GDR_EINVAL),
    (dict(grad_dtype=2), _abi.GDR_EINVAL),                     # neither fp32 nor bf16
    (dict(grad_dtype=-1), _abi.GDR_EINVAL),
    (dict(dv=None), _abi.GDR_EINVAL),
    (dict(dq=FAKE + 8), _abi.GDR_EINVAL),
    (dict(in_dtype=_abi.GDR_F32), _abi.GDR_EUNSUPPORTED),
    (dict(Dk=32, Dv=32), _abi.GDR_EUNSUPPORTED),
    (dict(workspace=None), _abi.GDR_EWORKSPACE),
    (dict(B=0, q=None, k=None, v=None, d_o=None, dq=None, dk=None, dv=None, dbeta=None,
          workspace=None, workspace_bytes=0), _abi.GDR_OK),
])
def test_chunk_bwd_ex_validates_like_chunk_bwd(kw, want, saved):
    """gdr_chunk_bwd_ex checks its arguments as gdr_chunk_bwd does, with either
    gradient dtype and either value of `saved`, and refuses an unknown
    gradient dtype."""
    for grad in (_abi.GDR_F32, _abi.GDR_BF16):
        a = dict(B=1, T=8, H=1, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
                 grad_dtype=grad, gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE,
                 beta=FAKE, log_alpha=FAKE, initial_state=None, d_o=FAKE, d_final_state=None,
                 dq=FAKE, dk=FAKE, dv=FAKE, dbeta=FAKE, dlog_alpha=FAKE, d_initial_state=None,
                 workspace=FAKE, workspace_bytes=1 << 40, saved=saved, stream=None)
        a.update(kw)
        assert _abi.gdr_chunk_bwd_ex(**a) == want, grad


def fwd_train(**kw):
    a = dict(B=1, T=8, H=1, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
             out_dtype=_abi.GDR_F32, gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE,
             beta=FAKE, log_alpha=FAKE, initial_state=None, o=FAKE, final_state=None,
             workspace=FAKE, workspace_bytes=1 << 40, stream=None)
    a.update(kw)
    return _abi.gdr_chunk_fwd_train(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), _abi.GDR_EINVAL),
    (dict(q=None), _abi.GDR_EINVAL),
    (dict(o=None), _abi.GDR_EINVAL),
    (dict(log_alpha=None), _abi.GDR_EINVAL),
    (dict(gate=_abi.GDR_GATE_NONE), _abi.GDR_EINVAL),          # log_alpha without a gate
    (dict(final_state=FAKE + 4), _abi.GDR_EINVAL),
    (dict(in_dtype=_abi.GDR_F32), _abi.GDR_EUNSUPPORTED),      # the backward's supported set
    (dict(Dk=32, Dv=32), _abi.GDR_EUNSUPPORTED),
    (dict(Dk=128, Dv=64), _abi.GDR_EUNSUPPORTED),
    (dict(chunk=48), _abi.GDR_EUNSUPPORTED),
    (dict(workspace=None), _abi.GDR_EWORKSPACE),
    (dict(workspace=FAKE + 16), _abi.GDR_EWORKSPACE),
    (dict(workspace_bytes=4 * (2 * 128 * 128 + 2 * 32 * 128) - 1), _abi.GDR_EWORKSPACE),
    (dict(gate=_abi.GDR_GATE_CHANNEL, workspace_bytes=4 * (2 * 128 * 128 + 2 * 16 * 128) - 1),
     _abi.GDR_EWORKSPACE),
])
def test_chunk_fwd_train_rejects(kw, want):
    assert fwd_train(**kw) == want


def test_chunk_fwd_train_empty_calls_need_nothing():
    assert fwd_train(B=0, q=None, k=None, v=None, o=None, workspace=None,
                     workspace_bytes=0) == _abi.GDR_OK
    assert fwd_train(T=0, q=None, k=None, v=None, o=None, workspace=None,
                     workspace_bytes=0) == _abi.GDR_OK


def test_chunk_bwd_empty_batch_is_a_no_op():
    assert bwd(B=0, q=None, k=None, v=None, d_o=None, dq=None, dk=None, dv=None, dbeta=None,
               workspace=None, workspace_bytes=0) == _abi.GDR_OK



def test_noalloc_backward_refuses_more_than_its_array():
    """gdr_chunk_bwd_noalloc rejects, before any launch, a call whose workspace
    would not fit its static array; empty calls succeed without one."""
    limit = _abi.NOALLOC_SCRATCH_BYTES
    assert limit == 64 << 20
    # 8 x 16 chains x 128 chunks need about 2.8 GiB
    assert bwd_ws() > limit
    a = dict(B=8, T=4096, H=16, Dk=128, Dv=128, chunk=0, in_dtype=_abi.GDR_BF16,
             gate=_abi.GDR_GATE_SCALAR, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, log_alpha=FAKE,
             initial_state=None, d_o=FAKE, d_final_state=None, dq=FAKE, dk=FAKE, dv=FAKE,
             dbeta=FAKE, dlog_alpha=FAKE, d_initial_state=None, stream=None)
    assert _abi.gdr_chunk_bwd_noalloc(**a) == _abi.GDR_EWORKSPACE
    # one chain-chunk more than fits is refused too
    per = 4 * (2 * 128 * 128 + 2 * 32 * 128)
    fit = limit // per
    assert bwd_ws(B=1, H=1, T=32 * (fit + 1)) > limit >= bwd_ws(B=1, H=1, T=32 * fit)
    assert _abi.gdr_chunk_bwd_noalloc(**dict(a, B=1, H=1, T=32 * (fit + 1))) == \
        _abi.GDR_EWORKSPACE
    # invalid and empty calls: the usual statuses, nothing launched
    assert _abi.gdr_chunk_bwd_noalloc(**dict(a, B=-1)) == _abi.GDR_EINVAL
    assert _abi.gdr_chunk_bwd_noalloc(**dict(a, B=0, q=None)) == _abi.GDR_OK
    assert _abi.gdr_chunk_bwd_noalloc(**dict(a, in_dtype=_abi.GDR_F32)) == \
        _abi.GDR_EUNSUPPORTED
