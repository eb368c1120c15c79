"""Build libgdr.so (HIP kernels + C ABI) for gfx950 with hipcc.

    python -m gated_delta_rule_28_amd.csrc.build        # from the repo root

Every translation unit is compiled to an object in parallel, then linked
into gated_delta_rule_28_amd/libgdr.so.  The build always recompiles.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdr.so")
SOURCES = ["abi.cpp", "passthrough.hip", "recurrent_step.hip", "chunk_fwd_bf16.hip",
           "chunk_fwd_kda.hip", "chunk_fwd_small.hip", "chunk_bwd.hip", "chunk_bwd_kda.hip",
           "bwd_noalloc.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdr.so)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        # packed fp32 ops stay off: only ordinary fp32 VALU code is emitted
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wno-unused-result",
    ]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + common_flags() + lang + ["-c", os.path.join(HERE, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose=True, jobs=None):
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for obj, err in results:
        objs.append(obj)
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
