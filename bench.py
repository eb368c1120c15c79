"""Benchmark of the gated delta-rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
    python bench.py --only counters        # the kernels alone, for rocprofv3 --pmc
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR   # (CPU) counter CSVs -> profiles/

One "step" is one gdr_chunk_fwd call over the Gated DeltaNet layer workload
gdn_bf16_b8h16t4096 (B=8, H=16, T=4096, d_k = d_v = 128, bf16 q/k/v, fp32
beta/log alpha, fp32 state, fp32 output): every row of the chunkwise hot path
(in-chunk log-decay cumsum, K K^T and Q K^T with the decay, the unit-lower
triangular solve, the WY factors, the serial inter-chunk state pass and the
outputs) runs inside that one kernel.  Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts.

Printed: ONE JSON line with tokens/s (B*T / wall time per step), the roofline
of the chunk kernel (HBM-bound: algorithmic bytes / mean kernel time from HIP
events on the launch stream / 8 TB/s; measured HBM traffic from the committed
counter summary when it was taken on the current kernel source), the fp64
oracle timed on the host cores, and secondary lines: bf16 output, the KDA
workload kda_bf16_b2h32t8192, both shapes without the erase term and with the
fused prologue / output gate, and the batched decode step (256 sequences x 32
heads, 128 consecutive steps, eager and as one HIP graph), the tiny fp32
workload (microseconds per call: launch-latency bound), the B=4, H=8,
T=2048 DeltaNet and Gated DeltaNet workloads (timed cold, after an untimed
512 MiB write between calls, and warm), and a 1 GiB device copy whose rate
is the measured HBM ceiling each roofline is also quoted against.

The oracle baseline runs the fp64 recurrence over every chain of the
headline run, on the timed run's own inputs copied from the device, split
across the host cores (one process per core, one BLAS thread each); its
output is what the `parity` field of the line compares the GPU output with.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gated_delta_rule_28_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

# tokens per chunk of the MFMA kernels' state pass (the chunk argument of
# gdr_chunk_fwd only changes rounding, so the kernels use their own)
KERNEL_CHUNK = {"none": 32, "scalar": 32, "channel": 16}
KERNEL_OF_GATE = {"none": "chunk_fwd_bf16_kernel", "scalar": "chunk_fwd_bf16_kernel",
                  "channel": "chunk_fwd_kda_kernel"}
KERNEL_SOURCES = {
    "chunk_fwd_bf16_kernel": ["chunk_fwd_bf16.hip", "mfma_util.h", "common.h"],
    "chunk_fwd_kda_kernel": ["chunk_fwd_kda.hip", "mfma_util.h", "common.h"],
    "recurrent_step_kernel": ["recurrent_step.hip", "common.h"],
    "chunk_bwd_grad_kernel": ["chunk_bwd.hip", "mfma_util.h", "common.h", "internal.h"],
}
# the plain copy used to calibrate the byte counters: |x| over 1 GiB of fp32
COPY_BYTES = 1 << 30
COPY_REGEX = "AbsFunctor"
# the bf16 GEMM of known size that checks the MFMA operation counter's scale
GEMM_N = 4096
GEMM_REGEX = "Cijk"
SIMD_PER_GPU = 256 * 4            # MI355X: 256 compute units x 4 SIMDs
PARITY_TOL = 2e-3                 # max|d| / RMS(ref), bf16 inputs with fp32 state
MAX_ORACLE_PROCS = 16             # the host-core share of one GPU


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(kernel, workload, root=PROFILES):
    return os.path.join(root, f"traffic_{kernel}_{workload}.txt")


def read_traffic(kernel, workload, root=PROFILES):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = traffic_file(kernel, workload, root)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != source_hash(kernel):
        return None
    return float(kv["traffic_bytes_per_launch"])


def mfma_file(kernel, workload, root=PROFILES):
    return os.path.join(root, f"mfma_{kernel}_{workload}.txt")


def read_mfma(kernel, workload, root=PROFILES):
    """MFMA counters per launch from the committed summary (busy fraction,
    issued bf16 flops), or None when there is none or the kernel source
    changed since it was taken."""
    path = mfma_file(kernel, workload, root)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != source_hash(kernel):
        return None
    return {"busy_frac": float(kv["mfma_busy_frac"]),
            "issued_flops_per_launch": float(kv["issued_bf16_flops_per_launch"])}


# ---------------------------------------------------------------------------
# algorithmic counts


def chunk_alg_bytes(w, out_bytes=4, out_gate=False):
    """Single-pass minimum HBM bytes of one chunk_fwd call (zero initial
    state, final state written): q, k, v in, beta and log alpha in, o out
    (and the output gate in, when it is fused)."""
    th = w.B * w.T * w.H
    in_b = 2 if w.in_dtype == "bf16" else 4
    per_th = in_b * (2 * w.Dk + w.Dv) + 4
    if out_gate:
        per_th += in_b * w.Dv
    if w.gate == "scalar":
        per_th += 4
    elif w.gate == "channel":
        per_th += 4 * w.Dk
    per_th += out_bytes * w.Dv
    return th * per_th + w.B * w.H * w.Dk * w.Dv * 4


def chunk_alg_flops(w, C, erase=True):
    """Algorithmic flops per call at chunk length C: per token-head 6 dk dv
    (W S, Q S, K~^T U) + 2 C dk (Q K^T and K K^T halves) + (C-1)(dk+dv)
    (solve on [bV | bgK]) + (C+1) dv (masked P U).  Without the erase term
    there is no W S, K K^T or solve: 4 dk dv + C dk + (C+1) dv."""
    dk, dv = w.Dk, w.Dv
    if erase:
        per_th = 6 * dk * dv + 2 * C * dk + (C - 1) * (dk + dv) + (C + 1) * dv
    else:
        per_th = 4 * dk * dv + C * dk + (C + 1) * dv
    return w.B * w.T * w.H * per_th


def decode_alg_bytes(w):
    """Per step: fp32 state read + written, q/k/v in, beta/log alpha in, o out."""
    n = w.N * w.H
    in_b = 2 if w.in_dtype == "bf16" else 4
    return n * (2 * 4 * w.Dk * w.Dv + in_b * (2 * w.Dk + w.Dv) + 8 + 4 * w.Dv)


# ---------------------------------------------------------------------------
# GPU timing


def time_launches(torch, fn, steps, warmup, settle_s=0.0, pre=None):
    """Run fn for `settle_s` seconds of wall time (untimed: the GPU clock
    ramps up over the first ~80 launches of a fresh process and the first
    launches run up to ~20% slower), then `warmup` times, then exactly
    `steps` times between two full synchronisations; each timed call is also
    bracketed by events on the current stream, the stream the kernels are
    launched on.  `pre`, when given, runs before every timed call, outside
    its events (the cache flush of the cold timings)."""
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        if pre is not None:
            pre()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    return wall, per


def copy_ceiling(torch, nbytes=COPY_BYTES, steps=10):
    """Measured HBM ceiling: a plain device-to-device pass over `nbytes`
    (read once, written once), GB/s of read + written bytes at the median
    call, for torch's copy_ (which may use a DMA engine) and for an
    elementwise kernel (|x|); the faster of the two is the ceiling."""
    src = torch.empty(nbytes // 4, device="cuda", dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    rates = {}
    for kind, fn in (("torch copy_", lambda: dst.copy_(src)),
                     ("torch abs (elementwise kernel)", lambda: torch.abs(src, out=dst))):
        _, per = time_launches(torch, fn, steps, 2, settle_s=0.1)
        rates[kind] = 2 * nbytes / (statistics.median(per) * 1e-3) / 1e9
    del src, dst
    best = max(rates, key=rates.get)
    return {"bytes_moved_per_pass": 2 * nbytes, "GB/s": rates[best], "kind": best,
            "all_GB/s": rates, "tensor": "1 GiB fp32"}


def with_copy_frac(roof, copy):
    """The roofline dict with its achieved rate also quoted against the
    measured copy ceiling."""
    if copy is not None:
        roof = dict(roof, copy_GBs=copy["GB/s"], frac_of_copy=roof["achieved"] / copy["GB/s"])
    return roof


def fused_inputs(torch, inp, w):
    """Pre-activations whose fused transforms give back the workload's own
    b and decay: beta as the logit of b, log_alpha as x with
    -softplus(x) = log a, q and k rows rescaled (the L2 normalisation undoes
    it), and a seeded bf16 output gate."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    out = dict(inp)
    for name in ("q", "k"):
        x = inp[name].float()
        scale = 0.5 + 1.5 * torch.rand(*x.shape[:-1], 1, device="cuda", generator=g)
        out[name] = (x * scale).to(inp[name].dtype)
    b = inp["beta"].clamp(1e-4, 1.0 - 1e-4)
    out["beta"] = torch.log(b / (1.0 - b))
    if inp["log_alpha"] is not None:
        out["log_alpha"] = torch.log(torch.expm1(-inp["log_alpha"].clamp(max=-1e-6)))
    out["out_gate"] = torch.randn(w.B, w.T, w.H, w.Dv, device="cuda", generator=g).to(inp["q"].dtype)
    return out


def separate_passes_line(torch, gdr, W, w, steps, warmup, settle_s, copy_gbs, unfused_ms):
    """The fused options done as separate passes around the unfused kernel,
    for comparison with the fused line: log a = -softplus(x) of the decay
    pre-activations, q and k L2-normalised, b = sigmoid of its logit, the
    kernel, then o *= silu(gate).  One step = all of them, timed with the
    same events (torch's elementwise kernels for the passes).  Also the bytes
    the passes move (each reads its input and writes its output once) and
    their time at the measured copy rate."""
    import torch.nn.functional as F
    inp = fused_inputs(torch, W.make_workload_inputs(w, seed=0, device="cuda"), w)
    o = torch.empty(w.B, w.T, w.H, w.Dv, device="cuda", dtype=torch.float32)
    S = torch.empty(w.B, w.H, w.Dk, w.Dv, device="cuda", dtype=torch.float32)

    def step():
        la = F.logsigmoid(-inp["log_alpha"]) if inp["log_alpha"] is not None else None
        qn = F.normalize(inp["q"], dim=-1)
        kn = F.normalize(inp["k"], dim=-1)
        b = torch.sigmoid(inp["beta"])
        gdr.chunk_fwd(qn, kn, inp["v"], b, la, None, chunk=w.chunk, o=o, final_state=S)
        o.mul_(F.silu(inp["out_gate"]))
    _, per = time_launches(torch, step, steps, warmup, settle_s)
    th = w.B * w.T * w.H
    in_b = 2 if w.in_dtype == "bf16" else 4
    la_n = {"none": 0, "scalar": th, "channel": th * w.Dk}[w.gate]
    passes_bytes = (2 * 4 * la_n + 2 * 2 * in_b * th * w.Dk + 2 * 4 * th
                    + (4 + in_b + 4) * th * w.Dv)
    at_copy = passes_bytes / (copy_gbs * 1e9) * 1e3 if copy_gbs else None
    return {"ms": statistics.fmean(per), "passes_bytes": passes_bytes,
            "passes_ms_at_copy_rate": at_copy,
            "unfused_kernel_plus_passes_at_copy_rate_ms": (unfused_ms + at_copy) if at_copy else None,
            "note": "torch elementwise passes (logsigmoid, normalize, sigmoid, silu and mul) "
                    "around the unfused kernel, timed as one step"}


def chunk_setup(torch, gdr, W, w, out_dtype, erase=True, fused=False, keep=None):
    inp = W.make_workload_inputs(w, seed=0, device="cuda")
    o = torch.empty(w.B, w.T, w.H, w.Dv, device="cuda", dtype=out_dtype)
    S = torch.empty(w.B, w.H, w.Dk, w.Dv, device="cuda", dtype=torch.float32)
    kw = {}
    if fused:
        inp = fused_inputs(torch, inp, w)
        kw = dict(qk_l2norm=True, beta_sigmoid=True, out_gate=inp["out_gate"],
                  decay="softplus" if inp["log_alpha"] is not None else None)

    def step():
        gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None,
                      chunk=w.chunk, out_dtype=out_dtype, o=o, final_state=S, erase=erase, **kw)
    if keep is not None:
        keep.update(inp=inp, o=o, S=S)
    return step, o, S


def chunk_line(torch, gdr, W, w, steps, warmup, out_dtype, settle_s=0.0, erase=True,
               fused=False, cold=False, keep=None):
    """Timed launches of one chunk workload.  cold=True writes a 512 MiB
    scratch buffer (untimed, on the launch stream) before every timed call,
    so no input is left in the caches; `keep`, a dict, receives the run's
    inputs and outputs."""
    step, o, S = chunk_setup(torch, gdr, W, w, out_dtype, erase, fused, keep=keep)
    pre = None
    if cold:
        scratch = torch.empty(512 << 20, device="cuda", dtype=torch.uint8)
        pre = scratch.zero_
    wall, per = time_launches(torch, step, steps, warmup, settle_s, pre=pre)
    if not (bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())):
        raise RuntimeError(f"non-finite output in the timed run of {w.name}")
    out_b = 2 if out_dtype == torch.bfloat16 else 4
    kern = KERNEL_OF_GATE[w.gate]
    C = KERNEL_CHUNK[w.gate]
    mean_ms = statistics.fmean(per)
    alg_b = chunk_alg_bytes(w, out_b, out_gate=fused)
    alg_f = chunk_alg_flops(w, C, erase)
    achieved = alg_b / (mean_ms * 1e-3) / 1e9
    # counters are taken for the erasing, unfused fp32-output launches only
    plain = out_b == 4 and erase and not fused
    traffic = read_traffic(kern, w.name) if plain else None
    mc = read_mfma(kern, w.name) if plain else None
    mfma_counter = None
    if mc is not None:
        issued = mc["issued_flops_per_launch"] / (mean_ms * 1e-3) / 1e12
        mfma_counter = {"busy_frac": mc["busy_frac"], "issued_tflops": issued,
                        "issued_frac_of_peak": issued / BF16_PEAK_TFLOPS,
                        "issued_over_alg": mc["issued_flops_per_launch"] / alg_f,
                        "source": os.path.basename(mfma_file(kern, w.name)),
                        "note": "rocprofv3 counters: busy = MFMA-busy SIMD cycles / (GPU-active "
                                "cycles x 1024 SIMDs); issued = bf16 MFMA operations x 512 "
                                "(hi/lo split products included) / mean event time"}
    if cold:
        del scratch
    return {
        "workload": w.name, "tokens": w.B * w.T, "wall_s": wall, "steps": steps,
        "ms_per_step": 1e3 * wall / steps,
        "value": w.B * w.T / (wall / steps),
        "kernel": kern, "kernel_chunk": C,
        "kernel_ms": {"mean": mean_ms, "median": statistics.median(per), "min": min(per)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": alg_b},
        "mfma_alg": {"achieved": alg_f / (mean_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": alg_f / (mean_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "alg_flops_per_launch": alg_f},
        "mfma_counter": mfma_counter,
    }


def decode_setup(torch, gdr, W, d):
    inp = W.make_decode_inputs(d.N, d.H, d.Dk, d.Dv, d.steps, d.gate, d.in_dtype, seed=0,
                               device="cuda", alpha_mu=d.alpha_mu, alpha_sigma=d.alpha_sigma,
                               state_std=d.state_std)
    state = inp["state"]
    o = torch.empty(d.steps, d.N, d.H, d.Dv, device="cuda", dtype=torch.float32)

    def one_pass():
        # the workload: `steps` consecutive tokens, each consuming the state
        for t in range(d.steps):
            gdr.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["beta"][t],
                               inp["log_alpha"][t], state, o=o[t])
    return one_pass, state, o


def decode_line(torch, gdr, W, d, passes=3, settle_s=0.0):
    one_pass, state, o = decode_setup(torch, gdr, W, d)
    _, per_eager = time_launches(torch, one_pass, passes, 1, settle_s)
    # the same 128 launches captured once and replayed as one HIP graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    _, per_graph = time_launches(torch, graph.replay, passes, 1)
    if not (bool(torch.isfinite(o).all()) and bool(torch.isfinite(state).all())):
        raise RuntimeError("non-finite decode output")
    db = decode_alg_bytes(d)
    ms_eager = statistics.fmean(per_eager) / d.steps
    ms_graph = statistics.fmean(per_graph) / d.steps
    traffic = read_traffic("recurrent_step_kernel", d.name)
    return {
        "workload": d.name, "unit": "tokens/s",
        "value": d.N / (ms_graph * 1e-3),
        "ms_per_token_step": {"graph": ms_graph, "eager": ms_eager},
        "roofline": {"bound": "hbm", "achieved": db / (ms_graph * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": db / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "alg_bytes_per_launch": db,
                     "note": "per-step time of the 128-step graph replay (launch gaps included)"},
    }


def _oracle_worker(args):
    """One host process's share of the oracle baseline: the fp64 recurrence
    over a group of chains (laid out as the heads of one sequence), with one
    BLAS thread.  Returns (o, S_T, seconds)."""
    q, k, v, beta, log_alpha = args
    from threadpoolctl import threadpool_limits
    from oracle import gated_delta_recurrence
    with threadpool_limits(1):
        t0 = time.perf_counter()
        o, S = gated_delta_recurrence(q, k, v, beta, log_alpha)
        dt = time.perf_counter() - t0
    return o, S, dt


def _warm_worker(_):
    import numpy  # noqa: F401  (imports paid before the timed map)
    import oracle  # noqa: F401
    import threadpoolctl  # noqa: F401
    return os.getpid()


def chain_groups(q, k, v, beta, log_alpha, nproc):
    """Split [B, T, H, D] inputs into `nproc` groups of whole (batch, head)
    chains, each laid out as the heads of one sequence ([1, T, n, D]).
    Returns the groups and, per group, the flat chain indices (b * H + h)."""
    import numpy as np
    B, T, H, _ = q.shape
    chains = np.arange(B * H)
    parts = [p for p in np.array_split(chains, nproc) if len(p)]

    def take(x, idx):
        if x is None:
            return None
        xt = np.moveaxis(x, 1, 2).reshape((B * H, T) + x.shape[3:])   # [chain, T, ...]
        return np.moveaxis(xt[idx], 0, 1)[None]                        # [1, T, n, ...]
    groups = [(take(q, p), take(k, p), take(v, p), take(beta, p), take(log_alpha, p))
              for p in parts]
    return groups, parts


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rel_err(got, ref):
    """max |got - ref| / RMS(ref), in float64."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref * ref)))


def cpu_baseline(torch, w, kept, nproc=None):
    """The fp64 oracle over every chain of the timed headline run, on that
    run's inputs copied from the device, split over the host cores (one
    process per core, one BLAS thread each).  Returns the baseline record
    and the parity of the run's o and final state against the oracle."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import numpy as np
    inp = kept["inp"]

    def host(t):   # the rounded values, upcast exactly (fp32 holds every bf16)
        return None if t is None else t.detach().to("cpu", torch.float32).numpy()
    q, k, v, beta, la = (host(inp[n]) for n in ("q", "k", "v", "beta", "log_alpha"))
    o_gpu = kept["o"].detach().float().cpu().numpy()
    S_gpu = kept["S"].detach().float().cpu().numpy()
    avail = len(os.sched_getaffinity(0))
    P = nproc or min(avail, MAX_ORACLE_PROCS)
    groups, parts = chain_groups(q, k, v, beta, la, P)
    B, T, H, Dv = o_gpu.shape
    o_ref = np.empty((B * H, T, Dv))
    S_ref = np.empty((B * H,) + S_gpu.shape[2:])
    # spawned workers (the parent holds a GPU context, so no fork); their
    # start-up and imports are paid before the timed region
    with cf.ProcessPoolExecutor(max_workers=len(groups),
                                mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_warm_worker, range(len(groups))))
        t0 = time.perf_counter()
        results = list(ex.map(_oracle_worker, groups))
        wall = time.perf_counter() - t0
    for idx, (o, S, _) in zip(parts, results):
        o_ref[idx] = np.moveaxis(o[0], 1, 0)
        S_ref[idx] = S[0]
    o_gpu_c = np.moveaxis(o_gpu, 1, 2).reshape(B * H, T, Dv)
    S_gpu_c = S_gpu.reshape((B * H,) + S_gpu.shape[2:])
    e_o, e_S = rel_err(o_gpu_c, o_ref), rel_err(S_gpu_c, S_ref)
    tokens = B * T
    base = {"value": tokens / wall, "unit": "tokens/s", "cores": len(groups), "kind": "oracle",
            "cpu": cpu_model(), "host_cpus_visible": avail,
            "sample": f"the whole headline run: {B} sequences x {H} heads x {T} tokens "
                      f"({B * H} chains in {len(groups)} processes of one BLAS thread, "
                      f"{wall:.1f} s wall, per-process compute "
                      f"{min(r[2] for r in results):.1f}-{max(r[2] for r in results):.1f} s, "
                      f"fp64 numpy on the timed run's inputs)"}
    parity = {"o_max_abs_over_rms": e_o, "S_T_max_abs_over_rms": e_S, "tol": PARITY_TOL,
              "chains_checked": B * H, "chains_total": B * H,
              "pass": bool(e_o <= PARITY_TOL and e_S <= PARITY_TOL),
              "against": "fp64 oracle of this run (cpu_baseline)"}
    return base, parity


def decode_parity(torch, W, d, seqs=(0, 97, 255)):
    """One fresh 128-step decode pass at the full shape (N=256 x H=32),
    checked on sampled sequences (all heads, every step's output and the
    final state) against the fp64 oracle recurrence run over the same steps."""
    import numpy as np
    import gated_delta_rule_28_amd as gdr
    from oracle import gated_delta_recurrence
    inp = W.make_decode_inputs(d.N, d.H, d.Dk, d.Dv, d.steps, d.gate, d.in_dtype, seed=0,
                               device="cuda", alpha_mu=d.alpha_mu, alpha_sigma=d.alpha_sigma,
                               state_std=d.state_std)
    S0 = inp["state"].clone()
    state = inp["state"]
    o = torch.empty(d.steps, d.N, d.H, d.Dv, device="cuda", dtype=torch.float32)
    for t in range(d.steps):
        gdr.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["beta"][t],
                           inp["log_alpha"][t], state, o=o[t])
    torch.cuda.synchronize()
    idx = list(seqs)

    def pick(x):   # [steps, N, ...] -> [n, steps, ...] for the sampled sequences
        return None if x is None else np.moveaxis(W.to_f64(x)[:, idx], 0, 1)
    o_ref, S_ref = gated_delta_recurrence(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]),
                                          pick(inp["beta"]), pick(inp["log_alpha"]),
                                          W.to_f64(S0)[idx])
    e_o = rel_err(np.moveaxis(W.to_f64(o)[:, idx], 0, 1), o_ref)
    e_S = rel_err(W.to_f64(state)[idx], S_ref)
    return {"o_max_abs_over_rms": e_o, "S_max_abs_over_rms": e_S, "tol": 1e-5,
            "sequences_checked": idx, "heads": d.H, "steps": d.steps,
            "pass": bool(e_o <= 1e-5 and e_S <= 1e-5)}


def sampled_parity(torch, W, kept, chains, tol=PARITY_TOL):
    """The timed run's o and S_T on sampled (batch, head) chains, over the
    whole sequence, against the fp64 oracle recurrence on the same inputs."""
    import numpy as np
    from oracle import gated_delta_recurrence
    inp = kept["inp"]

    def pick(x):   # [B, T, H, ...] -> [n, T, 1, ...]: the sampled chains as a batch
        if x is None:
            return None
        a = W.to_f64(x)
        return np.stack([a[b, :, h] for b, h in chains])[:, :, None]
    o_ref, S_ref = gated_delta_recurrence(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]),
                                          pick(inp["beta"]), pick(inp["log_alpha"]), None)
    e_o = rel_err(pick(kept["o"]), o_ref)
    S = W.to_f64(kept["S"])
    e_S = rel_err(np.stack([S[b, h] for b, h in chains]), S_ref[:, 0])
    return {"o_max_abs_over_rms": e_o, "S_T_max_abs_over_rms": e_S, "tol": tol,
            "chains_checked": [list(c) for c in chains], "pass": bool(e_o <= tol and e_S <= tol),
            "against": "fp64 oracle recurrence on the timed run's inputs, whole sequences"}


def bwd_alg_bytes(w, grad_b=4):
    """Single-pass minimum HBM bytes of one chunk_bwd call (zero initial state,
    no loss on the final state, dS_0 written): q, k, v, dO in (input dtype),
    beta and log alpha in, dq, dk, dv out (grad_b bytes each: fp32 or bf16),
    dbeta and dlog alpha out (log alpha and its gradient per channel with the
    per-channel gate)."""
    th = w.B * w.T * w.H
    in_b = 2 if w.in_dtype == "bf16" else 4
    per_th = in_b * (2 * w.Dk + 2 * w.Dv) + 4 + grad_b * (2 * w.Dk + w.Dv) + 4
    if w.gate == "scalar":
        per_th += 8
    elif w.gate == "channel":
        per_th += 8 * w.Dk
    return th * per_th + w.B * w.H * w.Dk * w.Dv * 4


def train_line(torch, gdr, W, w, steps, warmup, settle_s=0.0):
    """One training step's chunk work on a workload: the forward and the
    backward, timed as gdr_chunk_fwd + gdr_chunk_bwd (the backward
    recomputes the forward) and as gdr_chunk_fwd_train + gdr_chunk_bwd_saved
    (the forward stores what the backward would recompute), with every
    output and the workspace preallocated."""
    inp = W.make_workload_inputs(w, seed=0, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    d_o = torch.randn(w.B, w.T, w.H, w.Dv, device="cuda", generator=g).to(inp["q"].dtype)
    ws = torch.empty(gdr.chunk_bwd_workspace_bytes(inp["q"], inp["log_alpha"]), device="cuda",
                     dtype=torch.uint8)
    f32 = dict(device="cuda", dtype=torch.float32)
    o = torch.empty(w.B, w.T, w.H, w.Dv, **f32)
    S = torch.empty(w.B, w.H, w.Dk, w.Dv, **f32)
    out = {"dq": torch.empty(w.B, w.T, w.H, w.Dk, **f32), "dk": torch.empty(w.B, w.T, w.H, w.Dk, **f32),
           "dv": torch.empty(w.B, w.T, w.H, w.Dv, **f32), "dbeta": torch.empty(w.B, w.T, w.H, **f32),
           "dlog_alpha": (None if inp["log_alpha"] is None
                          else torch.empty(*inp["log_alpha"].shape, **f32)),
           "d_initial_state": torch.empty(w.B, w.H, w.Dk, w.Dv, **f32)}
    a = (inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None)

    def plain():
        gdr.chunk_fwd(*a, o=o, final_state=S)
        gdr.chunk_bwd(*a, d_o, None, workspace=ws, out=out)

    def saved():
        gdr.chunk_fwd_train(*a, o=o, final_state=S, workspace=ws)
        gdr.chunk_bwd(*a, d_o, None, workspace=ws, out=out, saved=True)
    bf = dict(device="cuda", dtype=torch.bfloat16)
    out_b = dict(out, dq=torch.empty(w.B, w.T, w.H, w.Dk, **bf),
                 dk=torch.empty(w.B, w.T, w.H, w.Dk, **bf), dv=torch.empty(w.B, w.T, w.H, w.Dv, **bf))

    def saved_bf16():
        gdr.chunk_fwd_train(*a, o=o, final_state=S, workspace=ws)
        gdr.chunk_bwd(*a, d_o, None, workspace=ws, out=out_b, saved=True,
                      grad_dtype=torch.bfloat16)
    def saved_cast():   # fp32 gradients cast to the bf16 of the inputs afterwards
        saved()
        for n in ("dq", "dk", "dv"):
            out[n].to(torch.bfloat16)
    res = {"workload": w.name, "unit": "tokens/s"}
    for key, fn in (("recompute", plain), ("saved", saved), ("saved_fp32_grads_cast", saved_cast),
                    ("saved_bf16_grads", saved_bf16)):
        _, per = time_launches(torch, fn, steps, warmup, settle_s)
        ms = statistics.fmean(per)
        res[key] = {"ms": ms, "value": w.B * w.T / (ms * 1e-3)}
    res["value"] = res["saved_bf16_grads"]["value"]
    res["note"] = ("forward + backward of the chunk layer per step: chunk_fwd + chunk_bwd "
                   "(recompute), chunk_fwd_train + chunk_bwd(saved=True) (saved), the same "
                   "with dq, dk, dv cast to bf16 afterwards (saved_fp32_grads_cast) and written "
                   "as bf16 by the kernels (saved_bf16_grads, the value: what the autograd "
                   "wrapper runs)")
    return res


def bwd_line(torch, gdr, W, w, steps, warmup, settle_s=0.0, chains=((0, 0), (7, 15))):
    """Timed gdr_chunk_bwd calls on a chunk workload (the recompute pass, the
    reverse pass and the chunk-parallel gradients), outputs and workspace
    preallocated; then the gradients of sampled chains against the fp64
    oracle's reverse sweep."""
    import numpy as np
    from oracle import gated_delta_backward
    inp = W.make_workload_inputs(w, seed=0, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    d_o = torch.randn(w.B, w.T, w.H, w.Dv, device="cuda", generator=g).to(inp["q"].dtype)
    ws = torch.empty(gdr.chunk_bwd_workspace_bytes(inp["q"], inp["log_alpha"]), device="cuda",
                     dtype=torch.uint8)
    f32 = dict(device="cuda", dtype=torch.float32)
    out = {"dq": torch.empty(w.B, w.T, w.H, w.Dk, **f32), "dk": torch.empty(w.B, w.T, w.H, w.Dk, **f32),
           "dv": torch.empty(w.B, w.T, w.H, w.Dv, **f32), "dbeta": torch.empty(w.B, w.T, w.H, **f32),
           "dlog_alpha": (None if inp["log_alpha"] is None
                          else torch.empty(*inp["log_alpha"].shape, **f32)),
           "d_initial_state": torch.empty(w.B, w.H, w.Dk, w.Dv, **f32)}

    bf = dict(device="cuda", dtype=torch.bfloat16)
    out_b = dict(out, dq=torch.empty(w.B, w.T, w.H, w.Dk, **bf),
                 dk=torch.empty(w.B, w.T, w.H, w.Dk, **bf), dv=torch.empty(w.B, w.T, w.H, w.Dv, **bf))

    def step_b():   # dq, dk, dv written as bf16 (what a bf16 training step keeps)
        gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None, d_o,
                      None, workspace=ws, out=out_b, grad_dtype=torch.bfloat16)
    _, per_b = time_launches(torch, step_b, steps, warmup, settle_s)

    def step():
        gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None, d_o,
                      None, workspace=ws, out=out)
    wall, per = time_launches(torch, step, steps, warmup, settle_s)
    torch.cuda.synchronize()
    rounded = all(torch.equal(out_b[n], out[n].to(torch.bfloat16)) for n in ("dq", "dk", "dv"))
    mean_ms = statistics.fmean(per)
    alg_b = bwd_alg_bytes(w)
    achieved = alg_b / (mean_ms * 1e-3) / 1e9
    mean_b = statistics.fmean(per_b)
    alg_bb = bwd_alg_bytes(w, grad_b=2)
    achieved_b = alg_bb / (mean_b * 1e-3) / 1e9
    # sampled chains against the oracle
    errs = {}
    for b, h in chains:
        sl = lambda x: None if x is None else W.to_f64(x[b:b + 1, :, h:h + 1])
        ref = gated_delta_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]),
                                   sl(inp["log_alpha"]), None, sl(d_o), None)
        pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"),
                 ("dlog_alpha", "dlog_alpha")]
        for n, rn in pairs:
            if out[n] is None:
                continue
            e = rel_err(W.to_f64(out[n][b:b + 1, :, h:h + 1]), ref[rn])
            errs[n] = max(errs.get(n, 0.0), e)
        e = rel_err(W.to_f64(out["d_initial_state"][b:b + 1, h:h + 1]), ref["dS0"])
        errs["dS0"] = max(errs.get("dS0", 0.0), e)
    return {
        "workload": w.name, "unit": "tokens/s", "value": w.B * w.T / (mean_ms * 1e-3),
        "kernel_ms": {"mean": mean_ms, "median": statistics.median(per), "min": min(per)},
        "kernels": ("chunk_fwd_kda_kernel <.., mode 1> (recompute), <.., mode 2> (reverse), "
                    "chunk_bwd_kda_kernel (token gradients): one event pair around the three"
                    if w.gate == "channel" else
                    "chunk_fwd_bf16_kernel <.., mode 1> (recompute), <.., mode 2> (reverse), "
                    "chunk_bwd_grad_kernel (token gradients): one event pair around the three"),
        "workspace_bytes": int(ws.numel()),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "alg_bytes_per_launch": alg_b,
                     "note": "algorithmic bytes exclude the workspace the three passes "
                             "write and read"},
        "parity": {"max_abs_over_rms": errs, "tol": PARITY_TOL,
                   "chains_checked": [list(c) for c in chains], "chains_total": w.B * w.H,
                   "pass": bool(all(v <= PARITY_TOL for v in errs.values()))},
        "bf16_grads": {
            "value": w.B * w.T / (mean_b * 1e-3),
            "kernel_ms": {"mean": mean_b, "median": statistics.median(per_b), "min": min(per_b)},
            "roofline": {"bound": "hbm", "achieved": achieved_b, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved_b / HBM_PEAK_GBS,
                         "alg_bytes_per_launch": alg_bb},
            "equals_fp32_rounded": bool(rounded),
            "note": "grad_dtype=bf16: dq, dk, dv written as bf16 (the fp32 values rounded to "
                    "nearest even; every element compared with the fp32 call's)"},
    }


def small_lines(torch, gdr, W, settle_s):
    """The tiny fp32 workload (launch-latency bound: microseconds per call,
    warm) and the B=4, H=8, T=2048 DeltaNet / Gated DeltaNet workloads,
    timed cold (a 512 MiB write between calls: their inputs fit the 256 MB
    last-level cache) and warm."""
    out = {}
    tiny = W.by_name("gdn_f32_tiny")
    step, _, _ = chunk_setup(torch, gdr, W, tiny, torch.float32)
    _, per = time_launches(torch, step, 200, 10, settle_s)
    wall, _ = time_launches(torch, step, 200, 0)
    out["tiny_fp32"] = {"workload": tiny.name, "unit": "us per call",
                        "event_us": {"mean": 1e3 * statistics.fmean(per),
                                     "median": 1e3 * statistics.median(per),
                                     "min": 1e3 * min(per)},
                        "wall_us_per_call": 1e6 * wall / 200,
                        "note": "launch-latency bound (64 tokens, d = 16): no roofline"}
    for key, name in (("deltanet_b4h8", "deltanet_bf16_b4h8t2048"),
                      ("gdn_b4h8", "gdn_bf16_b4h8t2048")):
        wl = W.by_name(name)
        cold = chunk_line(torch, gdr, W, wl, 20, 3, torch.float32, settle_s, cold=True)
        warm = chunk_line(torch, gdr, W, wl, 20, 3, torch.float32, 0.0)
        out[key] = {"workload": name, "unit": "tokens/s",
                    "cold": {"value": wl.B * wl.T / (cold["kernel_ms"]["median"] * 1e-3),
                             "kernel_ms": cold["kernel_ms"], "roofline": cold["roofline"]},
                    "warm": {"value": wl.B * wl.T / (warm["kernel_ms"]["median"] * 1e-3),
                             "kernel_ms": warm["kernel_ms"], "roofline": warm["roofline"]},
                    "kernel": cold["kernel"], "kernel_chunk": cold["kernel_chunk"],
                    "note": "cold: 512 MiB written between timed calls (untimed); "
                            "warm: back-to-back calls"}
    return out


# ---------------------------------------------------------------------------
# counter runs


def run_counter_targets(torch, gdr, W, reps=3):
    """The three measured kernels on their workloads, `reps` launches each,
    then the calibration copy; prints a line per part."""
    for w in (W.HEADLINE, W.by_name("kda_bf16_b2h32t8192")):
        step, _, _ = chunk_setup(torch, gdr, W, w, torch.float32)
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        print(f"counters: {w.name} x{reps}", flush=True)
    d = W.DECODE
    one_pass, _, _ = decode_setup(torch, gdr, W, d)
    one_pass()
    torch.cuda.synchronize()
    print(f"counters: {d.name} x{d.steps}", flush=True)
    # the backward on the headline shape (its three kernels)
    w = W.HEADLINE
    inp = W.make_workload_inputs(w, seed=0, device="cuda")
    d_o = torch.randn(w.B, w.T, w.H, w.Dv, device="cuda").to(inp["q"].dtype)
    ws = torch.empty(gdr.chunk_bwd_workspace_bytes(inp["q"], inp["log_alpha"]), device="cuda",
                     dtype=torch.uint8)
    for _ in range(reps):
        gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None, d_o,
                      workspace=ws)
    torch.cuda.synchronize()
    del inp, d_o, ws
    print(f"counters: backward {w.name} x{reps}", flush=True)
    src = torch.empty(COPY_BYTES // 4, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.abs(src, out=dst)
    torch.cuda.synchronize()
    print(f"counters: copy {COPY_BYTES} bytes x{reps}", flush=True)
    # a bf16 GEMM of known size: 2 N^3 flops, the check of the MFMA counter scale
    a = torch.randn(GEMM_N, GEMM_N, device="cuda").to(torch.bfloat16)
    b = torch.randn(GEMM_N, GEMM_N, device="cuda").to(torch.bfloat16)
    for _ in range(reps):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    print(f"counters: bf16 GEMM {GEMM_N}^3 x{reps}", flush=True)


# The template instance each counter summary covers: the launch the bench
# line times (the backward's passes and the training forward are instances
# of the same kernel templates, with their own traffic, so the name alone is
# not enough).  Mangled template arguments: <Dk, Dv slice, output type, gate,
# erase, fused, mode> and <Dk, Dv slice, output type, erase, fused, mode>.
COUNTED_INSTANCE = {
    "chunk_fwd_bf16_kernel": "chunk_fwd_bf16_kernelILi128ELi64EfLi1ELb1ELb0ELi0E",
    "chunk_fwd_kda_kernel": "chunk_fwd_kda_kernelILi128ELi32EfLb1ELb0ELi0E",
    "recurrent_step_kernel": "recurrent_step_kernel",
}


def _pmc_means(d, counter):
    """Mean per dispatch of `counter` (summed over its dimensions), by kernel."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row.get("Dispatch_Id") or row["Correlation_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    return per


def summarize_pmc(fetch_dir, write_dir, command, out_dir=PROFILES):
    """Write profiles/traffic_<kernel>_<workload>.txt from a FETCH_SIZE run and
    a WRITE_SIZE run of `bench.py --only counters`."""
    import workloads as W
    fetch = _pmc_means(fetch_dir, "FETCH_SIZE")
    write = _pmc_means(write_dir, "WRITE_SIZE")

    def mean_of(per, pat):
        vals = [v for (k, _), v in per.items() if pat in k]
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    cf, ncf = mean_of(fetch, COPY_REGEX)
    cw, ncw = mean_of(write, COPY_REGEX)
    if not cf or not cw:
        raise RuntimeError("calibration copy not found in the counter runs")
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    os.makedirs(out_dir, exist_ok=True)
    targets = [("chunk_fwd_bf16_kernel", W.HEADLINE.name,
                chunk_alg_bytes(W.HEADLINE)),
               ("chunk_fwd_kda_kernel", "kda_bf16_b2h32t8192",
                chunk_alg_bytes(W.by_name("kda_bf16_b2h32t8192"))),
               ("recurrent_step_kernel", W.DECODE.name, decode_alg_bytes(W.DECODE))]
    for kern, wname, alg in targets:
        kf, nf = mean_of(fetch, COUNTED_INSTANCE[kern])
        kw, nw = mean_of(write, COUNTED_INSTANCE[kern])
        if kf is None or kw is None:
            print(f"{kern}: no dispatches in the counter runs", file=sys.stderr)
            continue
        traffic = kf * 1024.0 * f_scale + kw * 1024.0 * w_scale
        lines = [
            f"# HBM traffic of {kern} on {wname}, from rocprofv3 byte counters",
            "# counter runs (each on its own):",
            f"#   {command.format(counter='FETCH_SIZE', dir=fetch_dir)}",
            f"#   {command.format(counter='WRITE_SIZE', dir=write_dir)}",
            f"# summary: python bench.py --summarize-pmc {fetch_dir} {write_dir}",
            "# The counters are scaled by what they read for a plain copy of known",
            f"# size in the same runs ({COPY_BYTES} bytes read + written, torch abs).",
            f"kernel: {kern}",
            f"workload: {wname}",
            f"source_sha256: {source_hash(kern)}",
            f"dispatches: fetch {nf}, write {nw}",
            f"fetch_kib_per_dispatch: {kf:.1f}",
            f"write_kib_per_dispatch: {kw:.1f}",
            f"copy_dispatches: fetch {ncf}, write {ncw}",
            f"copy_fetch_kib_per_dispatch: {cf:.1f}",
            f"copy_write_kib_per_dispatch: {cw:.1f}",
            f"fetch_scale: {f_scale:.4f}",
            f"write_scale: {w_scale:.4f}",
            f"read_bytes_per_launch: {kf * 1024.0 * f_scale:.0f}",
            f"written_bytes_per_launch: {kw * 1024.0 * w_scale:.0f}",
            f"traffic_bytes_per_launch: {traffic:.0f}",
            f"algorithmic_bytes_per_launch: {alg}",
            f"traffic_over_algorithmic: {traffic / alg:.3f}",
        ]
        path = traffic_file(kern, wname, out_dir)
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {path}: traffic/alg = {traffic / alg:.3f}")
    return 0


def summarize_mfma(ops_dir, util_dir, command, out_dir=PROFILES):
    """Write profiles/mfma_<kernel>_<workload>.txt from a run of the MFMA
    operation and busy-cycle counters and a run of the derived MfmaUtil of
    `bench.py --only counters`."""
    import workloads as W
    mops = _pmc_means(ops_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    insts = _pmc_means(ops_dir, "SQ_INSTS_MFMA")
    busy = _pmc_means(ops_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    util = _pmc_means(util_dir, "MfmaUtil")

    def mean_of(per, pat):
        vals = [v for (k, _), v in per.items() if pat in k]
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    gm, ngm = mean_of(mops, GEMM_REGEX)
    gemm_flops = 2.0 * GEMM_N ** 3
    gemm_ratio = (gm * 512.0 / gemm_flops) if gm else None
    os.makedirs(out_dir, exist_ok=True)
    kda = W.by_name("kda_bf16_b2h32t8192")
    targets = [("chunk_fwd_bf16_kernel", W.HEADLINE.name,
                chunk_alg_flops(W.HEADLINE, KERNEL_CHUNK["scalar"])),
               ("chunk_fwd_kda_kernel", kda.name, chunk_alg_flops(kda, KERNEL_CHUNK["channel"]))]
    for kern, wname, alg in targets:
        m, nm = mean_of(mops, COUNTED_INSTANCE[kern])
        u, nu = mean_of(util, COUNTED_INSTANCE[kern])
        ni, _ = mean_of(insts, COUNTED_INSTANCE[kern])
        nb, _ = mean_of(busy, COUNTED_INSTANCE[kern])
        if m is None or u is None:
            print(f"{kern}: no dispatches in the counter runs", file=sys.stderr)
            continue
        issued = m * 512.0
        lines = [
            f"# MFMA counters of {kern} on {wname}, from rocprofv3",
            "# counter runs (each on its own):",
            f"#   {command.format(counter='SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES', dir=ops_dir)}",
            f"#   {command.format(counter='MfmaUtil', dir=util_dir)}",
            f"# summary: python bench.py --summarize-mfma {ops_dir} {util_dir}",
            "# mfma_busy_frac = MfmaUtil / 100, the tool's derived metric: MFMA-busy",
            "#   SIMD cycles summed over the GPU / (GPU-active cycles x 1024 SIMDs).",
            "# issued_bf16_flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the tool's",
            "#   MfmaFlopsBF16); it counts every hi/lo split product the kernel issues.",
            f"# scale check: a bf16 GEMM of {GEMM_N}^3 (2 N^3 = {gemm_flops:.4e} flops) in the same",
            "#   run reads MOPS x 512 / (2 N^3) = gemm_issued_over_exact below.",
            f"kernel: {kern}",
            f"workload: {wname}",
            f"source_sha256: {source_hash(kern)}",
            f"dispatches: ops {nm}, util {nu}",
            f"mfma_instructions_per_launch: {ni:.0f}" if ni is not None else "mfma_instructions_per_launch: none",
            f"mfma_busy_simd_cycles_per_launch: {nb:.0f}" if nb is not None else "mfma_busy_simd_cycles_per_launch: none",
            f"mfma_busy_frac: {u / 100.0:.4f}",
            f"issued_bf16_flops_per_launch: {issued:.6e}",
            f"algorithmic_flops_per_launch: {alg:.6e}",
            f"issued_over_algorithmic: {issued / alg:.3f}",
            f"gemm_dispatches: {ngm}",
            f"gemm_issued_over_exact: {gemm_ratio:.4f}" if gemm_ratio else "gemm_issued_over_exact: none",
        ]
        path = mfma_file(kern, wname, out_dir)
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {path}: busy {u:.1f}%, issued/alg {issued / alg:.2f}")
    return 0


# ---------------------------------------------------------------------------


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="untimed seconds of the same launches before each line's warm-up, "
                         "so the timed steps run at the settled GPU clock")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline line only (no bf16-output, KDA and decode lines)")
    ap.add_argument("--only", choices=["counters"], default=None)
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("OPS_DIR", "UTIL_DIR"))
    ap.add_argument("--pmc-command", default="rocprofv3 --pmc {counter} --kernel-include-regex "
                    "'chunk_fwd|chunk_bwd|recurrent_step|AbsFunctor|Cijk' --output-format csv -d {dir} "
                    "-o pmc -- python3 bench.py --only counters")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.pmc_command)
    if args.summarize_mfma:
        return summarize_mfma(*args.summarize_mfma, args.pmc_command)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here "
              "(every (batch, head) chain is independent, so batch or heads shard "
              "across GPUs with no exchange).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import gated_delta_rule_28_amd as gdr
    import workloads as W

    if args.only == "counters":
        run_counter_targets(torch, gdr, W)
        return 0

    w = W.HEADLINE
    kept = {}
    head = chunk_line(torch, gdr, W, w, args.steps, args.warmup, torch.float32, args.settle_s,
                      keep=kept)
    copy = None if args.no_extra else copy_ceiling(torch)
    rec = {
        "metric": "tokens/s gated-delta chunk fwd (H=16,d=128,T=4096) + % MFMA/HBM roofline",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": args.settle_s,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "Dk": w.Dk, "Dv": w.Dv,
                   "gate": "scalar (Gated DeltaNet)", "kernel_chunk": head["kernel_chunk"],
                   "inputs": "bf16 q/k/v, fp32 beta/log_alpha, fp32 state, fp32 output",
                   "parallelism": "single GPU"},
        "roofline": dict(with_copy_frac(head["roofline"], copy), kernel=head["kernel"],
                         kernel_ms=head["kernel_ms"]),
        "mfma_alg": head["mfma_alg"],
        "mfma_counter": head["mfma_counter"],
        "copy_ceiling": copy,
    }
    if not args.no_cpu:
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(torch, w, kept)
    kept.clear()
    keys = ("workload", "value", "kernel", "kernel_chunk", "kernel_ms", "roofline", "mfma_alg",
            "mfma_counter")
    if not args.no_extra:
        nb = max(5, args.steps // 2)
        b = chunk_line(torch, gdr, W, w, nb, 2, torch.bfloat16, args.settle_s)
        rec["bf16_output"] = {"value": w.B * w.T / (b["kernel_ms"]["mean"] * 1e-3),
                              "unit": "tokens/s", "kernel_ms": b["kernel_ms"],
                              "roofline": b["roofline"]}
        kept_kda = {}
        kda = chunk_line(torch, gdr, W, W.by_name("kda_bf16_b2h32t8192"), nb, 2, torch.float32,
                         args.settle_s, keep=kept_kda)
        rec["kda"] = {k: kda[k] for k in keys}
        rec["kda"]["roofline"] = with_copy_frac(kda["roofline"], copy)
        rec["kda"]["unit"] = "tokens/s"
        rec["kda"]["parity"] = sampled_parity(torch, W, kept_kda, ((0, 0), (1, 31)))
        kept_kda.clear()
        # the erase-free variant (additive write) through the same kernels:
        # the Mamba-2 / SSD decay on the headline shape, GLA's on the KDA shape
        for key, wl in (("additive_scalar", w), ("additive_channel", W.by_name("kda_bf16_b2h32t8192"))):
            ln = chunk_line(torch, gdr, W, wl, nb, 2, torch.float32, args.settle_s, erase=False)
            rec[key] = {k: ln[k] for k in keys if k != "mfma_counter"}
            rec[key]["unit"] = "tokens/s"
            rec[key]["variant"] = "no erase term (S = a S + b k v^T)"
        # the fused prologue (q, k L2 normalisation, sigmoid b, softplus
        # decay) and SiLU output gate through the same kernels
        for key, wl in (("fused", w), ("kda_fused", W.by_name("kda_bf16_b2h32t8192"))):
            ln = chunk_line(torch, gdr, W, wl, nb, 2, torch.float32, args.settle_s, fused=True)
            rec[key] = {k: ln[k] for k in keys if k != "mfma_counter"}
            rec[key]["unit"] = "tokens/s"
            rec[key]["variant"] = ("fused prologue (q, k L2 norm, sigmoid b, softplus decay) "
                                   "and SiLU output gate")
            unfused_ms = (head if key == "fused" else kda)["kernel_ms"]["mean"]
            rec[key]["separate_passes"] = separate_passes_line(
                torch, gdr, W, wl, nb, 2, args.settle_s, copy["GB/s"] if copy else None, unfused_ms)
        rec["decode"] = decode_line(torch, gdr, W, W.DECODE, settle_s=args.settle_s)
        rec["decode"]["roofline"] = with_copy_frac(rec["decode"]["roofline"], copy)
        rec["decode"]["parity"] = decode_parity(torch, W, W.DECODE)
        rec.update(small_lines(torch, gdr, W, args.settle_s))
        rec["backward"] = bwd_line(torch, gdr, W, w, nb, 2, args.settle_s)
        rec["kda_backward"] = bwd_line(torch, gdr, W, W.by_name("kda_bf16_b2h32t8192"), nb, 2,
                                       args.settle_s, chains=((0, 0), (1, 31)))
        rec["train_step"] = train_line(torch, gdr, W, w, nb, 2, args.settle_s)
        rec["kda_train_step"] = train_line(torch, gdr, W, W.by_name("kda_bf16_b2h32t8192"), nb,
                                           2, args.settle_s)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
