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
heads, 128 consecutive steps, eager and as one HIP graph).
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
}
# the plain copy used to calibrate the byte counters: |x| over 1 GiB of fp32
COPY_BYTES = 1 << 30
COPY_REGEX = "AbsFunctor"


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


def time_launches(torch, fn, steps, warmup, settle_s=0.0):
    """Run fn for `settle_s` seconds of wall time (untimed: the GPU clock
    ramps up over the first ~80 launches of a fresh process and the first
    launches run up to ~20% slower), then `warmup` times, then exactly
    `steps` times between two full synchronisations; each timed call is also
    bracketed by events on the current stream, the stream the kernels are
    launched on."""
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
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    return wall, per


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


def chunk_setup(torch, gdr, W, w, out_dtype, erase=True, fused=False):
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
    return step, o, S


def chunk_line(torch, gdr, W, w, steps, warmup, out_dtype, settle_s=0.0, erase=True,
               fused=False):
    step, o, S = chunk_setup(torch, gdr, W, w, out_dtype, erase, fused)
    wall, per = time_launches(torch, step, steps, warmup, settle_s)
    if not (bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())):
        raise RuntimeError(f"non-finite output in the timed run of {w.name}")
    out_b = 2 if out_dtype == torch.bfloat16 else 4
    kern = KERNEL_OF_GATE[w.gate]
    C = KERNEL_CHUNK[w.gate]
    mean_ms = statistics.fmean(per)
    alg_b = chunk_alg_bytes(w, out_b, out_gate=fused)
    alg_f = chunk_alg_flops(w, C, erase)
    achieved = alg_b / (mean_ms * 1e-3) / 1e9
    # counter traffic is taken for the erasing, unfused fp32-output launches only
    traffic = read_traffic(kern, w.name) if out_b == 4 and erase and not fused else None
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


def cpu_baseline(W, w, batches=8):
    """The fp64 oracle on a bounded sample of the same workload: `batches`
    sequences x all heads x all tokens, the same seeded inputs, one thread."""
    from oracle import gated_delta_recurrence
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    inp = W.make_chunk_inputs(batches, w.T, w.H, w.Dk, w.Dv, w.gate, w.in_dtype, seed=0,
                              device="cpu", alpha_mu=w.alpha_mu, alpha_sigma=w.alpha_sigma)
    a = {k: W.to_f64(v) for k, v in inp.items()}
    t0 = time.perf_counter()
    if threadpool_limits is not None:
        with threadpool_limits(1):
            gated_delta_recurrence(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"])
    else:
        gated_delta_recurrence(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"])
    dt = time.perf_counter() - t0
    tokens = batches * w.T
    return {"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{batches} of {w.B} sequences x {w.H} heads x {w.T} tokens "
                      f"({tokens * w.H} token-heads, {dt:.1f} s wall, fp64 numpy, 1 thread)"}


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
    src = torch.empty(COPY_BYTES // 4, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.abs(src, out=dst)
    torch.cuda.synchronize()
    print(f"counters: copy {COPY_BYTES} bytes x{reps}", flush=True)


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
        kf, nf = mean_of(fetch, kern)
        kw, nw = mean_of(write, kern)
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
    ap.add_argument("--pmc-command", default="rocprofv3 --pmc {counter} --kernel-include-regex "
                    "'chunk_fwd|recurrent_step|AbsFunctor' --output-format csv -d {dir} -o pmc "
                    "-- python3 bench.py --only counters")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.pmc_command)
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
    head = chunk_line(torch, gdr, W, w, args.steps, args.warmup, torch.float32, args.settle_s)
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
        "roofline": dict(head["roofline"], kernel=head["kernel"], kernel_ms=head["kernel_ms"]),
        "mfma_alg": head["mfma_alg"],
    }
    if not args.no_extra:
        nb = max(5, args.steps // 2)
        b = chunk_line(torch, gdr, W, w, nb, 2, torch.bfloat16, args.settle_s)
        rec["bf16_output"] = {"value": w.B * w.T / (b["kernel_ms"]["mean"] * 1e-3),
                              "unit": "tokens/s", "kernel_ms": b["kernel_ms"],
                              "roofline": b["roofline"]}
        kda = chunk_line(torch, gdr, W, W.by_name("kda_bf16_b2h32t8192"), nb, 2, torch.float32,
                         args.settle_s)
        rec["kda"] = {k: kda[k] for k in ("workload", "value", "kernel", "kernel_chunk",
                                          "kernel_ms", "roofline", "mfma_alg")}
        rec["kda"]["unit"] = "tokens/s"
        # the erase-free variant (additive write) through the same kernels:
        # the Mamba-2 / SSD decay on the headline shape, GLA's on the KDA shape
        for key, wl in (("additive_scalar", w), ("additive_channel", W.by_name("kda_bf16_b2h32t8192"))):
            ln = chunk_line(torch, gdr, W, wl, nb, 2, torch.float32, args.settle_s, erase=False)
            rec[key] = {k: ln[k] for k in ("workload", "value", "kernel", "kernel_chunk",
                                           "kernel_ms", "roofline", "mfma_alg")}
            rec[key]["unit"] = "tokens/s"
            rec[key]["variant"] = "no erase term (S = a S + b k v^T)"
        # the fused prologue (q, k L2 normalisation, sigmoid b, softplus
        # decay) and SiLU output gate through the same kernels
        for key, wl in (("fused", w), ("kda_fused", W.by_name("kda_bf16_b2h32t8192"))):
            ln = chunk_line(torch, gdr, W, wl, nb, 2, torch.float32, args.settle_s, fused=True)
            rec[key] = {k: ln[k] for k in ("workload", "value", "kernel", "kernel_chunk",
                                           "kernel_ms", "roofline", "mfma_alg")}
            rec[key]["unit"] = "tokens/s"
            rec[key]["variant"] = ("fused prologue (q, k L2 norm, sigmoid b, softplus decay) "
                                   "and SiLU output gate")
        rec["decode"] = decode_line(torch, gdr, W, W.DECODE, settle_s=args.settle_s)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(W, w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
