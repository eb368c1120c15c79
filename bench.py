"""Benchmark of the gated delta-rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode]

One "step" is one gdr_chunk_fwd call over the Gated DeltaNet layer workload
(B=8, H=16, T=4096, d_k = d_v = 128, chunk 64, bf16 q/k/v, fp32 state, fp32
output): every row of the chunkwise hot path (in-chunk log-decay cumsum,
K K^T / Q K^T with the decay, the unit-lower triangular solve, the WY
factors, the serial inter-chunk state pass and the outputs) runs inside
that one kernel.  Inputs are seeded synthetic tensors already resident in
HBM when the timed region starts.

Printed: ONE JSON line with tokens/s (B*T per step time), the roofline of
the chunk kernel (HBM-bound: algorithmic bytes / measured kernel time / 8
TB/s), the fp64 oracle timed on the host cores on a bounded sample, and a
secondary measurement of the batched decode step (256 sequences x 32 heads,
128 consecutive steps, HBM-bound state read-modify-write).
"""

import argparse
import json
import os
import sys
import time

import torch

import gated_delta_rule_28_amd as gdr
import workloads as W

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def chunk_alg_bytes(w, out_bytes=4):
    """Single-pass minimum HBM bytes of one chunk_fwd call (zero initial
    state, final state written): q, k, v in, beta and log alpha in, o out."""
    th = w.B * w.T * w.H
    in_b = 2 if w.in_dtype == "bf16" else 4
    per_th = in_b * (2 * w.Dk + w.Dv) + 4
    if w.gate == "scalar":
        per_th += 4
    elif w.gate == "channel":
        per_th += 4 * w.Dk
    per_th += out_bytes * w.Dv
    return th * per_th + w.B * w.H * w.Dk * w.Dv * 4


def chunk_alg_flops(w):
    """Algorithmic flops per call: per token-head 6 dk dv (W S, Q S, K~^T U)
    + 2 C dk (Q K^T and K K^T halves) + (C-1)(dk+dv) (solve on [bV | bgK])
    + (C+1) dv (masked P U)."""
    C, dk, dv = w.chunk, w.Dk, w.Dv
    per_th = 6 * dk * dv + 2 * C * dk + (C - 1) * (dk + dv) + (C + 1) * dv
    return w.B * w.T * w.H * per_th


def decode_alg_bytes(w):
    """Per step: fp32 state read + written, q/k/v in, beta/log alpha in, o out."""
    n = w.N * w.H
    in_b = 2 if w.in_dtype == "bf16" else 4
    return n * (2 * 4 * w.Dk * w.Dv + in_b * (2 * w.Dk + w.Dv) + 8 + 4 * w.Dv)


def time_launches(fn, steps, warmup):
    """Run fn warmup times, then exactly `steps` times between two full
    synchronisations; every launch is also bracketed by events on the
    current stream (the stream the kernels are launched on)."""
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


def bench_chunk(w, steps, warmup, out_dtype=torch.float32):
    inp = W.make_workload_inputs(w, seed=0, device="cuda")
    o = torch.empty(w.B, w.T, w.H, w.Dv, device="cuda", dtype=out_dtype)
    S = torch.empty(w.B, w.H, w.Dk, w.Dv, device="cuda", dtype=torch.float32)

    def step():
        gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], None,
                      chunk=w.chunk, out_dtype=out_dtype, o=o, final_state=S)

    wall, per = time_launches(step, steps, warmup)
    if not bool(torch.isfinite(o).all()):
        raise RuntimeError("non-finite output in the timed run")
    return wall, per


def bench_decode(w, passes, warmup_passes):
    inp = W.make_decode_inputs(w.N, w.H, w.Dk, w.Dv, w.steps, w.gate, w.in_dtype, seed=0,
                               device="cuda", alpha_mu=w.alpha_mu, alpha_sigma=w.alpha_sigma,
                               state_std=w.state_std)
    state = inp["state"]
    o = torch.empty(w.N, w.H, w.Dv, device="cuda", dtype=torch.float32)

    def one_pass():
        # the workload: `steps` consecutive tokens, each step consumes the state
        for t in range(w.steps):
            gdr.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["beta"][t],
                               inp["log_alpha"][t], state, o=o)

    wall, per = time_launches(one_pass, passes, warmup_passes)
    return wall, per


def cpu_baseline(w, batches=6):
    """The fp64 oracle on a bounded sample of the same workload: `batches`
    sequences x all heads x all tokens, the same seeded inputs."""
    import numpy as np  # noqa: F401
    from oracle import gated_delta_recurrence
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    inp = W.make_chunk_inputs(batches, w.T, w.H, w.Dk, w.Dv, w.gate, w.in_dtype, seed=0,
                              device="cpu", alpha_mu=w.alpha_mu, alpha_sigma=w.alpha_sigma)
    a = {k: W.to_f64(v) for k, v in inp.items()}
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    if ctx:
        with ctx:
            gated_delta_recurrence(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"])
    else:
        gated_delta_recurrence(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"])
    dt = time.perf_counter() - t0
    tokens = batches * w.T
    return {"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{batches} of {w.B} sequences x {w.H} heads x {w.T} tokens "
                      f"({tokens * w.H} token-heads, {dt:.1f} s wall, fp64 numpy, 1 thread)"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) chain is independent; see the sharding notes).",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    w = W.HEADLINE
    wall, per = bench_chunk(w, args.steps, args.warmup)
    ms_per_step = 1e3 * wall / args.steps
    kern_ms = sum(per) / len(per)
    tokens = w.B * w.T
    alg_bytes = chunk_alg_bytes(w)
    alg_flops = chunk_alg_flops(w)
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    rec = {
        "metric": "tokens/s gated-delta chunk fwd (H=16,d=128,T=4096) + % MFMA/HBM roofline",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "Dk": w.Dk, "Dv": w.Dv,
                   "chunk": w.chunk, "gate": "scalar (Gated DeltaNet)",
                   "inputs": "bf16 q/k/v, fp32 beta/log_alpha, fp32 state, fp32 output",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "chunk_fwd_bf16_kernel", "kernel_ms": kern_ms,
                     "alg_bytes_per_launch": alg_bytes},
        "mfma_alg": {"achieved_tflops": alg_flops / (kern_ms * 1e-3) / 1e12,
                     "peak_tflops": BF16_PEAK_TFLOPS,
                     "frac": alg_flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "alg_flops_per_launch": alg_flops},
    }
    # bf16-output variant of the same step (secondary)
    wall_b, per_b = bench_chunk(w, max(5, args.steps // 5), 2, out_dtype=torch.bfloat16)
    kb = sum(per_b) / len(per_b)
    rec["bf16_output"] = {"value": tokens / (kb * 1e-3), "unit": "tokens/s", "kernel_ms": kb,
                          "hbm_frac": chunk_alg_bytes(w, 2) / (kb * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if not args.no_decode:
        d = W.DECODE
        passes = 3
        wall_d, per_d = bench_decode(d, passes, 1)
        ms_pass = sum(per_d) / len(per_d)
        ms_step = ms_pass / d.steps
        db = decode_alg_bytes(d)
        rec["decode"] = {"workload": d.name, "value": d.N * d.steps / (ms_pass * 1e-3),
                         "unit": "tokens/s", "ms_per_token_step": ms_step,
                         "roofline": {"bound": "hbm", "achieved": db / (ms_step * 1e-3) / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": db / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                      "alg_bytes_per_launch": db}}
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
