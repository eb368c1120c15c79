"""Host-side logic of bench.py: algorithmic counts, the multi-GPU refusal,
and the counter summary that feeds the roofline's measured traffic."""

import csv
import os

import pytest

import bench
import workloads as W


def test_headline_algorithmic_counts():
    w = W.HEADLINE
    # q, k, v bf16 + beta + log alpha + fp32 o per token-head, plus the final state
    th = w.B * w.T * w.H
    assert bench.chunk_alg_bytes(w) == th * (2 * 384 + 4 + 4 + 4 * 128) + w.B * w.H * 128 * 128 * 4
    assert bench.chunk_alg_bytes(w) == 683_671_552
    # 139,136 flop per token-head at 64-token chunks
    assert bench.chunk_alg_flops(w, 64) == th * 139_136
    # without the erase term: 4 dk dv + C dk + (C + 1) dv = 82,048 at C = 64
    assert bench.chunk_alg_flops(w, 64, erase=False) == th * 82_048
    d = W.DECODE
    assert bench.decode_alg_bytes(d) == 256 * 32 * (2 * 4 * 128 * 128 + 2 * 384 + 8 + 4 * 128)


def test_fused_line_counts_the_output_gate():
    # the fused lines read the output gate (dtype of q) once per output value
    for w in (W.HEADLINE, W.by_name("kda_bf16_b2h32t8192")):
        th = w.B * w.T * w.H
        assert bench.chunk_alg_bytes(w, out_gate=True) - bench.chunk_alg_bytes(w) == th * 2 * w.Dv
    # the KDA shape: per-channel log decays (4 Dk bytes per token-head)
    k = W.by_name("kda_bf16_b2h32t8192")
    th = k.B * k.T * k.H
    assert bench.chunk_alg_bytes(k) == th * (2 * 384 + 4 + 4 * 128 + 4 * 128) + k.B * k.H * 128 * 128 * 4


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _write_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, ["Dispatch_Id", "Correlation_Id", "Kernel_Name",
                                 "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (kern, val) in enumerate(rows):
            # each dispatch reports its counter in two dimensions that add up
            for part in (0.25, 0.75):
                wr.writerow({"Dispatch_Id": i, "Correlation_Id": i, "Kernel_Name": kern,
                             "Counter_Name": counter, "Counter_Value": val * part})


def test_counter_summary_scales_by_the_copy(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024.0
    kern = "void gdr::(anonymous namespace)::chunk_fwd_bf16_kernel<128, 64, float, 1>(...)"
    # the counters read half of the true bytes: the copy calibrates that away
    _write_csv(tmp_path / "f", "FETCH_SIZE",
               [("at::native::vectorized_elementwise_kernel<4, at::native::AbsFunctor<float>>", copy_kib / 2)] * 3 + [(kern, 1000.0), (kern, 1200.0)])
    _write_csv(tmp_path / "w", "WRITE_SIZE",
               [("at::native::vectorized_elementwise_kernel<4, at::native::AbsFunctor<float>>", copy_kib / 4)] * 3 + [(kern, 500.0), (kern, 500.0)])
    out = tmp_path / "prof"
    assert bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "cmd {counter} {dir}",
                               out_dir=str(out)) == 0
    got = bench.read_traffic("chunk_fwd_bf16_kernel", W.HEADLINE.name, root=str(out))
    assert got == pytest.approx((1100.0 * 2 + 500.0 * 4) * 1024.0, abs=1.0)
    # a summary taken on another kernel source is not used
    path = bench.traffic_file("chunk_fwd_bf16_kernel", W.HEADLINE.name, str(out))
    text = open(path).read().replace(bench.source_hash("chunk_fwd_bf16_kernel"), "0" * 16)
    open(path, "w").write(text)
    assert bench.read_traffic("chunk_fwd_bf16_kernel", W.HEADLINE.name, root=str(out)) is None
