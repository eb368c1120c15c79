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


# kernel names as rocprofv3 reports them (mangled): the timed forward launch,
# and a pass of the backward, an instance of the same template
FWD = ("_ZN3gdr12_GLOBAL__N_121chunk_fwd_bf16_kernelILi128ELi64EfLi1ELb1ELb0ELi0EEEvPKDF16bS3_"
       "S3_PKfS5_S5_PT1_PfiiiiS3_S8_S8_S8_")
BWD_PASS = FWD.replace("ELi0EEEv", "ELi1EEEv")


def test_counter_summary_scales_by_the_copy(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024.0
    kern = FWD
    # the counters read half of the true bytes: the copy calibrates that away;
    # the backward's pass (same template, other traffic) is not counted
    _write_csv(tmp_path / "f", "FETCH_SIZE",
               [("at::native::vectorized_elementwise_kernel<4, at::native::AbsFunctor<float>>", copy_kib / 2)] * 3 + [(kern, 1000.0), (kern, 1200.0), (BWD_PASS, 9.0e6)])
    _write_csv(tmp_path / "w", "WRITE_SIZE",
               [("at::native::vectorized_elementwise_kernel<4, at::native::AbsFunctor<float>>", copy_kib / 4)] * 3 + [(kern, 500.0), (kern, 500.0), (BWD_PASS, 9.0e6)])
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


def test_chain_groups_cover_every_chain_once():
    import numpy as np
    B, T, H, D = 2, 5, 3, 4
    rng = np.random.default_rng(0)
    q = rng.standard_normal((B, T, H, D))
    beta = rng.standard_normal((B, T, H))
    groups, parts = bench.chain_groups(q, q, q, beta, None, 4)
    assert sorted(np.concatenate(parts).tolist()) == list(range(B * H))
    for (gq, _, _, gb, gla), idx in zip(groups, parts):
        assert gla is None and gq.shape == (1, T, len(idx), D) and gb.shape == (1, T, len(idx))
        for j, c in enumerate(idx):
            assert np.array_equal(gq[0, :, j], q[c // H, :, c % H])
            assert np.array_equal(gb[0, :, j], beta[c // H, :, c % H])


def test_cpu_baseline_splits_chains_and_checks_parity():
    """The oracle baseline over two processes reproduces the oracle run on
    the whole input, and its parity field catches a wrong output value."""
    import torch
    from oracle import gated_delta_recurrence
    w = W.HEADLINE
    inp = W.make_chunk_inputs(2, 9, 3, 16, 16, "scalar", "bf16", seed=3)
    a = {k: W.to_f64(v) for k, v in inp.items()}
    o, S = gated_delta_recurrence(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"])
    kept = {"inp": inp, "o": torch.from_numpy(o).float(), "S": torch.from_numpy(S).float()}
    base, parity = bench.cpu_baseline(torch, w, kept, nproc=2)
    assert base["cores"] == 2 and base["kind"] == "oracle"
    assert parity["pass"] and parity["o_max_abs_over_rms"] < 1e-6
    assert parity["chains_checked"] == 6
    o_bad = o.copy()
    o_bad[1, 4, 2, 7] += 0.01 * float((o * o).mean() ** 0.5)
    kept["o"] = torch.from_numpy(o_bad).float()
    _, parity = bench.cpu_baseline(torch, w, kept, nproc=2)
    assert not parity["pass"] and parity["o_max_abs_over_rms"] > 5e-3


def test_mfma_summary(tmp_path):
    kern = FWD
    gemm = "Cijk_Alik_Bljk_BBS_BH_MT256x256x64"
    gemm_mops = 2.0 * bench.GEMM_N ** 3 / 512.0
    _write_csv(tmp_path / "o", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               [(gemm, gemm_mops)] * 2 + [(kern, 1.0e8), (kern, 1.0e8), (BWD_PASS, 5.0e9)])
    _write_csv(tmp_path / "u", "MfmaUtil", [(gemm, 80.0), (kern, 25.0), (kern, 27.0), (BWD_PASS, 90.0)])
    out = tmp_path / "prof"
    assert bench.summarize_mfma(str(tmp_path / "o"), str(tmp_path / "u"),
                                "cmd {counter} {dir}", out_dir=str(out)) == 0
    got = bench.read_mfma("chunk_fwd_bf16_kernel", W.HEADLINE.name, root=str(out))
    assert got["busy_frac"] == pytest.approx(0.26)
    assert got["issued_flops_per_launch"] == pytest.approx(1.0e8 * 512)
    text = open(bench.mfma_file("chunk_fwd_bf16_kernel", W.HEADLINE.name, str(out))).read()
    assert "gemm_issued_over_exact: 1.0000" in text
