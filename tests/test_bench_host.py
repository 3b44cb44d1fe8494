"""Host-side logic of bench.py (CPU only): the work counts behind its figures, the oracle's row
sample, and the writers that turn rocprofv3 CSVs into the summaries under profiles/."""

from __future__ import annotations

import csv
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import fox_inputs as fi  # noqa: E402


def test_forward_flops_count_causal_pairs():
    cfg = fi.FWD["c4"]
    # 4 d flop per (i, j <= i) pair, over every (b, h)
    pairs = sum(i + 1 for i in range(cfg.N))
    assert bench.fwd_flops(cfg) == 4 * cfg.d * pairs * cfg.B * cfg.H
    assert abs(bench.fwd_flops(cfg) - 2199.157e9) < 1e6  # the figure the bench line reports


def test_decode_bytes_parts():
    cfg = fi.DECODE["c5"]
    b = bench.decode_bytes(cfg)
    eb = 2
    kv = 2 * cfg.S * cfg.H * cfg.L * cfg.d * eb
    assert b["kv"] == kv
    # the c cache is read for the L-1 slots before the new one; q, log f_new read; O, lse, c written
    assert b["read"] == kv + cfg.S * cfg.H * (cfg.L - 1) * 4 + cfg.S * cfg.H * (cfg.d * eb + 4)
    assert b["write"] == cfg.S * cfg.H * (cfg.d * eb + 8)
    assert b["total"] == b["read"] + b["write"]
    lens = [5, cfg.L, 1]
    small = bench.decode_bytes(type(cfg)(**{**cfg.__dict__, "S": 3}), lens=lens)
    assert small["kv"] == 2 * cfg.H * sum(lens) * cfg.d * eb


def test_sample_rows_cover_every_stride_and_the_tail():
    for n in (1, 100, 16384):
        r = bench.sample_rows(n)
        assert np.all(np.diff(r) > 0) and r[0] == 0 and r[-1] == n - 1
        assert set(range(0, n, 64)) <= set(r.tolist())
        assert set(range(max(0, n - 128), n)) <= set(r.tolist())


def test_demangle_names_own_kernels():
    m = "_ZN3fox12_GLOBAL__N_120fwd_bf16_pipe_kernelILi128ELi8ELi1ELb0ELb1ELb0EEEvPKDF16bS3_S3_PKfPDF16b"
    assert bench._demangle(m) == "fwd_bf16_pipe_kernel<128,8,1,0,1,0>"
    assert bench._demangle("_ZN3fox12_GLOBAL__N_120bwd_gate_rows_kernelEPKf") == "bwd_gate_rows_kernel"
    plain = "void fox::(anonymous namespace)::bwd_pre_kernel<128>(x)"
    assert bench._demangle(plain) == plain


def _counter_csv(path, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    # a copy of 1 GiB whose FETCH_SIZE reads half its bytes and whose WRITE_SIZE reads them whole
    kib = bench.COPY_CAL_BYTES / 1024
    _counter_csv(tmp_path / "cf.csv", [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2, 0, 1)])
    _counter_csv(tmp_path / "cw.csv", [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib, 0, 1)])
    # two dispatches of a kernel: 1000 and 3000 KiB fetched, 500 KiB written each
    _counter_csv(tmp_path / "f.csv", [(1, "kernA", "FETCH_SIZE", 1000.0, 0, 1), (2, "kernA", "FETCH_SIZE", 3000.0, 0, 1),
                                      (3, "other", "FETCH_SIZE", 9e9, 0, 1)])
    _counter_csv(tmp_path / "w.csv", [(1, "kernA", "WRITE_SIZE", 500.0, 0, 1), (2, "kernA", "WRITE_SIZE", 500.0, 0, 1)])
    out = tmp_path / "t.txt"
    args = types.SimpleNamespace(fetch_csv=str(tmp_path / "f.csv"), write_csv=str(tmp_path / "w.csv"),
                                 copy_fetch_csv=str(tmp_path / "cf.csv"), copy_write_csv=str(tmp_path / "cw.csv"),
                                 kernel_match="kernA", kernel="kernA<1>", workload="c2", kind="fwd",
                                 alg_bytes=2048.0 * 1024, out=str(out))
    bench.write_traffic_summary(args)
    kv = bench._read_summary(str(out))
    assert float(kv["read_bytes_per_launch"]) == pytest.approx(2000 * 1024 * 2)  # mean 2000 KiB, factor 2
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(500 * 1024)
    assert float(kv["traffic_over_algorithmic"]) == pytest.approx((4000 + 500) / 2048, rel=1e-3)
    assert kv["source_digest"] == bench.kernel_source_digest("fwd")


def test_stored_traffic_requires_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda kind: "feedbeef")
    summary = prof / "x_traffic.txt"
    summary.write_text("workload: c9\nkernel: k<1>\nsource_digest: 0000\ntraffic_bytes_per_launch: 123\n")
    assert bench.stored_traffic("c9", "k<1>", "fwd") is None  # taken on other sources
    summary.write_text("workload: c9\nkernel: k<1>\nsource_digest: feedbeef\ntraffic_bytes_per_launch: 123\n")
    assert bench.stored_traffic("c9", "k<1>", "fwd") == 123.0
    assert bench.stored_traffic("c9", "k<2>", "fwd") is None


def test_mfma_summary_from_counters(tmp_path):
    cfg = fi.FWD["c2"]
    pairs = cfg.B * cfg.H * cfg.N * (cfg.N + 1) / 2
    k = "_ZN3fox12_GLOBAL__N_120fwd_bf16_pipe_kernelILi64ELi4ELi2ELb0ELb1ELb0EEEv"
    mops = 4 * cfg.d * pairs / 512  # exactly the algorithmic flops
    rows = []
    for disp in (1, 2):
        rows += [(disp, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops, 0, 20000),
                 (disp, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000 * 0.25, 0, 20000),
                 (disp, k, "GRBM_GUI_ACTIVE", 8 * 1000, 0, 20000)]
    _counter_csv(tmp_path / "m.csv", rows)
    out = tmp_path / "m.txt"
    args = types.SimpleNamespace(pmc_csv=[f"c2:fwd:{tmp_path / 'm.csv'}"], out=str(out), note=None)
    bench.write_mfma_summary(args)
    line = [l for l in out.read_text().splitlines() if l.startswith("c2 ")][0].split()
    assert line[1] == "fwd_bf16_pipe_kernel<64,4,2,0,1,0>"
    assert int(line[2]) == 2 and float(line[3]) == pytest.approx(20.0)
    assert float(line[6]) == pytest.approx(1.0) and line[7] == "25.0%"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
