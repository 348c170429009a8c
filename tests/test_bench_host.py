"""CPU checks of bench.py's host logic: the algorithmic byte and flop counts
behind hbm_frac and the rooflines (against figures worked out by hand for
the batch-32 / block-16 workload), the roofline's bound, the parser of the
committed counter summary, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
W = synth.WORKLOADS["b32_blk16_v151936_conv"]     # B 32, T 15, K 16, V 151,936, d 5120, r 256


def test_cycle_bytes_by_hand():
    logits = 32 * 15 * 151936 * 2            # 145,858,560
    target = 32 * 16 * 151936 * 2            # 155,582,464
    gathered = (7680 + 32 + 480) * 5120 * 2  # candidates, last tokens, context rows: 83,886,080
    weights = 3 * 256 * 5120 * 2             # W_A, W_B, W_H: 7,864,320
    site = 2 * 512 * 5120 * 2 + 32 * 5120 * 2 + 640 * 5120 * 2   # x and y, x_prev, W: 17,367,040
    assert bench.cycle_bytes(W, conv=False) == logits + target + gathered + weights == 393_191_424
    assert bench.cycle_bytes(W, conv=True) == 393_191_424 + 20 * site == 740_532_224
    rows = (7680 + 32) * 512 * 4             # fp32 table rows of the candidates and last tokens
    assert bench.cycle_bytes(W, conv=False, tables=True) == \
        logits + target + rows + 480 * 5120 * 2 + 256 * 5120 * 2
    # 8 TB/s for 1 ms moves 8 GB
    assert bench.hbm_frac(W, False, 1000.0) == round(393_191_424 / 8e9, 4)


def test_algorithmic_work_and_bounds():
    by, fl = bench.algorithmic(W, "conv_gemm")
    assert by == 512 * 5120 * 2 + 640 * 5120 * 2 == 11_796_480
    assert fl == 2 * 512 * 5120 * 640
    r = bench.roofline_of(W, "conv_gemm", 10.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"      # 284 flop/B, under the 312.5 ridge
    assert abs(r["achieved"] - 11_796_480 / 10e-6 / 1e9) < 0.1
    assert r["frac"] == round(11_796_480 / 10e-6 / 1e9 / 8000.0, 4)
    r = bench.roofline_of(W, "project_gemm", 60.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    outs = 7680 * 512 + 32 * 256 + 480 * 256
    assert r["algorithmic_flops"] == 2 * 5120 * outs
    assert bench.algorithmic(W, "topk_chunk")[0] == 32 * 15 * 151936 * 2 + 32 * 15 * 16 * 8
    assert bench.algorithmic(W, "argmax_part")[0] == 32 * 16 * 151936 * 2
    assert bench.roofline_of(W, "path", 5.0) is None


def test_counter_summary_parser(tmp_path, monkeypatch):
    f = tmp_path / "counters.txt"
    f.write_text("# header\nsource_sha256 = abc\nfetch_factor = 2.0\nwrite_factor = 1.0\n"
                 "kernel conv_gemm fetch_kib=100.0 write_kib=10.0\n")
    monkeypatch.setattr(bench, "COUNTERS", str(f))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")
    assert bench.measured_traffic("conv_gemm") == 1024 * (100 * 2 + 10)
    assert bench.measured_traffic("topk_chunk") is None
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.measured_traffic("conv_gemm") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_trace_summary_parser(tmp_path, monkeypatch):
    """The trace figure is read only when the summary was taken from the
    current kernel sources."""
    f = tmp_path / "trace.txt"
    f.write_text("# command: x\n# source_sha256 = abc\nkernel calls avg_us min_us max_us total_us\n"
                 "conv_gemm 10 12.50 9.9 19.1 125.0\ntopk_chunk 5 33.0 30 38 165\n")
    monkeypatch.setattr(bench, "TRACE", str(f))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")
    assert bench.trace_avg_us("conv_gemm") == 12.5
    assert bench.trace_avg_us("topk_chunk") == 33.0
    assert bench.trace_avg_us("path") is None
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.trace_avg_us("conv_gemm") is None
