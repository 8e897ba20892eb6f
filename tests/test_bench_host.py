"""Host-side checks of bench.py: the one-GPU contract and the arithmetic that turns
rocprofv3 counter files into HBM bytes per launch (no GPU needed)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def _counter_dir(path, counter, rows):
    os.makedirs(os.path.join(path, "host"), exist_ok=True)
    with open(os.path.join(path, "host", "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kern, val in rows:
            w.writerow({"Kernel_Name": kern, "Counter_Name": counter, "Counter_Value": val})


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    kern = f"void h3::(anonymous namespace)::{bench.DENSE_KERNEL}(h3::AttnArgs)"
    copy_kib = bench.COPY_BYTES / 1024.0
    # the copy kernel reads its buffer once and writes it once: a fetch counter that shows
    # half of its bytes gives a fetch scale of 2, a write counter that shows all gives 1
    _counter_dir(tmp_path / "f", "FETCH_SIZE", [(kern, 1000.0), (kern, 3000.0),
                                                ("other_kernel", 9e9)])
    _counter_dir(tmp_path / "w", "WRITE_SIZE", [(kern, 500.0)])
    _counter_dir(tmp_path / "cf", "FETCH_SIZE", [("copyBuffer", copy_kib / 2)])
    _counter_dir(tmp_path / "cw", "WRITE_SIZE", [("copyBuffer", copy_kib)])
    out_path = tmp_path / "summary.json"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(out_path))
    bench.pmc_summary([str(tmp_path / d) for d in ("f", "w", "cf", "cw")])
    out = json.loads(out_path.read_text())
    assert out["fetch_kib_per_launch"] == pytest.approx(2000.0)    # mean over launches
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    assert out["hbm_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2 + 500.0 * 1024)
    assert out["launches_averaged"] == [2, 1]
    assert str(tmp_path / "f") in out["commands"][0]


def test_pmc_summary_without_rows_fails_loudly(tmp_path, monkeypatch):
    _counter_dir(tmp_path / "f", "FETCH_SIZE", [("other_kernel", 1.0)])
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "summary.json"))
    with pytest.raises(SystemExit):
        bench.pmc_summary([str(tmp_path / "f")] * 4)
    assert not (tmp_path / "summary.json").exists()


def test_code_hash_ignores_comments_and_blank_lines():
    a = "int x = 1;  // one\n\n// note\nint y = 2;\n"
    b = "int x = 1;\nint y = 2;  // two\n"
    c = "int x = 1;\nint y = 3;\n"
    assert bench.code_hash(a) == bench.code_hash(b) != bench.code_hash(c)


def test_value_is_the_dense_call():
    """The headline value is the dense TARA call's dense-equivalent TFLOP/s (median
    ms/call); the block-sparse call carries ms and its speed-up, no dense-equivalent
    rate."""
    flop = 391.71e12
    rows = {"dense": [330.0, 320.0, 325.0], "router": [3.0, 2.8, 2.9],
            "sparse": [66.0, 65.0, 67.0], "via": [350.0, 351.0, 352.0]}
    calls = bench.call_summaries(rows, flop, 0.9, 170, 130, 300 / 1827)
    value = bench.headline_value(calls)
    assert value == calls["dense_tara"]["dense_equiv_tflops"]
    assert value == pytest.approx(flop / 0.325 / 1e12)
    sp = calls["block_sparse"]
    assert "dense_equiv_tflops" not in sp and "frac_peak" not in sp
    assert sp["ms"] == pytest.approx(2.9 + 66.0)
    assert sp["speedup_vs_dense"] == pytest.approx(325.0 / 68.9)
    assert bench.headline_value(bench.call_summaries({"sparse": [1.0], "router": [1.0]}, flop,
                                                     0.9, 170, 130, 0.16)) is None
