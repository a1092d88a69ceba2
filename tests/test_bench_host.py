"""Host-side logic of bench.py (no GPU): the one-GPU contract, and the rule
that HBM-traffic figures are reported only for the kernel source they were
taken on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n    return x + 1;\n}\n")
    b.write_text("// header\n/* block\n comment */\nint f(int x) {   // trailing\n\n    return x + 1;\n}\n")
    c.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.kernel_hash(str(a)) == bench.kernel_hash(str(b))
    assert bench.kernel_hash(str(a)) != bench.kernel_hash(str(c))


def test_traffic_only_for_the_current_kernel(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int k() { return 0; }\n")
    tf = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "GEMM_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    rec = {"workloads": {"W": {"hbm_bytes_per_launch": 123}}}
    tf.write_text(json.dumps(dict(rec, kernel_hash=bench.kernel_hash(str(src)))))
    assert bench.load_traffic("W") == 123
    assert bench.load_traffic("other workload") is None
    src.write_text("int k() { return 1; }\n")          # the kernel changed since the counters
    assert bench.load_traffic("W") is None
    tf.write_text("not json")
    assert bench.load_traffic("W") is None



def test_per_cu_clock_matches_samples_per_compute_unit():
    """Cycle counters are compared only within one compute unit (earliest sample
    before, latest after); CUs missing from either side are left out."""
    import numpy as np
    rate = 100000.0                         # kHz: 100 MHz wall counter
    before = [  # cycle, wall, xcd, hw_id (CU field bits 8..15)
        (1_000_000, 500, 0, 0x0100), (1_000_900, 509, 0, 0x0100),   # CU (0, 1): earliest at wall 500
        (9_000_000, 700, 1, 0x0100),                                # CU (1, 1): another counter base
        (5, 600, 2, 0x0300)]                                         # CU (2, 3): no sample after
    after = [
        (1_000_000 + 2_000 * 1000, 1500, 0, 0x0100), (1_000_000 + 1_500 * 1000, 1250, 0, 0x0100),
        (9_000_000 + 1_800 * 2000, 2700, 1, 0x0100)]
    pad = lambda rows: rows + [rows[0]] * (4 - len(rows))
    s = np.array([pad(before), pad(after)], dtype=np.int64)
    cu = bench.per_cu_clock(s, rate)
    assert set(cu) == {(0, 1), (1, 1)}
    # CU (0, 1): 2e6 cycles over 1000 wall ticks of 10 ns = 10 us -> 200000 MHz scaled: cycles / us
    assert abs(cu[(0, 1)] - 2_000_000 / 10.0) < 1e-6
    assert abs(cu[(1, 1)] - 3_600_000 / 20.0) < 1e-6
