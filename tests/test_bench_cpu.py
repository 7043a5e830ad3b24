"""Host-side checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_is_hash_guarded(tmp_path):
    import hashlib
    import json
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "alibi_linear_position_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_bytes(b"kernel v1")
    digest = hashlib.sha256(b"kernel v1").hexdigest()[:16]
    rec = {"source_sha256_16": digest, "traffic_bytes": 1234}
    (tmp_path / "profiles" / "k.md").write_text("# k\n\n    traffic_record: " + json.dumps(rec) + "\n")
    assert bench.traffic_bytes("k.md", ["k.hip"], root=str(tmp_path)) == 1234
    (csrc / "k.hip").write_bytes(b"kernel v2")  # the kernel changed since the counters were taken
    assert bench.traffic_bytes("k.md", ["k.hip"], root=str(tmp_path)) is None
    assert bench.traffic_bytes("missing.md", ["k.hip"], root=str(tmp_path)) is None


def test_flop_and_byte_conventions():
    sys.path.insert(0, ROOT)
    import bench
    # causal triangle including the diagonal, QK^T + PV
    assert bench.fwd_flops(1, 1, 2, 1) == 4.0 * 1 * 3
    assert bench.fwd_flops(8, 16, 4096, 128) == 4.0 * 128 * 8 * 16 * 4096 * 4097 / 2
    # K + V caches plus q and out
    assert bench.decode_bytes(1, 1, 10, 8) == 2 * 10 * 8 * 2 + 2 * 8 * 2


def test_underflow_report_runs_on_a_small_workload(monkeypatch, capsys):
    # the report's plumbing on a 2-head, 64-token stand-in of the workload
    import json
    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import bench
    import workloads as W
    small = W.FwdWorkload("small", 1, 2, 64, 16, "bf16")
    monkeypatch.setattr(W, "FWD_B1_H16_N16384_D128", small)
    bench.underflow_report(W)
    rec = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert rec["only"] == "underflow" and len(rec["heads"]) == 2
    h0 = rec["heads"][0]
    assert h0["steepest_two"] and h0["slope"] == 2.0 ** -4
    for name in ("tau_u", "tau_d"):
        for key in ("analytic_triangle", "analytic_last_row", "data_triangle", "data_last_row"):
            assert 0.0 <= h0[name][key] <= 1.0
