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


def test_traffic_record_is_hash_guarded(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    # the committed records match the committed kernel sources
    assert bench.traffic_bytes("fwd_mfma_B8_H16_N4096_d128.md", ["fwd_mfma.hip", "device_common.h"]) > 0
    assert bench.traffic_bytes("decode_split_B32_H32_L32768_d128.md", ["decode.hip", "device_common.h"]) > 0
    # a record measured on other sources is ignored
    assert bench.traffic_bytes("fwd_mfma_B8_H16_N4096_d128.md", ["decode.hip"]) is None
    assert bench.traffic_bytes("no_such_file.md", ["decode.hip"]) is None


def test_flop_and_byte_conventions():
    sys.path.insert(0, ROOT)
    import bench
    # causal triangle including the diagonal, QK^T + PV
    assert bench.fwd_flops(1, 1, 2, 1) == 4.0 * 1 * 3
    assert bench.fwd_flops(8, 16, 4096, 128) == 4.0 * 128 * 8 * 16 * 4096 * 4097 / 2
    # K + V caches plus q and out
    assert bench.decode_bytes(1, 1, 10, 8) == 2 * 10 * 8 * 2 + 2 * 8 * 2
