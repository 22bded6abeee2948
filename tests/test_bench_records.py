"""The bench line's recorded HBM traffic figures point at the rocprofv3 summaries they came from."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_traffic_records_name_existing_profiles():
    import bench
    for (kernel, workload), rec in bench.TRAFFIC.items():
        path = os.path.join(ROOT, rec["profile"])
        assert os.path.exists(path), path
        text = open(path).read()
        assert kernel in text and workload in text, path
        assert f"FETCH_SIZE {rec['fetch_kib']}" in text and f"WRITE_SIZE {rec['write_kib']}" in text, path
        for src in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, src)), src
        assert 0.4 < rec["fetch_per_byte"] < 0.6 and 0.9 < rec["write_per_byte"] < 1.1


def test_gpu_count_above_one_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
