"""Host-side logic of bench.py that needs no GPU: it refuses more than one GPU, and
the HBM traffic it reports is tied to the sources the measured kernels are built from."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=e,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_distributed_launch_is_refused():
    r = _run([], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr


def test_traffic_records_name_existing_sources():
    for kernel, files in bench.KERNEL_SOURCES.items():
        assert files, kernel
        for f in files:
            assert os.path.isfile(os.path.join(ROOT, f)), f
        h = bench.source_hash(kernel)
        assert len(h) == 16 and int(h, 16) >= 0


def test_traffic_is_null_without_a_matching_record():
    assert bench.traffic_record("mf_apply_translated", "no such workload") is None
    assert bench.traffic_record("no such kernel", "workload4") is None
