"""Host logic of bench.py that runs without a GPU: the command line, the
one-GPU guard, and the lookup of recorded traffic counters (reported only
for the configuration and kernel sources they were taken on)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_help_lists_every_option():
    r = _bench("--help")
    assert r.returncode == 0, r.stderr
    for opt in ("--gpus", "--steps", "--warmup", "--op", "--workload", "--chunk",
                "--sweep", "--vendor-gemm", "--record-traffic", "--copy-calibration"):
        assert opt in r.stdout


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = _bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_config_key_names_op_workload_and_slice():
    class A:
        op, workload, chunk = "loss", "t32k", None
    assert bench.config_key(A) == "loss t32k chunk 8192"
    A.chunk = 1024
    assert bench.config_key(A) == "loss t32k chunk 1024"
    A.op, A.chunk = "teacher_topk", None
    assert bench.config_key(A) == "teacher_topk t32k chunk 4096"


def test_traffic_is_reported_only_for_its_configuration_and_sources(tmp_path, monkeypatch):
    srcs = ["kd_gemm_fast.hip", "kd_mfma_tile.h"]
    rec = {"config": "loss t32k chunk 8192", "sources": srcs,
           "source_sha": bench.source_sha(srcs), "bytes_per_launch": 123}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernels": {"gemm_dw": rec}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("gemm_dw", "loss t32k chunk 8192") == 123
    assert bench.traffic_for("gemm_dw", "loss t32k chunk 1024") is None
    assert bench.traffic_for("gemm_dh", "loss t32k chunk 8192") is None
    f.write_text(json.dumps({"kernels": {"gemm_dw": dict(rec, source_sha="0" * 16)}}))
    assert bench.traffic_for("gemm_dw", "loss t32k chunk 8192") is None
    f.write_text("not json")
    assert bench.traffic_for("gemm_dw", "loss t32k chunk 8192") is None


def test_source_hash_depends_on_every_listed_file():
    a = bench.source_sha(["kd_gemm_fast.hip", "kd_mfma_tile.h"])
    assert a == bench.source_sha(["kd_mfma_tile.h", "kd_gemm_fast.hip"])
    assert a != bench.source_sha(["kd_gemm_fast.hip"])
    assert len(a) == 16


def test_committed_traffic_records_cover_the_headline_kernels():
    # the recorded counters name the benchmark's configurations and every
    # GEMM of the loss and the teacher build
    with open(bench.TRAFFIC_FILE) as fh:
        kernels = json.load(fh)["kernels"]
    for k in ("gemm_logits", "gemm_dh", "gemm_dw"):
        assert kernels[k]["config"] == "loss t32k chunk 8192"
        assert kernels[k]["bytes_per_launch"] > 0
    assert kernels["tk_filter"]["config"] == "teacher_topk t32k chunk 4096"
