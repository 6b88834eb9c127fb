"""bench.py's host-side parts (CPU only): argument handling that exits before
any GPU work, the per-(workload, rho) JSONL records and the rule that decides
which recorded sweep points a rerun may reuse, and the counter-traffic
bookkeeping."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0 and "one GPU" in r.stderr and not r.stdout.strip()


def test_resume_needs_a_jsonl_file():
    r = run_bench("--resume")
    assert r.returncode != 0 and "--jsonl" in r.stderr


def test_reuse_rule(tmp_path):
    rec = {"kind": "sweep", "workload": "c2", "rho": 0.5, "full_path": False, "inputs_sha256": "in",
           "library_sha256": "lib", "ms": 0.1}
    path = tmp_path / "runs.jsonl"
    path.write_text(json.dumps(rec) + "\n" + "not json\n" +
                    json.dumps({**rec, "kind": "headline", "ms": 0.3}) + "\n" + json.dumps({**rec, "ms": 0.2}) + "\n")
    rows = bench.read_jsonl(str(path))
    assert len(rows) == 3                                                        # the broken line is skipped
    assert bench.reusable_point(rows, "c2", 0.5, False, "in", "lib")["ms"] == 0.2  # the last matching record
    for args in [("c3", 0.5, False, "in", "lib"), ("c2", 0.7, False, "in", "lib"), ("c2", 0.5, True, "in", "lib"),
                 ("c2", 0.5, False, "other", "lib"), ("c2", 0.5, False, "in", "changed"),
                 ("c2", 0.5, False, None, "lib")]:
        assert bench.reusable_point(rows, *args) is None, args
    assert bench.read_jsonl(str(tmp_path / "missing.jsonl")) == []


def test_library_digest_tracks_the_sources():
    a = bench.library_digest()
    assert a == bench.library_digest() and len(a) == 64


def test_every_workload_names_its_dominant_kernel():
    # the roofline's traffic record is looked up by (kernel key, workload)
    for w in bench.WORKLOADS:
        if w != "mlp":
            assert w in bench.TRAFFIC_KERNELS, w
    for key, frag, src in bench.TRAFFIC_KERNELS.values():
        assert key in ("gemm", "gemv") and os.path.exists(
            os.path.join(ROOT, "input_adaptive_reduced_amd", "csrc", src)), (key, frag, src)


def test_traffic_record_survives_comment_edits_only(tmp_path, monkeypatch):
    # a counter record stays current while only comments or layout of its
    # kernel's source change, and is retired by any change of the code
    src = tmp_path / "k.hip"
    src.write_text("// note\n__global__ void k(int *p) { p[0] = 1; }  /* end */\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"source": "k.hip", "code_sha256": bench.code_digest(str(src)), "bytes_per_launch": 123.0}
    (prof / "traffic.json").write_text(json.dumps({"gemm@c2": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("gemm", "c2") == 123.0
    src.write_text("// a longer note\n/* and a block\n   comment */\n__global__ void k(int *p)\n{\n    p[0] = 1;\n}\n")
    assert bench.load_traffic("gemm", "c2") == 123.0
    src.write_text("__global__ void k(int *p) { p[0] = 2; }\n")
    assert bench.load_traffic("gemm", "c2") is None
    assert bench.load_traffic("gemm", "c3") is None
