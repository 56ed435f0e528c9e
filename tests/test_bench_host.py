"""Host-side pieces of bench.py that need no GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_strip_comments_keeps_code_and_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char *s = "x//y/*z*/";\nchar q = \'"\';  int b;'
    assert bench.strip_comments(src) == 'int a = 1; const char *s = "x//y/*z*/"; char q = \'"\'; int b;'
    assert bench.strip_comments('p = "a\\"//b"; // c') == 'p = "a\\"//b";'


def test_source_hash_ignores_comments_not_code():
    a = "__global__ void k(int *p) { p[0] = 1; }\n"
    b = "// a comment\n__global__ void k(int *p) {\n    p[0] = 1;   /* same code */\n}\n"
    c = "__global__ void k(int *p) { p[0] = 2; }\n"
    assert bench.strip_comments(a) == bench.strip_comments(b)
    assert bench.strip_comments(a) != bench.strip_comments(c)


def test_traffic_files_name_their_workload():
    for w in bench.DESCR:
        p = os.path.join(ROOT, "profiles", f"traffic_{w}.json")
        if not os.path.exists(p):
            continue
        d = json.load(open(p))
        assert d["workload"] == w
        # each figure is rounded from the same scaled counter values
        assert abs(d["bytes_per_launch"] - (d["fetch_bytes"] + d["write_bytes"])) <= 1
        assert len(d["kernel_source_sha256"]) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_cpu_baseline_record_names_its_protocol():
    """The oracle's CPU baseline: median of three multi-threaded batches, a
    median of three single-threaded runs, the threads used, the OS core
    count and the CPU model."""
    import gen
    import oracle
    inp = gen.make_inputs("tiny", 0)
    run = lambda: oracle.combine(inp.payload, inp.src_info, inp.weights, inp.shared,
                                 checked=False)
    rec = bench.time_cpu_oracle(run, inp.T, 394752, 0.3, oracle)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert len(rec["batch_tokens_per_s"]) == 3
    assert sorted(rec["batch_tokens_per_s"])[1] == rec["value"]
    assert len(rec["single_thread"]["runs_tokens_per_s"]) == 3
    assert rec["cores"] == rec["omp_threads"] == oracle.max_threads()
    assert rec["os_cpu_count"] == os.cpu_count() and rec["cpu_model"]
    assert oracle.max_threads() == rec["omp_threads"]       # threads restored
