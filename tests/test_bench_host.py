"""Host logic of bench.py that runs without a GPU: the code hash that keys
the committed counter records, the traffic lookup, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_hash_ignores_comments_and_layout():
    a = {"kernels_ffn.hip": "int f(int x) { return x + 1; } // add one\n", "common.h": "/* header */\n#define N 4\n"}
    b = {"kernels_ffn.hip": "int f(int x)\n{\n  return x + 1;  /* add one */\n}\n", "common.h": "#define N 4 // four\n"}
    c = {"kernels_ffn.hip": "int f(int x) { return x + 2; }\n", "common.h": "#define N 4\n"}
    assert bench.kernel_source_sha(a) == bench.kernel_source_sha(b)
    assert bench.kernel_source_sha(a) != bench.kernel_source_sha(c)


def test_traffic_only_for_matching_code(tmp_path, monkeypatch):
    rec = {"kernel_source_sha": "abc", "traffic_bytes_per_launch": 123}
    (tmp_path / "gateup_w_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic("w", "abc") == 123
    assert bench.load_traffic("w", "def") is None
    assert bench.load_traffic("other", "abc") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
