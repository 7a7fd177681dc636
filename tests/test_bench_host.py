"""Host logic of bench.py (CPU only): the device-code hash behind the traffic records, the staleness
guard, the process-pool cpu_baseline leg on a tiny oracle workload, and the refusal of N > 1 GPUs."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_device_code_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "flashattention_forward_02_amd" / "csrc"
    csrc.mkdir(parents=True)
    for n in ("fa_internal.h", "mfma_common.h"):
        (csrc / n).write_text("int shared_" + n.replace(".", "_") + ";\n")
    (csrc / "k.hip").write_text("// a comment\nint f(int x) { return x + 1; }  /* block */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.device_code_hash("k.hip")
    (csrc / "k.hip").write_text("/* another\n comment */ int f(int x)   {\n  return x + 1; }\n")
    assert bench.device_code_hash("k.hip") == h0          # comment and whitespace edits keep it
    (csrc / "k.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.device_code_hash("k.hip") != h0          # a code edit changes it


def test_traffic_record_is_used_only_for_matching_device_code(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    rec = {"headline": {"device_code_hash": "abc", "bytes_per_launch": 123.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("headline", "abc") == 123.0
    assert bench.traffic_for("headline", "abd") is None
    assert bench.traffic_for("causal", "abc") is None


def test_committed_traffic_records_name_existing_profiles():
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert recs
    for key, rec in recs.items():
        assert len(rec["device_code_hash"]) == 16 and rec["bytes_per_launch"] > 0, key
        assert os.path.exists(os.path.join(ROOT, rec["profile"])), rec["profile"]


def test_cpu_baseline_pool_on_a_tiny_workload():
    """Two heads of 64 rows in tasks of 16 rows: every task is checked, the parity record compares the
    oracle with itself (zero error), and the record names the worker count and the CPU."""
    r = np.random.default_rng(5)
    q, k, v = (r.standard_normal((2, 64, 16)) for _ in range(3))
    ref = [oracle.attention_rows_fp64(q[h], k[h], v[h], 0.25)[0] for h in range(2)]
    tasks = [("fwd", (0, h, r0, r0 + 16), (q[h, r0:r0 + 16], k[h], v[h], r0, 64), 0.25, False)
             for h in range(2) for r0 in range(0, 64, 16)]

    def compare(key, got):
        _, h, r0, r1 = key
        return [bench.err_triplet(got, ref[h][r0:r1])]

    base, check = bench.cpu_baseline(tasks, lambda key: 4.0 * 16 * 64 * 16, 30.0, compare)
    assert check["tasks_checked"] == len(tasks) == base["tasks_done"]
    assert check["max_abs"] < 1e-12 and check["rel_l2"] < 1e-12
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in json.loads(p.stdout.strip().splitlines()[-1])["error"]
