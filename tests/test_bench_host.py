"""Host-side logic of bench.py, on a machine without a GPU: the algorithmic byte counts every
reported GB/s figure divides by, the guard that ties committed HBM counter records to the kernel
code they were taken on, and the refusal of a multi-GPU run."""

import json
import os
import subprocess
import sys

import bench
from nosa_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hand_count(R, k, n, d, B, Hq, eb):
    kv = R * k * 64 * d * eb * 2          # selected K and V blocks (64 tokens each)
    kp = R * n * 2 * d * 4                # fp32 pooled keys, two 32-token sub-blocks per block
    ev = R * n * 4                        # one fp32 eviction score per block
    qo = 2 * B * Hq * d * eb              # the query in, the output out
    ids = R * k * 4                       # the selected ids
    return kv + kp + ev + qo + ids


def test_algorithmic_bytes_match_the_workload_shapes():
    # bs16/16K: 128 rows of 256 blocks, 64 selected; bs64/4K: 512 rows of 64 blocks, 16 selected;
    # bs4/128K: 32 rows of 2048 blocks, 64 selected; all bf16, d = 128, 32 query heads.
    assert bench.algorithmic_bytes(WORKLOADS["C2"])["step"] == _hand_count(128, 64, 256, 128, 16, 32, 2) == 302415872
    assert bench.algorithmic_bytes(WORKLOADS["C3"])["step"] == _hand_count(512, 16, 64, 128, 64, 32, 2) == 303202304
    assert bench.algorithmic_bytes(WORKLOADS["C5"])["step"] == _hand_count(32, 64, 2048, 128, 4, 32, 2) == 134553600
    # the attention call moves the selected K/V plus q, the output and the table
    b = bench.algorithmic_bytes(WORKLOADS["C2"])
    assert b["decode"] == 128 * 64 * 64 * 128 * 2 * 2 + 2 * 16 * 32 * 128 * 2 + 128 * 64 * 4


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    a = _write(tmp_path, "a.hip", "// header\nint f(int x) {\n    return x + 1;   // add one\n}\n")
    b = _write(tmp_path, "b.hip", "/* another\n   header */\n\nint f(int x) {\n\n    return x + 1;\n}\n")
    c = _write(tmp_path, "c.hip", "// header\nint f(int x) {\n    return x + 2;   // add one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [a])
    ha = bench.kernel_src_sha256()
    monkeypatch.setattr(bench, "KERNEL_SRCS", [b])
    assert bench.kernel_src_sha256() == ha
    monkeypatch.setattr(bench, "KERNEL_SRCS", [c])
    assert bench.kernel_src_sha256() != ha


def test_traffic_record_needs_matching_code_and_workload(tmp_path, monkeypatch):
    good = {"workload": "C2", "kernel_src_sha256": bench.kernel_src_sha256(), "bytes_per_launch": 123}
    p = _write(tmp_path, "t.json", json.dumps(good))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", {"C2": p})
    assert bench.traffic_record("C2") == 123
    assert bench.traffic_record("C3") is None                      # no record for that workload
    _write(tmp_path, "t.json", json.dumps(dict(good, kernel_src_sha256="0" * 64)))
    assert bench.traffic_record("C2") is None                      # taken on other kernel code
    _write(tmp_path, "t.json", json.dumps(dict(good, workload="C3")))
    assert bench.traffic_record("C2") is None                      # taken on another workload


def test_committed_traffic_records_are_close_to_the_algorithmic_bytes():
    # Whatever code they were taken on, the committed counter records must describe the workload
    # they name: measured HBM bytes within a few percent of the algorithmic bytes.
    for cfg, key in (("C2", "decode"), ("C3", "step")):
        rec = json.load(open(bench.PROFILE_TRAFFIC[cfg]))
        assert rec["workload"] == cfg
        alg = bench.algorithmic_bytes(WORKLOADS[cfg])[key]
        assert rec["algorithmic_bytes_per_launch"] == alg
        assert alg <= rec["bytes_per_launch"] <= 1.03 * alg


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
