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


def test_kernel_bytes_of_each_plan():
    # The dominant kernel of each plan of nosa_decode_step: the one-launch step moves the step's
    # bytes; the attention launch with the pick inside also reads each row's block scores and
    # query-agnostic ids and writes the selection; the two-call attention reads K/V, q and the ids.
    for cfg in ("C2", "C3", "C5", "F1"):
        w = WORKLOADS[cfg]
        b = bench.algorithmic_bytes(w)
        kv = w.rows * w.k * 64 * w.head_dim * 2 * 2
        q = w.batch * w.n_q_heads * w.head_dim * 2
        ids = w.rows * w.k * 4
        assert b["kernel"]["row_step_kernel"] == b["step"]
        assert b["kernel"]["step_decode_kernel"] == kv + q + w.rows * w.n_blocks * 4 + w.rows * w.ke * 4 + ids
        assert b["kernel"]["decode_mfma_kernel"] == kv + q + ids
    assert bench.algorithmic_bytes(WORKLOADS["C2"])["kernel"]["step_decode_kernel"] == 268746752


def test_traffic_record_needs_matching_code_workload_and_kernel(tmp_path, monkeypatch):
    good = {"workload": "C2", "kernel": "step_decode_kernel", "kernel_src_sha256": bench.kernel_src_sha256(),
            "bytes_per_launch": 123}
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    p = bench.traffic_path("C2", "step_decode_kernel")
    open(p, "w").write(json.dumps(good))
    assert bench.traffic_record("C2", "step_decode_kernel") == 123
    assert bench.traffic_record("C3", "step_decode_kernel") is None          # no record for that workload
    assert bench.traffic_record("C2", "row_step_kernel") is None             # nor for that kernel
    open(p, "w").write(json.dumps(dict(good, kernel_src_sha256="0" * 64)))
    assert bench.traffic_record("C2", "step_decode_kernel") is None          # taken on other kernel code
    open(p, "w").write(json.dumps(dict(good, workload="C3")))
    assert bench.traffic_record("C2", "step_decode_kernel") is None          # names another workload


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for d, k, c, v in rows:
            f.write('%d,"%s",%s,%s\n' % (d, k, c, v))


def test_record_traffic_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    # FETCH_SIZE reads half of the copy's 256 MiB, WRITE_SIZE all of it: the factors are 2 and 1, and
    # the kernel's per-dispatch means are scaled by them.
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    kib = 256 * 1024
    _counter_csv(str(tmp_path / "f" / "x" / "pmc_counter_collection.csv"),
                 [(1, "void nosa::step_decode_kernel<128, 4>(nosa::DecodeArgs)", "FETCH_SIZE", 100.0),
                  (2, "void nosa::step_decode_kernel<128, 4>(nosa::DecodeArgs)", "FETCH_SIZE", 300.0),
                  (3, "void nosa::combine_kernel<unsigned short, 128, 4>(nosa::DecodeArgs)", "FETCH_SIZE", 7.0)])
    _counter_csv(str(tmp_path / "w" / "pmc_counter_collection.csv"),
                 [(1, "void nosa::step_decode_kernel<128, 4>(nosa::DecodeArgs)", "WRITE_SIZE", 10.0)])
    mul = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, " \
          "at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >(int)"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, " \
           "std::array<char*, 1ul> >(int)"
    _counter_csv(str(tmp_path / "cf" / "cal_counter_collection.csv"),
                 [(1, fill, "FETCH_SIZE", 17.0), (2, mul, "FETCH_SIZE", kib / 2)])
    _counter_csv(str(tmp_path / "cw" / "cal_counter_collection.csv"),
                 [(1, fill, "WRITE_SIZE", kib), (2, mul, "WRITE_SIZE", kib)])
    bench.record_traffic("C2", "step_decode_kernel", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                         str(tmp_path / "cw"), ["cmd"])
    rec = json.load(open(bench.traffic_path("C2", "step_decode_kernel")))
    assert rec["raw_kib_per_dispatch"] == {"FETCH_SIZE": 200.0, "WRITE_SIZE": 10.0}
    assert rec["fetch_bytes_per_launch"] == 200 * 1024 * 2 and rec["write_bytes_per_launch"] == 10 * 1024
    assert rec["kernel_src_sha256"] == bench.kernel_src_sha256()
    assert bench.traffic_record("C2", "step_decode_kernel") == 200 * 1024 * 2 + 10 * 1024


def test_committed_traffic_records_are_close_to_the_algorithmic_bytes():
    # Whatever code they were taken on, the committed counter records must describe the workload and
    # kernel they name: measured HBM bytes within a few percent of the algorithmic bytes.
    import glob
    recs = glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))
    for path in recs:
        rec = json.load(open(path))
        assert os.path.basename(path) == "traffic_%s_%s.json" % (rec["kernel"], rec["workload"])
        alg = bench.algorithmic_bytes(WORKLOADS[rec["workload"]])["kernel"][rec["kernel"]]
        assert rec["algorithmic_bytes_per_launch"] == alg
        assert alg <= rec["bytes_per_launch"] <= 1.03 * alg


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
