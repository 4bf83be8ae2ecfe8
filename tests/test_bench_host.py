"""Host-side logic of bench.py (no GPU): the code hash that keys the stored traffic figure, the
rocprofv3 counter parsing and scaling, and the one-GPU guard."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, text):
    with open(path, "w", encoding="utf-8") as f:
        f.write(text)
    return str(path)


def test_code_hash_ignores_comments_and_spacing_only(bench, tmp_path):
    a = _write(tmp_path / "a.hip", "int f(int x) {  // add one\n    return x + 1; /* done */ }\n")
    b = _write(tmp_path / "b.hip", "int f(int x) { return x + 1; }")
    c = _write(tmp_path / "c.hip", "int f(int x) { return x + 2; }")
    assert bench._sha([a]) == bench._sha([b])
    assert bench._sha([a]) != bench._sha([c])
    assert bench._sha([a, b]) != bench._sha([b]), "file boundaries are part of the hash"


def _pmc_csv(d, rows):
    """A counter_collection.csv as rocprofv3 writes it (quoted fields: kernel names hold commas)."""
    import csv
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)
    return str(d)


def test_record_and_report_traffic(bench, tmp_path, monkeypatch):
    src = _write(tmp_path / "k.hip", "void k() {}")
    monkeypatch.setattr(bench, "SCORE_SRC", [src])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kern = "void dllm::score_kernel<true, true>(dllm::StepParams, int)"
    dec = "void dllm::decide_kernel<0, 4>(dllm::StepParams)"
    # two counter instances per dispatch (summed), three dispatches (median taken)
    fetch = _pmc_csv(tmp_path / "f", [(1, kern, "FETCH_SIZE", 40.0), (1, kern, "FETCH_SIZE", 60.0),
                                      (2, kern, "FETCH_SIZE", 100.0), (3, kern, "FETCH_SIZE", 500.0),
                                      (4, "other", "FETCH_SIZE", 9e9), (5, dec, "FETCH_SIZE", 6.0),
                                      (6, dec, "FETCH_SIZE", 8.0), (7, dec, "FETCH_SIZE", 7.0)])
    write = _pmc_csv(tmp_path / "w", [(1, kern, "WRITE_SIZE", 3.0), (2, kern, "WRITE_SIZE", 5.0),
                                      (3, kern, "WRITE_SIZE", 4.0), (5, dec, "WRITE_SIZE", 2.0)])
    known = bench.COPY_MIB * 1024.0
    cfetch = _pmc_csv(tmp_path / "cf", [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", known / 2)])
    cwrite = _pmc_csv(tmp_path / "cw", [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", known)])
    bench.record_traffic(fetch, write, cfetch, cwrite, masked=7)
    rec = json.load(open(bench.TRAFFIC_FILE))
    sk = rec["score_kernel"]
    assert sk["fetch_kib_per_dispatch"] == 100.0 and sk["write_kib_per_dispatch"] == 4.0
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    score = (100.0 * 2 + 4.0) * 1024
    step = score + (7.0 * 2 + 2.0) * 1024
    assert rec["hbm_bytes_per_launch"] == pytest.approx(score)
    assert rec["dllm_step_hbm_bytes"] == pytest.approx(step)
    assert bench.stored_traffic(7) == pytest.approx((score, step))
    assert bench.stored_traffic(8) == (None, None)               # another workload
    _write(src, "void k() { int x; }")
    assert bench.stored_traffic(7) == (None, None)               # the kernels' code changed
    _write(src, "void k() {} // a comment only")
    assert bench.stored_traffic(7) != (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_loop_names_are_checked():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--loop", "no-such-workload"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "llada-sync" in (r.stderr + r.stdout)


def test_oracle_baseline_batches(bench):
    # the oracle's timed sample is the workload's own first batch: the headline step's 64 rows as
    # packed, and for the large run the 256 requests the admission takes from the empty box first
    from workload import configs
    _, rows, W, pk = bench._first_batch(configs.make("dream-dynamic-step"))
    assert rows == 64 and int(pk["mask"].sum()) == 1005 and pk["box_ids"].shape == (64, W)
    w = configs.make("large-fdfo")
    assert w.rows == 0
    rr, rows, W, pk = bench._first_batch(w)
    assert rows == 256 and pk["mask"].shape == (256, 64) and bool(pk["mask"].all())
    assert len(set(int(q) for q in rr[:rows])) == rows
