"""bench.py's host-side pieces, on the CPU: the oracle timing leg, the counter
summary arithmetic and the refusal of more than one GPU."""

import os
import subprocess
import sys

import numpy as np

import seeded_inputs as si
from oracle.schedules import make_plan
from oracle.simulate import run_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_repeats_the_oracle_and_compares_with_a_sample():
    import bench
    N, count = 4, 4096
    a = si.rank_arrays(5, N, count, "float32")
    cols = np.arange(0, count, 7)
    want = run_plan(make_plan("allreduce", "ring", N, count), "float32", "sum", a)
    sample = [np.ascontiguousarray(w[cols]) for w in want]
    r = bench.cpu_baseline(a, N, count, "ring", cols, sample, min_seconds=0.05, max_calls=3)
    assert (r["kind"], r["cores"], r["unit"]) == ("oracle", 1, "GB/s") and r["value"] > 0
    assert r["host_cpu_count"] == os.cpu_count() and r["host_cpus_in_affinity"] == len(os.sched_getaffinity(0))
    assert r["matches_gpu"] is True
    assert r["sample"].split()[0] in ("1", "2", "3") and "calls of the full workload" in r["sample"]
    bad = [s.copy() for s in sample]
    bad[1][3] += np.float32(1)
    r = bench.cpu_baseline(a, N, count, "ring", cols, bad, min_seconds=0.0, max_calls=1)
    assert r["matches_gpu"] is False and r["sample"].startswith("1 calls")
    # row checksums, in the library's row order (coll_plan runs on the host)
    import collective_communication_algorithms_amd as coll
    plan = make_plan("allreduce", "ring", N, count)
    _, osums = run_plan(plan, "float32", "sum", a, trace=True)
    by_row, idx = {}, 0
    for st, srows in enumerate(plan.steps):
        for q in srows:
            by_row[(st, q.src, q.dst, q.src_off, q.dst_off, q.n)] = int(osums[idx])
            idx += 1
    rows, _ = coll.coll_plan("allreduce", "ring", N, count, "float32")
    sums = np.array([by_row[tuple(q[:6])] for q in rows], dtype=np.uint64)
    r = bench.cpu_baseline(a, N, count, "ring", cols, sample, min_seconds=0.0, max_calls=1, gpu_sums=sums)
    assert r["checksums_match_gpu"] is True
    sums[5] += np.uint64(1)
    r = bench.cpu_baseline(a, N, count, "ring", cols, sample, min_seconds=0.0, max_calls=1, gpu_sums=sums)
    assert r["checksums_match_gpu"] is False


def test_summarize_counters_scales_by_the_copy_kernel(tmp_path):
    import bench
    name = "void coll::rows_kernel<2, 0, false, 1, false>"
    copy = "void coll::calib_kernel<false>"

    def write(path, kernel, values):
        with open(path, "w") as f:
            f.write("Kernel_Name,Counter_Value\n")
            for v in values:
                f.write(f'"{kernel}(coll::RowsArgs)",{v}\n')

    write(tmp_path / "f.csv", name, [100.0, 300.0])     # mean 200 KiB
    write(tmp_path / "w.csv", name, [50.0])
    write(tmp_path / "cf.csv", copy, [1048576.0])       # half of the known 2 GiB: factor 2
    write(tmp_path / "cw.csv", copy, [2097152.0])       # factor 1
    out = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                                   str(tmp_path / "cw.csv"), name, str(tmp_path / "t.json"))
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["traffic_bytes_per_launch"] == (200 * 2 + 50) * 1024
    assert out["dispatches"] == [2, 1] and len(out["kernel_source_hash"]) == 16


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "--gpus above 1 is not supported" in p.stderr
