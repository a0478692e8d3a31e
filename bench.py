"""Headline benchmark: Ring AllReduce, fp32, 8 virtual ranks x 256 MiB, one GPU.

    python bench.py [--steps K] [--warmup W] [--algo ring|rhd|dbt] [--exec auto|rows|step]

A step is one whole AllReduce call (every row of the schedule's 2(N-1) steps,
with the per-row checksums unless --no-checksums) over the 8 rank buffers, in
place, inputs resident in HBM.  Before every call (warm-up and timed) the
inputs are restored from a pristine device copy, untimed; each timed call is
bracketed by HIP events on its stream.  Prints one JSON line:
  value         busbw in GB/s = algbw * 2(N-1)/N, algbw = M / median call time
                ("集合通信算法延迟公式", @tbl-model-algo-busbw-coef)
  ms_per_step   the median call time (minimum and every call's time beside it)
  hbm_pct_of_peak  bytes the call moves through memory / median call time, as
                a percentage of MI355X's 8 TB/s HBM peak
  roofline      the column kernel's algorithmic bytes per launch (each rank's
                input read once and its result written once: 2NM; what the
                schedule's steps pass from row to row stays in registers) over
                its mean launch time, timed live by the library's own HIP
                events (COLL_OPT_TIMING) in a second pass of restored calls
  access_pattern_ceiling  the same buffers under the kernel's memory access
                pattern alone (8 loads, a sum, 8 stores per 1 KiB tile), and
                the column kernel's rate as a fraction of it
  cpu_baseline  the CPU oracle on the same inputs, one core
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "busbw GB/s & % HBM peak, Ring AllReduce fp32 N=8 M=256MiB (1 GPU)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_col_kernel_ring_allreduce_fp32_n8_256MiB.json")
# the column kernel variant the default run times: fp32, sum, 8 register
# slots, 16 checksum accumulators, nontemporal loads and stores, no batches,
# room for 16 ranks' buffer addresses
HEADLINE_KERNEL = "void coll::(anonymous namespace)::col_kernel<2, 0, 8, 16, 5, false, 16>"


def kernel_source_hash() -> str:
    """Hash of the code (comments and blank space removed) that decides what the
    column kernel does: the kernel, its programs and launch shapes, so that the
    committed counter summary is dropped whenever any of it changes."""
    import re
    h = hashlib.sha256()
    for f in ("colkernel.hip", "device_common.h", "device_types.h", "colprog.h", "colprog.cpp", "abi.cpp"):
        with open(os.path.join(ROOT, "collective_communication_algorithms_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(per_launch_bytes_expected: float):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel source as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(inputs_host, N: int, count: int, algo: str, cols=None, gpu_sample=None,
                 min_seconds: float = 10.0, max_calls: int = 40, gpu_sums=None):
    """The oracle as it stands, timed on the host on the same inputs: calls of
    the whole workload repeated until ``min_seconds`` of CPU work (at most
    ``max_calls``), the mean per call reported.  With ``cols`` / ``gpu_sample``
    (the GPU's result of one call on the same inputs at those columns) it also
    reports whether the first call's result agrees with it bit for bit, and
    with ``gpu_sums`` (that call's per-row checksums, in the library's row
    order) whether every row's checksum equals the oracle's."""
    import numpy as np
    from oracle.schedules import make_plan
    from oracle.simulate import run_plan
    plan = make_plan("allreduce", algo, N, count)
    times, out, osums = [], None, None
    while not times or (sum(times) < min_seconds and len(times) < max_calls):
        t0 = time.perf_counter()
        res_i = run_plan(plan, "float32", "sum", inputs_host)
        times.append(time.perf_counter() - t0)
        if out is None:
            out = res_i
        del res_i
    if gpu_sums is not None:
        _, osums = run_plan(plan, "float32", "sum", inputs_host, trace=True)
    dt = sum(times) / len(times)
    M = count * 4
    busbw = M / dt * 2 * (N - 1) / N / 1e9
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    res = {"value": round(busbw, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{len(times)} calls of the full workload ({N} x {M >> 20} MiB fp32, one {algo} "
                     f"AllReduce each), numpy single-threaded, {sum(times):.1f} s in all, {dt:.2f} s per call",
           "host_cpu_count": os.cpu_count(), "host_cpus_in_affinity": affinity}
    if cols is not None:
        res["matches_gpu"] = all(np.array_equal(o[cols].view(np.uint32), g.view(np.uint32))
                                 for o, g in zip(out, gpu_sample))
    if gpu_sums is not None:
        import collective_communication_algorithms_amd as coll
        rows, _ = coll.coll_plan("allreduce", algo, N, count, "float32")
        want, idx = {}, 0
        for st, srows in enumerate(plan.steps):
            for r in srows:
                want[(st, r.src, r.dst, r.src_off, r.dst_off, r.n)] = int(osums[idx])
                idx += 1
        res["checksums_match_gpu"] = len(rows) == len(gpu_sums) and all(
            int(gpu_sums[j]) == want.get(tuple(r[:6])) for j, r in enumerate(rows))
    return res


def summarize_counters(fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, kernel_prefix, out_json,
                       calib_gib: int = 2) -> dict:
    """Traffic per launch of the row kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by what the same
    counter reads for the plain copy kernel (which reads and writes calib_gib
    GiB): the factor is the copy's known bytes over its counter reading."""
    import csv
    import statistics

    def mean_kib(path, prefix):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if r["Kernel_Name"].startswith(prefix)]
        if not vals:
            raise SystemExit(f"no dispatch of {prefix!r} in {path}")
        return statistics.mean(vals), len(vals)

    copy_prefix = "void coll::calib_kernel<false>"
    known_kib = calib_gib << 20
    cf, _ = mean_kib(calib_fetch_csv, copy_prefix)
    cw, _ = mean_kib(calib_write_csv, copy_prefix)
    f, nf = mean_kib(fetch_csv, kernel_prefix)
    w, nw = mean_kib(write_csv, kernel_prefix)
    ff, fw = known_kib / cf, known_kib / cw
    traffic = (f * ff + w * fw) * 1024
    out = {"kernel": kernel_prefix, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w, "dispatches": [nf, nw],
           "copy_kernel_fetch_kib": cf, "copy_kernel_write_kib": cw, "copy_kernel_known_kib": known_kib,
           "fetch_scale": ff, "write_scale": fw,
           "traffic_bytes_per_launch": round(traffic)}
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out


def sweep(out_path: str, dev, quick: bool = False) -> None:
    """Every configuration's calls, one JSON line each, into ``out_path``.

    Protocol: 5 warm-up calls, then 20 calls, each timed alone with HIP events
    on the call's stream; before every call the inputs are restored from a
    pristine device copy (not timed).  Median and minimum are reported, with
    algbw = M / t, busbw = algbw x the pages' coefficient, schedule bytes / t
    against the 8 TB/s HBM spec, the pages' alpha-beta prediction (alpha 5 us,
    beta 450 GB/s) and a least-squares fit t = alpha_call + moved bytes /
    beta_g over the fp32 Ring AllReduce sizes.  The oracle is timed on the host (one
    core) on the same inputs where that takes seconds; larger calls give none.
    """
    import numpy as np
    import torch

    import collective_communication_algorithms_amd as coll
    import seeded_inputs as si
    from collective_communication_algorithms_amd import model

    rows = []
    stream = torch.cuda.current_stream(dev)
    reps, warm = (5, 2) if quick else (20, 5)

    def time_call(fn, pristine, live):
        restore = (lambda: live.copy_(pristine)) if live is not pristine else (lambda: None)
        for _ in range(warm):
            restore()
            fn()
        ts = []
        for _ in range(reps):
            restore()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            e.synchronize()
            ts.append(s.elapsed_time(e))
        restore()
        torch.cuda.synchronize()
        return float(np.median(ts)), float(np.min(ts))

    def oracle_time(kind, algo, host, dtype, root=0, k=1):
        from oracle.schedules import make_plan
        from oracle.simulate import run_plan
        plan = make_plan(kind, algo, len(host), len(host[0]), root, k)
        t0 = time.perf_counter()
        run_plan(plan, dtype, "sum", host)
        return time.perf_counter() - t0

    def record(cfg, kind, algo, dtype, N, count, k, med, mn, oracle_s=None, root=0):
        sz = si.ITEMSIZE[dtype]
        M = count * sz
        _, cnt = coll.coll_plan(kind, algo, N, count, dtype, root, k)
        st = coll.coll_get_stats()
        algbw = M / (med * 1e-3) / 1e9
        r = {"config": cfg, "kind": kind, "algo": algo, "dtype": dtype, "N": N, "M": M, "k": k,
             "steps": cnt["steps"], "sched_bytes": st["hbm_bytes"], "crit_bytes": cnt["crit_bytes"],
             "t_med_us": round(med * 1e3, 2), "t_min_us": round(mn * 1e3, 2),
             "algbw_GBps": round(algbw, 3), "busbw_GBps": round(algbw * model.busbw_coef(kind, N), 3),
             # the bytes the schedule's rows stand for, over the call's time
             # (above the HBM peak wherever the kernels keep them in registers)
             "sched_TBps": round(st["hbm_bytes"] / (med * 1e-3) / 1e12, 3),
             # what the launched kernels moved through memory (operands passed in
             # registers and skipped stores left out), its rate and share of 8 TB/s
             "moved_bytes": st["moved_bytes"],
             "moved_TBps": round(st["moved_bytes"] / (med * 1e-3) / 1e12, 3),
             "moved_pct_of_8TBps": round(100 * st["moved_bytes"] / (med * 1e-3) / 8e12, 2)}
        try:
            mk = "broadcast" if kind == "broadcast" else kind
            r["ab_page_us"] = round(model.time(mk, algo, N, M, 5e-6, 450e9, k) * 1e6, 2)
        except ValueError:
            pass
        if oracle_s is not None:
            r["oracle_s"] = round(oracle_s, 4)
            r["oracle_cores"] = 1
        rows.append(r)
        with open(out_path, "a") as fh:
            fh.write(json.dumps(r) + "\n")
        print(json.dumps(r), file=sys.stderr, flush=True)

    open(out_path, "w").close()

    # C1: Ring / RHD / DBT AllReduce, 4 ranks x 1,024 int32
    host = si.rank_arrays(1, 4, 1024, "int32")
    pristine = torch.stack([si.host_to_tensor(x, "int32", dev) for x in host])
    live = pristine.clone()
    for algo in ("ring", "rhd", "dbt"):
        med, mn = time_call(lambda: coll.coll_allreduce(list(live), algo=algo), pristine, live)
        record("C1", "allreduce", algo, "int32", 4, 1024, 1, med, mn, oracle_time("allreduce", algo, host, "int32"))

    # C2: Broadcast / Scatter / Gather, 8 ranks, uint8
    for M in ((1 << 10, 1 << 16, 1 << 22) if quick else (1 << 10, 1 << 16, 1 << 22, 1 << 26)):
        host = si.rank_arrays(2, 8, M, "uint8") if M <= (1 << 22) else None
        pristine = (torch.stack([si.host_to_tensor(x, "uint8", dev) for x in host]) if host is not None else
                    torch.stack(si.device_rank_tensors(2, 8, M, "uint8", dev)))
        live = pristine.clone()
        cases = [("broadcast", "binomial", 1)]
        for algo in ("chain_pipe", "binomial_pipe", "bidir_ring"):
            kstar = model.best_chunks(algo, 8, M, 5e-6, 450e9)
            cases += [("broadcast", algo, k) for k in sorted({1, 8, 64, kstar}) if k <= M]
        cases += [("broadcast", "scatter_allgather", 1), ("scatter", "binomial", 1), ("scatter", "linear", 1),
                  ("gather", "binomial", 1)]
        for kind, algo, k in cases:
            fn = coll.COLLECTIVE_FNS[kind]
            med, mn = time_call(lambda: fn(list(live), algo=algo, root=0, chunks=k), pristine, live)
            ot = oracle_time(kind, algo, host, "uint8", 0, k) if host is not None else None
            record("C2", kind, algo, "uint8", 8, M, k, med, mn, ot)
        del pristine, live

    # C3: AllReduce, 8 ranks, fp32 N(0,1) / bf16 N(0,0.02), 4 KiB .. 256 MiB
    for dtype, sigma in (("float32", 1.0), ("bfloat16", 0.02)):
        for lg in range(12, 29, 4 if quick else 1):
            count = (1 << lg) // si.ITEMSIZE[dtype]
            small = lg <= 24
            host = si.rank_arrays(3, 8, count, dtype, sigma=sigma) if small else None
            pristine = (torch.stack([si.host_to_tensor(x, dtype, dev) for x in host]) if small else
                        torch.stack(si.device_rank_tensors(3, 8, count, dtype, dev, sigma=sigma)))
            live = pristine.clone()
            for algo in ("ring", "rhd", "dbt"):
                med, mn = time_call(lambda: coll.coll_allreduce(list(live), algo=algo), pristine, live)
                ot = oracle_time("allreduce", algo, host, dtype) if small and lg <= 22 else None
                record("C3", "allreduce", algo, dtype, 8, count, 1, med, mn, ot)
            del pristine, live
            torch.cuda.empty_cache()

    # Tree Reduce, 8 ranks, fp32 (the Reduce the pages pair with the tree Broadcast)
    for lg in ((20, 28) if quick else (12, 16, 20, 24, 28)):
        count = (1 << lg) // 4
        pristine = torch.stack(si.device_rank_tensors(3, 8, count, "float32", dev))
        live = pristine.clone()
        med, mn = time_call(lambda: coll.coll_reduce(list(live), algo="binomial", root=0), pristine, live)
        record("reduce", "reduce", "binomial", "float32", 8, count, 1, med, mn)
        del pristine, live

    # C4: ReduceScatter and AllGather, 64 ranks x 256 MiB bf16 (16 GiB resident)
    if not quick:
        count = (256 << 20) // 2
        pristine = torch.empty((64, count), dtype=torch.bfloat16, device=dev)
        si.device_rank_tensors(4, 64, count, "bfloat16", dev, sigma=1e-3, out=pristine)
        live = pristine.clone()
        for algo in ("ring", "rhd"):
            for kind in ("reducescatter", "allgather"):
                fn = coll.COLLECTIVE_FNS[kind]
                med, mn = time_call(lambda: fn(list(live), algo=algo), pristine, live)
                record("C4", kind, algo, "bfloat16", 64, count, 1, med, mn)
        del pristine, live
        torch.cuda.empty_cache()

    # C5: AllToAll, 32 ranks, 512 tokens x 4096 bf16 per peer
    N, B = 32, 512 * 4096
    pristine = torch.empty((N, N * B), dtype=torch.bfloat16, device=dev)
    si.device_rank_tensors(5, N, N * B, "bfloat16", dev, out=pristine)
    recv = torch.empty_like(pristine)
    for algo in ("pairwise", "bruck", "ring"):
        med, mn = time_call(lambda: coll.coll_alltoall(list(pristine), list(recv), algo=algo), pristine, pristine)
        record("C5", "alltoall", algo, "bfloat16", N, N * B, 1, med, mn)
    del pristine, recv
    torch.cuda.empty_cache()

    # the pages' alpha-beta form refitted to this engine over the fp32 Ring
    # AllReduce sizes: one launch per call whatever the step count, so
    # t = alpha_call + moved_bytes / beta_g
    pts = [r for r in rows if r["config"] == "C3" and r["algo"] == "ring" and r["dtype"] == "float32"]
    A = np.array([[1.0, r["moved_bytes"]] for r in pts], dtype=np.float64)
    t = np.array([r["t_med_us"] * 1e-6 for r in pts])
    coef, *_ = np.linalg.lstsq(A, t, rcond=None)
    fit = {"fit": "t = alpha_call + moved_bytes / beta_g over C3 fp32 Ring",
           "alpha_call_us": round(coef[0] * 1e6, 3), "beta_g_TBps": round(1 / coef[1] / 1e12, 3) if coef[1] > 0 else None}
    with open(out_path, "a") as fh:
        fh.write(json.dumps(fit) + "\n")
    print(json.dumps(fit), file=sys.stderr)


def calibrate(dev, gib: int = 2, reps: int = 10) -> dict:
    """Achievable HBM rate of plain streams: copy reads and writes each byte
    once (2 x bytes moved), add reads two operands and writes one (3 x bytes);
    and of the column kernel's access patterns without its programs (loads of
    one 1 KiB tile from each of L buffers, stores to each of S buffers, per
    one-wave work group): a fill, an 8-rank AllReduce in place, Reduce and
    Broadcast over 8 ranks, a 64-rank ReduceScatter and AllGather segment."""
    import torch
    import collective_communication_algorithms_amd as coll
    n = (gib << 30) // 4
    a = torch.randn(n, device=dev)
    b = torch.randn(n, device=dev)
    c = torch.empty(n, device=dev)
    out = {}
    for name, fn, moved in (("copy", lambda: coll.coll_calib_copy(c, a), 2),
                            ("add", lambda: coll.coll_calib_add(c, a, b), 3)):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        out[name] = {"bytes": moved * n * 4, "ms": round(ms, 4), "GBps": round(moved * n * 4 / ms / 1e6, 1)}
    # the column kernel's access patterns without its programs, over one 2 GiB
    # pool cut into the buffers each pattern names (coll_calib_pattern)
    del a, b, c
    pool = torch.zeros((2 << 30) // 4, device=dev)
    pats = {}
    for name, nl, ns, nbuf, loads_of, stores_of in (
            ("fill", 0, 1, 1, lambda v: [], lambda v: v[:1]),
            ("allreduce_8_ranks_in_place", 8, 8, 8, lambda v: v, lambda v: v),
            ("reduce_8_ranks", 8, 1, 8, lambda v: v, lambda v: v[:1]),
            ("broadcast_8_ranks", 1, 7, 8, lambda v: v[:1], lambda v: v[1:]),
            ("reducescatter_64_ranks", 64, 1, 64, lambda v: v, lambda v: v[:1]),
            ("allgather_64_ranks", 1, 63, 64, lambda v: v[:1], lambda v: v[1:])):
        views = list(pool.view(nbuf, -1))
        ld, st = loads_of(views), stores_of(views)
        nbytes = views[0].numel() * 4
        coll.coll_calib_pattern(ld, st)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            coll.coll_calib_pattern(ld, st)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        moved = (nl + ns) * nbytes
        pats[name] = {"loads": nl, "stores": ns, "bytes_per_buffer": nbytes, "bytes": moved, "ms": round(ms, 4),
                      "GBps": round(moved / ms / 1e6, 1)}
        if name == "allreduce_8_ranks_in_place":
            # the same pattern with each CU held to fewer work groups at once
            for groups in (4, 8, 16):
                coll.coll_calib_pattern(ld, st, groups_per_cu=groups)
                torch.cuda.synchronize()
                s.record()
                for _ in range(reps):
                    coll.coll_calib_pattern(ld, st, groups_per_cu=groups)
                e.record()
                torch.cuda.synchronize()
                ms = s.elapsed_time(e) / reps
                pats[f"{name}_{groups}_groups_per_cu"] = {"loads": nl, "stores": ns, "bytes_per_buffer": nbytes,
                                                          "bytes": moved, "ms": round(ms, 4),
                                                          "GBps": round(moved / ms / 1e6, 1)}
    return {"calibration": out, "buffer_GiB": gib, "access_patterns": pats}


def overlap(out_path: str, dev) -> None:
    """A collective on a side stream beside a stand-in compute kernel (the HCCL
    blog, 延迟掩盖：计算与通信的Overlap and Overlap的性能收益).

    Workload: Ring AllReduce fp32, 8 ranks, 64 MiB and 256 MiB per rank, in
    place.  The compute is ``coll_calib_spin``: register-only FMA chains, sized
    to 0.5x, 1x and 2x the collective's time, on 256 or 1,024 work groups.
    Per configuration: compute alone, the collective alone, and both launched
    together (compute on the current stream, the collective on a second stream
    of default priority, each started after one event and joined by another),
    median of 10 after 2 warm-ups; the inputs are restored from a pristine copy
    before every run (not timed).  Reported beside the blog's estimate with and
    without overlap, and the share of the collective's time that was hidden.
    The collective is run at its default grid (every resident slot) and at
    smaller grids that leave compute units to the compute kernel.
    """
    import numpy as np
    import torch

    import collective_communication_algorithms_amd as coll
    import seeded_inputs as si
    from collective_communication_algorithms_amd import model

    main_s = torch.cuda.current_stream(dev)
    side_s = torch.cuda.Stream(dev)
    spin_out = torch.empty(1024 * 256, dtype=torch.float32, device=dev)
    reps, warm = 10, 2

    def run(fn_main, fn_side, restore):
        ts = []
        for i in range(warm + reps):
            restore()
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(main_s)
            side_s.wait_event(e0)
            if fn_main is not None:
                fn_main()
            if fn_side is not None:
                fn_side()
            e1.record(side_s)
            main_s.wait_event(e1)
            e2.record(main_s)
            e2.synchronize()
            if i >= warm:
                ts.append(e0.elapsed_time(e2))
        return float(np.median(ts))

    open(out_path, "w").close()
    N = 8
    for mib in (64, 256):
        count = (mib << 20) // 4
        pristine = torch.empty((N, count), dtype=torch.float32, device=dev)
        si.device_rank_tensors(3, N, count, "float32", dev, out=pristine)
        live = pristine.clone()
        ranks = list(live)

        def restore():
            live.copy_(pristine)

        def spin(iters, grid):
            return lambda: coll.coll_calib_spin(spin_out, iters, grid, stream=main_s)

        for spin_grid in (256, 1024):
            probe = 1 << 16
            t_probe = run(spin(probe, spin_grid), None, lambda: None)
            for max_grid in (0, 1536, 1024):
                coll.coll_set_option("max_grid", max_grid)
                comm = lambda: coll.coll_allreduce(ranks, algo="ring", stream=side_s)  # noqa: E731
                t_comm = run(None, comm, restore)
                for ratio in (0.5, 1.0, 2.0):
                    iters = int(min(1 << 28, max(1, probe * ratio * t_comm / t_probe)))
                    t_comp = run(spin(iters, spin_grid), None, lambda: None)
                    t_both = run(spin(iters, spin_grid), comm, restore)
                    r = {"workload": f"ring_allreduce_fp32_n8_{mib}MiB", "spin_grid": spin_grid,
                         "coll_max_grid": max_grid, "ratio": ratio, "spin_iters": iters,
                         "t_compute_ms": round(t_comp, 4), "t_comm_ms": round(t_comm, 4),
                         "t_both_ms": round(t_both, 4),
                         "model_overlap_ms": round(model.overlapped_time(t_comp, t_comm), 4),
                         "model_no_overlap_ms": round(model.serial_time(t_comp, t_comm), 4),
                         "hidden_fraction": round(model.hidden_fraction(t_comp, t_comm, t_both), 3),
                         "both_over_model": round(t_both / model.overlapped_time(t_comp, t_comm), 3)}
                    with open(out_path, "a") as fh:
                        fh.write(json.dumps(r) + "\n")
                    print(json.dumps(r), file=sys.stderr, flush=True)
        coll.coll_set_option("max_grid", 0)
        torch.cuda.synchronize()
        del pristine, live, ranks
        torch.cuda.empty_cache()


def latency(out_path: str, dev) -> None:
    """Small calls: where their time goes (C1: Ring / RHD / DBT AllReduce over
    4 ranks x 1,024 int32; C3's smallest: 8 ranks x 4 KiB fp32), in place.

    Per call, in microseconds:
      alone_api / alone_abi  one call between HIP events on its stream, after
                    the previous one finished (median of 300), through the
                    Python binding / straight through the C ABI (ctypes, the
                    pointer arrays built once);
      host_api / host_abi  host time per call of 2,000 calls issued back to
                    back (the stream's time per call is reported beside it);
      kernel        the library's own events around its kernels
                    (COLL_OPT_TIMING, median of 200);
      graph         a HIP graph of 20 calls captured once and replayed 50
                    times: the device's time per call with no host in the
                    loop (kernel launch and the kernel's dependent memory
                    round trips)."""
    import ctypes

    import numpy as np
    import torch

    import collective_communication_algorithms_amd as coll
    from collective_communication_algorithms_amd import _lib
    from collective_communication_algorithms_amd._lib import check

    lib = _lib.load()
    stream = torch.cuda.current_stream(dev)
    open(out_path, "w").close()

    def between_events(fn, n):
        ts = []
        for _ in range(n):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            e.synchronize()
            ts.append(s.elapsed_time(e) * 1e3)
        return float(np.median(ts)), float(np.min(ts))

    def back_to_back(fn, n=2000):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        h0 = time.perf_counter()
        for _ in range(n):
            fn()
        h1 = time.perf_counter()
        e1.record(stream)
        torch.cuda.synchronize()
        return (h1 - h0) / n * 1e6, e0.elapsed_time(e1) / n * 1e3

    for cfg, N, count, dtype in (("C1", 4, 1024, "int32"), ("C3", 8, 1024, "float32")):
        tdt = torch.int32 if dtype == "int32" else torch.float32
        buf = torch.ones((N, count), dtype=tdt, device=dev)
        ranks = list(buf)
        arr = (ctypes.c_void_p * N)(*[t.data_ptr() for t in ranks])
        for algo in ("ring", "rhd", "dbt"):
            def api():
                coll.coll_allreduce(ranks, algo=algo)

            def abi(s=None):
                check(lib.coll_allreduce(arr, None, N, count, _lib.DTYPES[dtype], _lib.OPS["sum"], _lib.ALGOS[algo],
                                         0, 1, ctypes.c_void_p(s if s is not None else stream.cuda_stream)))

            for _ in range(50):
                api()
            torch.cuda.synchronize()
            host_api, stream_api = back_to_back(api)
            host_abi, stream_abi = back_to_back(abi)
            alone_api = between_events(api, 300)
            alone_abi = between_events(abi, 300)
            coll.coll_set_option("timing", 1)
            ks = []
            for _ in range(200):
                abi()
                ks.append(coll.coll_last_kernel_ms() * 1e3)
            coll.coll_set_option("timing", 0)
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream(dev)
            cs.wait_stream(stream)
            with torch.cuda.graph(g, stream=cs):
                for _ in range(20):
                    abi(torch.cuda.current_stream(dev).cuda_stream)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(50):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_us = e0.elapsed_time(e1) / 50 / 20 * 1e3
            del g
            r = {"config": cfg, "algo": algo, "nranks": N, "bytes_per_rank": count * 4, "dtype": dtype,
                 "alone_api_us": round(alone_api[0], 2), "alone_api_min_us": round(alone_api[1], 2),
                 "alone_abi_us": round(alone_abi[0], 2), "alone_abi_min_us": round(alone_abi[1], 2),
                 "host_api_us": round(host_api, 2), "stream_api_us": round(stream_api, 2),
                 "host_abi_us": round(host_abi, 2), "stream_abi_us": round(stream_abi, 2),
                 "kernel_us": round(float(np.median(ks)), 2), "graph_us": round(graph_us, 2)}
            with open(out_path, "a") as fh:
                fh.write(json.dumps(r) + "\n")
            print(json.dumps(r), file=sys.stderr, flush=True)
        del buf, ranks


def single_call(args, dev) -> int:
    """``--call KIND``: one collective at one shape (``--mib`` or ``--kib`` per
    rank), for profiling its kernels.

    Inputs from torch's seeded device generator (workload 7).  One call on
    fresh inputs is checked on sampled columns against the collective's
    definition (copies and integer reductions exactly, floating-point sums
    within the binary32 error bound of the fp64 sum); then ``--warmup`` untimed
    and ``--steps`` timed calls, each alone between HIP events, on inputs
    restored before each call; with ``--checksums`` every call also computes
    the per-row checksums.  Prints one JSON line with the median time and the
    schedule bytes per second."""
    import numpy as np
    import torch

    import collective_communication_algorithms_amd as coll
    import seeded_inputs as si

    kind, algo, N, dtype = args.call, args.call_algo, args.nranks, args.dtype
    sz = si.ITEMSIZE[dtype]
    count = ((args.kib << 10) if args.kib else (args.mib << 20)) // sz
    if kind == "alltoall":
        count -= count % N
    root, k = args.root % N, args.chunks
    send = torch.empty((N, count), dtype=si.to_torch_dtype(dtype), device=dev)
    si.device_rank_tensors(7, N, count, dtype, dev, out=send)
    pristine = send.clone()
    recv = torch.empty_like(send) if kind == "alltoall" else None
    fn = coll.COLLECTIVE_FNS[kind]

    sums = None
    if args.checksums:
        # one slot per schedule row, set for every call below (the definition
        # check included)
        nrows = coll.coll_plan(kind, algo, N, count, dtype, root, k)[1]["rows"]
        sums = torch.zeros(max(nrows, 1), dtype=torch.int64, device=dev)

    def call():
        if sums is not None:
            coll.coll_set_checksums(sums)
        try:
            fn(list(send), list(recv) if recv is not None else None, algo=algo, root=root, chunks=k)
        finally:
            if sums is not None:
                coll.coll_set_checksums(None)

    def restore():
        send.copy_(pristine)

    # definition check on sampled columns (or, for AllToAll, sampled blocks)
    cols = np.unique(np.concatenate([np.arange(0, count, 4099), np.arange(0, min(count, 8192)),
                                     np.arange(max(0, count - 8192), count)]))
    cols_t = torch.from_numpy(cols).to(dev)
    x = pristine.index_select(1, cols_t).float().cpu().numpy().astype(np.float64) if dtype in ("float32", "bfloat16") \
        else pristine.index_select(1, cols_t).cpu().numpy().astype(np.int64)
    call()
    torch.cuda.synchronize()
    out = (recv if recv is not None else send)
    part = [i * count // N for i in range(N + 1)]
    ok = True
    if kind in ("allreduce", "reduce", "reducescatter"):
        got = out.index_select(1, cols_t).float().cpu().numpy().astype(np.float64) if dtype in ("float32", "bfloat16") \
            else out.index_select(1, cols_t).cpu().numpy().astype(np.int64)
        ranks = range(N) if kind == "allreduce" else ([root] if kind == "reduce" else range(N))
        for i in ranks:
            sel = np.ones(len(cols), bool) if kind != "reducescatter" else (cols >= part[i]) & (cols < part[i + 1])
            if dtype in ("float32", "bfloat16"):
                u = 2.0 ** -24 if dtype == "float32" else 2.0 ** -8
                bound = (N * u / (1 - N * u)) * np.abs(x).sum(axis=0) + (2.0 ** -8) * np.abs(x.sum(axis=0)) * (dtype == "bfloat16")
                ok &= bool(np.all(np.abs(got[i][sel] - x.sum(axis=0)[sel]) <= bound[sel]))
            else:
                want = (x.sum(axis=0) + 2 ** 31) % 2 ** 32 - 2 ** 31
                ok &= bool(np.array_equal(got[i][sel], want[sel]))
    elif kind == "alltoall":
        B = count // N
        for j in (0, N // 2, N - 1):
            for i in (0, N - 1):
                ok &= bool(torch.equal(out[j][i * B:(i + 1) * B], pristine[i][j * B:(j + 1) * B]))
    else:
        # copies: compare bit patterns (numpy has no bfloat16)
        bits = (lambda t: t.view(torch.int16)) if dtype == "bfloat16" else (lambda t: t)
        got = bits(out.index_select(1, cols_t)).cpu().numpy()
        src = bits(pristine.index_select(1, cols_t)).cpu().numpy()
        for i in range(N):
            if kind == "broadcast":
                ok &= bool(np.array_equal(got[i], src[root]))
            elif kind == "scatter":
                sel = (cols >= part[i]) & (cols < part[i + 1])
                ok &= bool(np.array_equal(got[i][sel], src[root][sel]))
            elif kind in ("gather", "allgather") and (kind == "allgather" or i == root):
                for r in range(N):
                    sel = (cols >= part[r]) & (cols < part[r + 1])
                    ok &= bool(np.array_equal(got[i][sel], src[r][sel]))
    if not ok:
        print(f"bench.py: {kind}/{algo} differs from the definition on sampled columns", file=sys.stderr)
        return 1
    stats = coll.coll_get_stats()
    for _ in range(args.warmup):
        restore()
        call()
    ts = []
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.steps):
        restore()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        call()
        e.record(stream)
        e.synchronize()
        ts.append(s.elapsed_time(e))
    ms = float(np.median(ts))
    # the host path and the device floor of a call: 200 calls issued back to
    # back (no restores, results not checked); the host's time per issued call
    # and the stream's time per call
    n_b2b = 200
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    h0 = time.perf_counter()
    for _ in range(n_b2b):
        call()
    h1 = time.perf_counter()
    b1.record(stream)
    torch.cuda.synchronize()
    restore()
    print(json.dumps({"call": kind, "algo": algo, "dtype": dtype, "nranks": N, "bytes_per_rank": count * sz,
                      "root": root, "chunks": k, "checksums": sums is not None, "steps": args.steps,
                      "ms_median": round(ms, 4),
                      "ms_min": round(float(np.min(ts)), 4),
                      "host_us_per_issued_call": round((h1 - h0) / n_b2b * 1e6, 2),
                      "back_to_back_us_per_call": round(b0.elapsed_time(b1) / n_b2b * 1e3, 2),
                      "schedule_steps": stats["steps"], "schedule_bytes": stats["hbm_bytes"],
                      "schedule_TBps": round(stats["hbm_bytes"] / (ms * 1e-3) / 1e12, 3),
                      "moved_bytes": stats["moved_bytes"], "round_trips": stats["round_trips"],
                      "moved_TBps": round(stats["moved_bytes"] / (ms * 1e-3) / 1e12, 3),
                      "check": "definition on sampled columns"}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--algo", default="ring", choices=["ring", "rhd", "dbt"])
    ap.add_argument("--exec", default="auto", choices=["auto", "rows", "step"],
                    help="auto: the column kernel; rows: the row kernel in one launch; step: a launch per step")
    ap.add_argument("--nranks", type=int, default=8)
    ap.add_argument("--mib", type=int, default=256, help="MiB per rank")
    ap.add_argument("--kib", type=int, default=0, help="with --call: KiB per rank (instead of --mib)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-checksums", action="store_true",
                    help="time the calls without the per-row checksums (the default computes them)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure the plain copy (1R+1W) and add (2R+1W) streams and exit")
    ap.add_argument("--sweep", metavar="OUT_JSONL", help="time every configuration's calls and exit")
    ap.add_argument("--quick", action="store_true", help="with --sweep: fewer sizes and repetitions")
    ap.add_argument("--call", choices=["allreduce", "reducescatter", "allgather", "broadcast", "scatter", "gather",
                                       "alltoall", "reduce"],
                    help="time one collective at one shape (with --call-algo, --nranks, --mib, --dtype) and exit")
    ap.add_argument("--call-algo", default="default")
    ap.add_argument("--checksums", action="store_true", help="with --call: every call computes the per-row checksums")
    ap.add_argument("--dtype", default="float32", choices=["int32", "uint8", "float32", "bfloat16"])
    ap.add_argument("--root", type=int, default=0)
    ap.add_argument("--chunks", type=int, default=1)
    ap.add_argument("--latency", metavar="OUT_JSONL",
                    help="time small calls (host path, kernels, graph replay) and exit")
    ap.add_argument("--overlap", metavar="OUT_JSONL",
                    help="time a collective on a side stream beside a stand-in compute kernel and exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                               "COPY_WRITE_CSV"),
                    help="write the traffic summary under profiles/ from rocprofv3 counter CSVs and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        out = summarize_counters(*args.summarize_counters, HEADLINE_KERNEL, TRAFFIC_FILE)
        print(json.dumps(out))
        return 0
    if args.gpus != 1:
        print("bench.py: the collectives run between N virtual ranks in one GPU's memory; "
              "--gpus above 1 is not supported", file=sys.stderr)
        return 2
    if args.steps < 1 or args.steps > 200:
        print("bench.py: --steps must be in [1, 200]", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import collective_communication_algorithms_amd as coll
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    if args.calibrate:
        print(json.dumps(calibrate(dev)))
        return 0
    if args.sweep:
        sweep(args.sweep, dev, args.quick)
        return 0
    if args.overlap:
        overlap(args.overlap, dev)
        return 0
    if args.latency:
        latency(args.latency, dev)
        return 0
    if args.call:
        return single_call(args, dev)
    N, M = args.nranks, args.mib << 20
    count = M // 4
    coll.coll_set_option("exec", {"auto": 0, "step": 1, "rows": 2}[args.exec])

    # inputs: 8 rank buffers of N(0,1) fp32 drawn by torch's seeded generator on
    # the device, and a pristine copy every call is restored from
    pristine = torch.empty((N, count), dtype=torch.float32, device=dev)
    si.device_rank_tensors(3, N, count, "float32", dev, out=pristine)
    buf = pristine.clone()
    ranks = list(buf)
    torch.cuda.synchronize()
    host_inputs = None
    if not args.no_cpu_baseline:
        host_inputs = [r.cpu().numpy() for r in pristine]

    def restore():
        buf.copy_(pristine)

    # before timing: one call on the fresh inputs, checked on sampled columns
    # against the definition (the fp64 sum over ranks) within the binary32
    # error bound of an N-term sum; the bit-exact comparison with the oracle
    # comes with the cpu_baseline leg below
    cols = np.unique(np.concatenate([np.arange(0, count, 4097), np.arange(0, 65536),
                                     np.arange(count - 65536, count),
                                     np.arange(count // N - 4096, count // N + 4096)]))
    cols_t = torch.from_numpy(cols).to(dev)
    sample_in = np.stack([r.index_select(0, cols_t).cpu().numpy() for r in pristine]).astype(np.float64)
    # per-row checksums (the u64 wrap-sum of each row's destination words after
    # the row) are part of every timed call unless --no-checksums
    sums = None
    if not args.no_checksums:
        plan_rows, _ = coll.coll_plan("allreduce", args.algo, N, count, "float32")
        sums = torch.zeros(len(plan_rows), dtype=torch.int64, device=dev)
        coll.coll_set_checksums(sums)
    coll.coll_allreduce(ranks, algo=args.algo)
    torch.cuda.synchronize()
    gpu_sample = [r.index_select(0, cols_t).cpu().numpy() for r in ranks]
    gpu_sums = sums.cpu().numpy().view(np.uint64).copy() if sums is not None else None
    exact = sample_in.sum(axis=0)
    u = 2.0 ** -24
    bound = (N * u / (1 - N * u)) * np.abs(sample_in).sum(axis=0)
    if not all(np.all(np.abs(g.astype(np.float64) - exact) <= bound) for g in gpu_sample):
        print("bench.py: GPU result outside the error bound of the fp64 sum", file=sys.stderr)
        return 1
    stats = coll.coll_get_stats()

    stream = torch.cuda.current_stream(dev)

    def timed_calls(k):
        ts = []
        for _ in range(k):
            restore()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            coll.coll_allreduce(ranks, algo=args.algo)
            e.record(stream)
            e.synchronize()
            ts.append(s.elapsed_time(e))
        return ts

    timed_calls(args.warmup)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    per_call = timed_calls(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = float(np.median(per_call))
    ms_min = float(np.min(per_call))
    # second pass: the data-moving kernels alone, between the library's events
    coll.coll_set_option("timing", 1)
    kernel_ms = []
    for _ in range(args.steps):
        restore()
        coll.coll_allreduce(ranks, algo=args.algo)
        kernel_ms.append(coll.coll_last_kernel_ms())
    coll.coll_set_option("timing", 0)
    # the same buffers under the kernel's access pattern alone: a tile of each
    # of the N ranks loaded, summed and stored back to each (no program, no
    # checksums), one-wave work groups of one 1 KiB tile, as the kernel runs
    # (the fastest of: every CU holding as many work groups as fit, or at most
    # 4 or 8 at once)
    pattern = None
    if N == 8:
        best = None
        for groups in (0, 4, 8):
            coll.coll_calib_pattern(ranks, ranks, groups_per_cu=groups)
            torch.cuda.synchronize()
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            for _ in range(args.steps):
                coll.coll_calib_pattern(ranks, ranks, groups_per_cu=groups)
            p1.record(stream)
            torch.cuda.synchronize()
            pattern_ms = p0.elapsed_time(p1) / args.steps
            if best is None or pattern_ms < best[0]:
                best = (pattern_ms, groups)
        pattern = {"pattern": "8 loads + 8 stores per 1 KiB tile, in place on the call's buffers (coll_calib_pattern), "
                              "the fastest of no cap and 4 or 8 work groups per CU",
                   "groups_per_cu": best[1], "ms": round(best[0], 4), "GBps": round(2 * N * M / best[0] / 1e6, 1)}
    # the earlier protocol, for reference: calls back to back on the same
    # buffers, no restore, mean time
    restore()
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(args.steps):
        coll.coll_allreduce(ranks, algo=args.algo)
    b1.record(stream)
    torch.cuda.synchronize()
    back_to_back_ms = b0.elapsed_time(b1) / args.steps
    if sums is not None:
        coll.coll_set_checksums(None)

    algbw = M / (ms * 1e-3) / 1e9
    busbw = algbw * 2 * (N - 1) / N
    moved = stats["moved_bytes"]           # what the kernels move: 2NM here
    hbm_bytes = stats["hbm_bytes"]         # 5(N-1)M: the schedule's row bytes
    launches = stats["steps"] if args.exec == "step" else 1
    launch_ms = float(np.mean(kernel_ms)) / launches
    achieved = moved / launches / (launch_ms * 1e-3) / 1e9
    traffic = load_traffic(moved / launches)
    from collective_communication_algorithms_amd import model
    pred_ms = model.time("allreduce", args.algo, N, M, 5e-6, 450e9) * 1e3
    engine = {"auto": "column kernel", "rows": "row kernel, one launch", "step": "row kernel, a launch per step"}

    result = {
        "metric": METRIC,
        "value": round(busbw, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: N(0,1) fp32 per rank from torch's seeded device generator",
        "config": {"workload": f"{args.algo}_allreduce_fp32_n{N}_{args.mib}MiB", "nranks": N,
                   "bytes_per_rank": M, "algo": args.algo, "op": "sum", "inplace": True,
                   "exec": engine[args.exec], "schedule_steps": stats["steps"], "checksums": sums is not None},
        "ms_min": round(ms_min, 4),
        "per_call_ms": [round(x, 4) for x in per_call],
        "timing": "each call alone between HIP events after an untimed restore of its inputs; median and min",
        "algbw_GBps": round(algbw, 2),
        "moved_bytes_per_call": moved,
        "hbm_pct_of_peak": round(100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "kernel_ms_mean": round(launch_ms, 4),
        "access_pattern_ceiling": (dict(pattern, kernel_frac=round(achieved / pattern["GBps"], 4))
                                   if pattern else None),
        # the schedule's row bytes (every row reading its operands and writing
        # its destination through memory) per median call: a rate no kernel
        # moves, kept for comparison with the pages' step model
        "schedule_bytes_per_call": hbm_bytes,
        "schedule_rate_GBps": round(hbm_bytes / (ms * 1e-3) / 1e9, 1),
        "back_to_back_mean_ms": round(back_to_back_ms, 4),
        "cpu_baseline": None,
        "alpha_beta_page_model_ms": round(pred_ms, 4),
        "parity": "within the binary32 error bound of the fp64 sum on %d sampled columns per rank" % len(cols),
        "wall_s_timed_region": round(wall, 4),
    }
    del buf, ranks, pristine
    torch.cuda.empty_cache()
    if host_inputs is not None:
        result["cpu_baseline"] = cpu_baseline(host_inputs, N, count, args.algo, cols, gpu_sample, gpu_sums=gpu_sums)
        if not result["cpu_baseline"]["matches_gpu"]:
            print("bench.py: GPU result differs from the oracle on sampled columns", file=sys.stderr)
            return 1
        if result["cpu_baseline"].get("checksums_match_gpu") is False:
            print("bench.py: GPU row checksums differ from the oracle's", file=sys.stderr)
            return 1
        result["parity"] = "bit-exact vs the oracle on %d sampled columns per rank" % len(cols) + (
            ", every row checksum equal to the oracle's" if gpu_sums is not None else "")
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
