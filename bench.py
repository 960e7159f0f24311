#!/usr/bin/env python3
"""Benchmark: one step = the whole SEACells FW hot path on one GPU.

A step runs the A update (T = 50 Frank-Wolfe steps for every cell), the
B-gradient argmin over all cells, and the B step, back to back on one
stream, over a seeded synthetic kNN-kernel workload already resident in
HBM. The JSON line reports cells/s for the whole step, the roofline of the
dominant kernel (algorithmic bytes per launch / average launch time from HIP
events on the library's stream), and the f64 CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config c5] [--gpus 1] [--prune THR]
                    [--no-operands] [--no-cpu-baseline]

After the timed steps it also times the device construction of the
operands from K, B and A^T ("operands": whole build and per step), a few
steps of the on-device B loop ("b_loop") and one whole outer iteration
("iteration": A update, operands, B loop, RSS).

The default workload is the largest single-GPU configuration (n = 1M cells,
k = 10000 archetypes); --config c1 .. c4 selects the smaller ones. --prune
runs the A update's pruning variant (weights at or below THR dropped after
every step, then the column renormalised); its byte model leaves out the t1
rows that drops take back out, so its GB/s is a lower bound.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "cells/s per FW A-update (T=50) + B-argmin; achieved HBM GB/s vs peak"


def algorithmic_bytes_a(w, trace, atom_cnt):
    """What the A update must move (index + value = 8 B per non-zero).

    K2B row and A_prev row once per cell, one t1 row (entries + its row
    pointer pair) per seed and per step, the two row-pointer pairs of each
    cell, and the atom lists written."""
    rt1 = np.diff(w.t1.indptr).astype(np.int64)
    ap = w.a_prev_t
    seed_rows = int(rt1[ap.indices].sum())
    pick_rows = int(rt1[trace.reshape(-1)].sum())
    n = w.n
    return (8 * w.k2b.nnz + 8 * ap.nnz + 8 * (seed_rows + pick_rows)
            + 8 * (ap.nnz + n * w.T) + 2 * 4 * (n + 1) + 8 * int(atom_cnt.sum()) + 4 * n)


def algorithmic_bytes_b(w):
    """What the B argmin must move: K2B, K2At and B once, one AAt row (entries
    + row-pointer pair) per non-zero of K2B, the row pointers, the output."""
    raat = np.diff(w.aat.indptr).astype(np.int64)
    gathers = int((raat[w.k2b.indices] + 1).sum())
    return (8 * w.k2b.nnz + 8 * w.k2at.nnz + 8 * w.b.nnz + 12 * (w.n + 1)
            + 8 * gathers + 8 * w.k)


def source_sha(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_archetypal_analysis_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, workload, sha):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(kernel, {}).get(workload)
    if not e or e.get("source_sha") != sha:
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s=12.0):
    """The f64 oracle, as it stands, on a bounded sample of the workload."""
    import scipy.sparse as sp
    import oracle

    threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    # A: one cell per thread to measure the rate, then a sample sized to the budget
    probe = rng.choice(w.n, size=min(threads, w.n), replace=False)
    t0 = time.time()
    oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=probe, n_threads=threads)
    rate = probe.shape[0] / max(time.time() - t0, 1e-6)
    m_a = int(min(w.n, max(threads, rate * budget_s / 2)))
    cells = rng.choice(w.n, size=m_a, replace=False)
    t0 = time.time()
    oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells, n_threads=threads)
    t_a = time.time() - t0
    # B: the first rows of every n x k operand, sized the same way
    def rows(m, r):
        return sp.csr_matrix(m[:r])
    r = min(w.n, 2000)
    t0 = time.time()
    oracle.fw_b_argmin(rows(w.k2b, r), w.aat, rows(w.k2at, r), rows(w.b, r), r, w.k,
                       n_threads=threads)
    per_row = max((time.time() - t0) / r, 1e-9)
    r = int(min(w.n, max(r, (budget_s / 2) / per_row)))
    t0 = time.time()
    oracle.fw_b_argmin(rows(w.k2b, r), w.aat, rows(w.k2at, r), rows(w.b, r), r, w.k,
                       n_threads=threads)
    t_b = time.time() - t0
    rate_a = cells.shape[0] / t_a
    rate_b = r / t_b
    value = 1.0 / (1.0 / rate_a + 1.0 / rate_b)
    cpu = "?"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": value, "unit": "cells/s", "cores": threads, "kind": "oracle",
            "sample": "A update on %d random cells (T=%d, %.1f s), B argmin over the first %d "
                      "cells (%.1f s); value = 1/(1/A + 1/B) in cells/s; %s"
                      % (cells.shape[0], w.T, t_a, r, t_b, cpu),
            "a_cells_per_s": rate_a, "b_cells_per_s": rate_b}


def time_operands(saa, W, w, stream, reps=3):
    """The operand construction on the device (K^2 B, t1, A A^T, K^2 A^T and
    the RSS from K, B and A^T): wall time of the whole build (one host
    synchronisation per product sizes its output) and the device time of each
    step from HIP events, outputs preallocated. For every product, the number
    of multiply-adds and the gathered bytes they imply: each reads its B
    entry's column in the rows pass and its column and value in the fill
    pass (12 B), plus the column once more (16 B) when the fill pass has to
    mark the row's columns again (no kept bitmaps)."""
    import torch
    D = saa.DeviceCSR.from_scipy
    K = W.kernel_matrix(w)
    dK, dB, dAt = D(K), D(w.b), D(w.a_prev_t)
    st = saa.new_status()
    ops = saa.device_operands(dK, dB, dAt, status=st)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        saa.device_operands(dK, dB, dAt, status=st)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / reps

    def dev_ms(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def n_products(a, b):
        cols = a.col_idx.cpu().numpy()
        lens = np.diff(b.row_ptr.cpu().numpy().astype(np.int64))
        return int(np.dot(np.bincount(cols, minlength=a.shape[1]).astype(np.int64), lens))

    res = {}
    plan = (("kb = K B", "kb", dK, dB), ("k2b = K kb", "k2b", dK, ops["kb"]),
            ("t1 = B^T k2b", "t1", ops["bt"], ops["k2b"]), ("aat = A A^T", "aat", ops["a"], dAt),
            ("kat = K A^T", "kat", dK, dAt), ("k2at = K kat", "k2at", dK, ops["kat"]))
    for label, nm, a, b in plan:
        c = ops[nm]
        # the workspace csr_matmul would take (the rows pass keeps its bitmaps)
        nbytes = saa.seacells_csr_matmul_pattern_workspace(a.shape[0], b.shape[1])
        kept = 0 < nbytes <= saa.native.PATTERN_WORKSPACE_LIMIT
        if not kept:
            nbytes = saa.seacells_csr_matmul_workspace(a.shape[0])
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

        def prod(a=a, b=b, c=c, ws=ws):
            saa.seacells_csr_matmul_rows(a, b, c.row_ptr, workspace=ws, status=st, stream=stream)
            saa.seacells_csr_matmul_fill(a, b, c.row_ptr, c.col_idx, c.val, workspace=ws,
                                         status=st, stream=stream)
        ms = dev_ms(prod)
        npr = n_products(a, b)
        per = 12.0 if kept else 16.0
        res[label] = {"ms": ms, "nnz": c.nnz, "products": npr, "gather_bytes_per_product": per,
                      "gather_gbps": per * npr / (ms * 1e-3) / 1e9}
    for label, src, nm in (("bt = B^T", dB, "bt"), ("a = (A^T)^T", dAt, "a")):
        t = ops[nm]
        res[label] = {"ms": dev_ms(lambda src=src, t=t: saa.seacells_csr_transpose(
            src, t.row_ptr, t.col_idx, t.val, status=st, stream=stream)), "nnz": t.nnz}
    acc = torch.zeros(1, dtype=torch.float64, device="cuda")
    res["rss"] = {"ms": dev_ms(lambda: saa.rss(dK, ops["k2b"], dAt, ops["t1"], ops["aat"],
                                               acc=acc, status=st, stream=stream))}
    saa.raise_on_status(st)
    return {"ms_total": wall_ms, "device_ms_sum": float(sum(v["ms"] for v in res.values())),
            "nnz_K": int(K.nnz), "steps": res,
            "note": "ms_total includes one host synchronisation per product (output sizing)"}


def time_b_loop(saa, W, w, steps, argmin_ms, stream):
    """The B update as a loop of Frank-Wolfe steps on the device (A fixed):
    per step the B argmin, the vertex matrix of its picks, B <- (1-g) B + g S
    and K^2 B <- (1-g) K^2 B + g K (K S). Wall time per step (the host reads
    output sizes once per product and sum); one update (g = 1/2) on the
    starting state timed on its own; and the argmin on the loop's last K^2 B,
    which grows with every step, so that the step splits into its parts."""
    import torch
    D = saa.DeviceCSR.from_scipy
    K = W.kernel_matrix(w)
    dK, k2b, aat, k2at, b = D(K), D(w.k2b), D(w.aat), D(w.k2at), D(w.b)
    st = saa.new_status()
    saa.fw_b_loop(dK, k2b, aat, k2at, b, 1, status=st, stream=stream)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    b2, k2b2, picks, _, _ = saa.fw_b_loop(dK, k2b, aat, k2at, b, steps, status=st, stream=stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps

    def update():
        S = saa.seacells_fw_b_vertex(picks[0], w.n, 1.0, status=st, stream=stream)
        saa.csr_add(0.5, b, 0.5, S, status=st, stream=stream)
        k2s = saa.csr_matmul(dK, saa.csr_matmul(dK, S, status=st, stream=stream), status=st,
                             stream=stream)
        saa.csr_add(0.5, k2b, 0.5, k2s, status=st, stream=stream)

    update()  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    update()
    torch.cuda.synchronize()
    upd_ms = (time.perf_counter() - t0) * 1000.0
    t0 = time.perf_counter()
    saa.seacells_fw_b_argmin(k2b2, aat, k2at, b2, w.n, w.k, status=st, stream=stream)
    torch.cuda.synchronize()
    last_ms = (time.perf_counter() - t0) * 1000.0
    saa.raise_on_status(st)
    return {"steps": steps, "ms_per_step": ms, "argmin_ms": argmin_ms,
            "argmin_ms_last_k2b": last_ms, "update_ms": upd_ms, "nnz_b": b2.nnz,
            "nnz_k2b": k2b2.nnz, "nnz_k2b_start": int(w.k2b.nnz)}


def time_iteration(saa, W, w, steps_b, stream):
    """One SEACells outer iteration on the device (saa.outer_iteration): t1,
    the A update (T steps), A^T, A A^T, K^2 A^T, steps_b B steps and the
    RSS. Wall time (one host read of each output size), and the RSS."""
    import torch
    D = saa.DeviceCSR.from_scipy
    K = W.kernel_matrix(w)
    dK, b, k2b, at = D(K), D(w.b), D(w.k2b), D(w.a_prev_t)
    st = saa.new_status()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = saa.outer_iteration(dK, b, k2b, at, w.T, steps_b, status=st, stream=stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0
    saa.raise_on_status(st)
    return {"steps_a": w.T, "steps_b": steps_b, "ms": ms, "rss": float(res["rss"].item()),
            "nnz_a_t": res["a_t"].nnz, "nnz_k2at": res["k2at"].nnz, "nnz_aat": res["aat"].nnz,
            "note": "first call of the process (includes the padded copies and one-off "
                    "allocations)"}


def copy_calibration(mib):
    """A plain elementwise copy of known size: it reads and writes exactly
    mib MiB per launch, so FETCH_SIZE / WRITE_SIZE of this kernel give the
    scale between those counters and bytes."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-operands", action="store_true",
                    help="skip timing the device operand construction")
    ap.add_argument("--b-loop-steps", type=int, default=3,
                    help="B-loop steps timed after the main steps (0 skips)")
    ap.add_argument("--iteration-b-steps", type=int, default=2,
                    help="B steps of the timed outer iteration (0 skips the iteration)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--prune", type=float, default=None, metavar="THR",
                    help="time the A update's pruning variant with threshold THR")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 launches), the reference "
                         "kernel that scales the HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path's multi-GPU sharding is a design, "
              "not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_archetypal_analysis_amd as saa
    import workloads as W

    t_gen = time.time()
    w = W.make(args.config, log=lambda m: print(m, file=sys.stderr, flush=True))
    t_gen = time.time() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    D = saa.DeviceCSR.from_scipy
    t1, k2b, ap_, aat, k2at, bm = (D(w.t1), D(w.k2b), D(w.a_prev_t), D(w.aat), D(w.k2at), D(w.b))
    n, k, T, cap = w.n, w.k, w.T, w.cap
    steps, warm = args.steps, args.warmup
    cap_b = int(np.diff(w.b.tocsc().indptr).max()) + steps + warm + 2
    bi, bv, bc = W.bt_padded(w.b, cap_b)
    bt_idx = torch.from_numpy(bi.astype(np.int32)).to(dev)
    bt_val = torch.from_numpy(bv).to(dev)
    bt_cnt = torch.from_numpy(bc.astype(np.int32)).to(dev)
    # outputs and workspaces, allocated once
    atom_idx = torch.empty((n, cap), dtype=torch.int32, device=dev)
    atom_val = torch.empty((n, cap), dtype=torch.float32, device=dev)
    atom_cnt = torch.empty(n, dtype=torch.int32, device=dev)
    ws_a_bytes = saa.seacells_fw_a_columns_workspace(n, k, T, cap, w.t1.nnz)
    ws_a = torch.empty(max(ws_a_bytes, 1), dtype=torch.uint8, device=dev)
    out_val = torch.empty(k, dtype=torch.float32, device=dev)
    out_idx = torch.empty(k, dtype=torch.int32, device=dev)
    gap = torch.empty(1, dtype=torch.float32, device=dev)
    ws_b = torch.empty(saa.seacells_fw_b_argmin_workspace(n, k, w.aat.nnz), dtype=torch.uint8,
                       device=dev)
    st_a, st_b, st_p = saa.new_status(dev), saa.new_status(dev), saa.new_status(dev)
    stream = torch.cuda.current_stream()

    prune = args.prune
    if prune is None:
        a_update = saa.seacells_fw_a_columns
    else:
        def a_update(*a, **kw):
            return saa.seacells_fw_a_columns_pruned(*a, threshold=prune, **kw)

    # one traced run (outside the timing) for the byte model: the trace is
    # deterministic, so the timed runs take the same picks
    trace = torch.empty((n, T), dtype=torch.int32, device=dev)
    a_update(t1, k2b, ap_, n, k, T, cap, atom_idx=atom_idx, atom_val=atom_val,
             atom_cnt=atom_cnt, trace=trace, workspace=ws_a, status=st_a)
    torch.cuda.synchronize()
    saa.raise_on_status(st_a)
    bytes_a = algorithmic_bytes_a(w, trace.cpu().numpy(), atom_cnt.cpu().numpy())
    bytes_b = algorithmic_bytes_b(w)
    del trace

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(t, marks=None):
        if marks:
            marks[0].record(stream)
        a_update(t1, k2b, ap_, n, k, T, cap, atom_idx=atom_idx, atom_val=atom_val,
                 atom_cnt=atom_cnt, workspace=ws_a, status=st_a, stream=stream)
        if marks:
            marks[1].record(stream)
        saa.seacells_fw_b_argmin(k2b, aat, k2at, bm, n, k, out_val=out_val, out_idx=out_idx,
                                 gap=gap, workspace=ws_b, status=st_b, stream=stream)
        if marks:
            marks[2].record(stream)
        # B loop index continues after the s_B prior steps of the workload
        saa.seacells_fw_b_apply(bt_idx, bt_val, bt_cnt, n, out_idx,
                                2.0 / (w.cfg.s_b + 1 + t + 2), status=st_p, stream=stream)
        if marks:
            marks[3].record(stream)

    for t in range(warm):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(steps):
        step(warm + t, ev[t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for st in (st_a, st_b, st_p):
        saa.raise_on_status(st)

    a_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    p_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    ms_step = wall * 1000.0 / steps
    a_gbps = bytes_a / (a_ms * 1e-3) / 1e9
    b_gbps = bytes_b / (b_ms * 1e-3) / 1e9
    dominant = "fw_a_columns" if a_ms >= b_ms else "fw_b_argmin"
    if dominant == "fw_a_columns":
        ach, per_launch, sha = a_gbps, bytes_a, source_sha("fw_a.hip")
    else:
        ach, per_launch, sha = b_gbps, bytes_b, source_sha("fw_b.hip")
    traffic = None if prune is not None else traffic_from_profile(dominant, args.config, sha)

    rec = {
        "metric": METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "cells/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (args.config, W.DESCRIPTIONS.get(args.config, "")),
                   "n": n, "k": k, "T": T, "cap": cap, "nnz": w.meta.get("nnz"),
                   "prune_threshold": prune},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": ach, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS,
                     "bytes_per_launch": per_launch, "traffic": traffic},
        "kernels_ms": {"fw_a_columns": a_ms, "fw_b_argmin": b_ms, "fw_b_apply": p_ms},
        "kernels_gbps": {"fw_a_columns": a_gbps, "fw_b_argmin": b_gbps},
        "a_cells_per_s": n / (a_ms * 1e-3),
        "b_cells_per_s": n / (b_ms * 1e-3),
        "generation_s": t_gen,
        "device": torch.cuda.get_device_name(dev),
    }
    if not args.no_operands:
        rec["operands"] = time_operands(saa, W, w, stream)
    if args.b_loop_steps > 0:
        rec["b_loop"] = time_b_loop(saa, W, w, args.b_loop_steps, b_ms, stream)
    if args.iteration_b_steps > 0:
        rec["iteration"] = time_iteration(saa, W, w, args.iteration_b_steps, stream)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
