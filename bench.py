#!/usr/bin/env python3
"""Benchmark: one step = the whole SEACells FW hot path on one GPU.

A step runs the A update (T = 50 Frank-Wolfe steps for every cell), the
B-gradient argmin over all cells, and the B step, back to back on one
stream, over a seeded synthetic kNN-kernel workload already resident in
HBM. The JSON line reports cells/s for the whole step, the roofline of the
dominant call (algorithmic bytes per launch / average launch time from HIP
events on the library's stream; beside it the bytes the rocprofv3 counters
saw beyond L2 and the compulsory bytes, each as a fraction of HBM peak), and
the f64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config c5] [--gpus 1] [--prune THR]
                    [--no-operands] [--no-cpu-baseline]
    python bench.py --table [--table-configs c1,c2,c3,c4,c5]
    python bench.py --summarize-profile OUT.md --config c5 --trace DIR --fetch DIR
                    --write DIR --copy-fetch DIR --copy-write DIR [--counters DIR ...]

--table times the A update and the B argmin alone on every workload (median
of at least 20 calls, 5 at the two largest), with the oracle's times beside
them (every cell and row at n <= 100k, 1 thread too at n <= 20k; a sample
scaled up above). --summarize-profile turns rocprofv3 output folders (kernel
trace, FETCH_SIZE and WRITE_SIZE runs of this script, the same counters on
--copy-calibration) into a markdown summary and the per-call traffic record
in profiles/traffic.json.

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


def compulsory_bytes_a(w, atom_cnt):
    """Every input of the A update read once (K2B, A_prev, t1 with their row
    pointers) and the atoms and counts written."""
    return (8 * (w.k2b.nnz + w.a_prev_t.nnz + w.t1.nnz) + 4 * (2 * (w.n + 1) + w.k + 1)
            + 8 * int(atom_cnt.sum()) + 4 * w.n)


def compulsory_bytes_b(w):
    """Every input of the B argmin read once (K2B, K2At, B, AAt with their
    row pointers) and the k (value, row) outputs written."""
    return (8 * (w.k2b.nnz + w.k2at.nnz + w.b.nnz + w.aat.nnz) + 4 * (3 * (w.n + 1) + w.k + 1)
            + 8 * w.k)


def source_sha(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_archetypal_analysis_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CALL_SOURCES = {"fw_a_columns": ("fw_a.hip", "common.hpp"),
                "fw_b_argmin": ("fw_b.hip", "common.hpp")}


def traffic_from_profile(call, workload, sha):
    """Bytes beyond L2 per call from the committed counter record, or None
    when the call's sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        rec = json.load(f)
    e = rec.get(call, {}).get(workload)
    if not e or e.get("source_sha") != sha:
        return None
    return e.get("bytes_per_call")


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
    walls = []
    for _ in range(2):  # the inputs are not modified: both calls do the same work
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = saa.outer_iteration(dK, b, k2b, at, w.T, steps_b, status=st, stream=stream)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) * 1000.0)
        saa.raise_on_status(st)
    return {"steps_a": w.T, "steps_b": steps_b, "ms": walls[1], "ms_first_call": walls[0],
            "rss": float(res["rss"].item()), "nnz_a_t": res["a_t"].nnz,
            "nnz_k2at": res["k2at"].nnz, "nnz_aat": res["aat"].nnz,
            "note": "ms: the second call; the first also makes the padded copies and the "
                    "caching allocator's first allocations"}


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


# --------------------------------------------------------------------------
# rocprofv3 summaries (CPU only)
# --------------------------------------------------------------------------

A_KERNELS = ("fw_a_", "pad_rows_kernel", "pad_fill_kernel", "cell_key_kernel", "key_scan_kernel",
             "cell_scatter_kernel", "fill_u32_kernel")
B_KERNELS = ("seg_table_kernel", "row_slice_kernel", "pa_count_kernel", "pa_bscan_kernel",
             "pa_offs_kernel", "pa_fill_kernel",
             "pc_fill_kernel", "col_walk_kernel", "slice_order_kernel", "hist_zero_kernel",
             "ref_hist_kernel", "slice_work_kernel", "xcd_assign_kernel", "xcd_work_zero_kernel",
             "fw_b_partials_kernel", "fw_b_reduce1_kernel", "fw_b_reduce2_kernel",
             "fw_b_fw_gap_kernel")


def _kname(raw):
    """A kernel's name without return type, namespaces and argument list."""
    nm = raw.strip()
    if nm.startswith("void "):
        nm = nm[5:]
    depth, cut = 0, len(nm)
    for i, ch in enumerate(nm):  # the argument list: the first '(' outside <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not nm[i:].startswith("(anonymous"):
            cut = i
            break
    nm = nm[:cut]
    for ns in ("seacells::(anonymous namespace)::", "seacells::"):
        nm = nm.replace(ns, "")
    return nm.strip()


def _call_of(kernel):
    if kernel.startswith(A_KERNELS):
        return "fw_a_columns"
    if kernel.startswith(B_KERNELS):
        return "fw_b_argmin"
    if kernel.startswith("fw_b_apply_kernel"):
        return "fw_b_apply"
    return None


def _csv_rows(folder, suffix):
    import csv
    import glob
    out = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    if not out:
        raise FileNotFoundError("no *%s under %s" % (suffix, folder))
    return out


def _field(row, *names):
    for nm in names:
        if nm in row and row[nm] != "":
            return row[nm]
    raise KeyError(names)


def _dispatches(folder):
    """Kernel trace: [(kernel, start_ns, end_ns)] in start order."""
    rows = _csv_rows(folder, "kernel_trace.csv")
    out = [(_kname(_field(r, "Kernel_Name", "Name")), int(_field(r, "Start_Timestamp")),
            int(_field(r, "End_Timestamp"))) for r in rows]
    return sorted(out, key=lambda x: x[1])


def _counter_totals(folder):
    """Counter run: {counter: {kernel: [value per dispatch]}}."""
    rows = _csv_rows(folder, "counter_collection.csv")
    per = {}
    for r in rows:
        c = _field(r, "Counter_Name")
        k = _kname(_field(r, "Kernel_Name", "Name"))
        d = _field(r, "Dispatch_Id", "Correlation_Id")
        per.setdefault(c, {}).setdefault(k, {}).setdefault(d, 0.0)
        per[c][k][d] += float(_field(r, "Counter_Value"))
    return {c: {k: list(v.values()) for k, v in ks.items()} for c, ks in per.items()}


def _calls_in(kernels):
    """Calls of the A update and the B argmin in a run, from one-per-call kernels."""
    def count(prefixes):
        for p in prefixes:
            n = sum(len(v) for k, v in kernels.items() if k.startswith(p))
            if n:
                return n
        return 0
    return {"fw_a_columns": count(("pad_rows_kernel", "fw_a_group_kernel")),
            "fw_b_argmin": count(("fw_b_reduce2_kernel",)),
            "fw_b_apply": count(("fw_b_apply_kernel",))}


def _copy_scale(folder, counter, nbytes):
    """Bytes per counted KiB / 1024: the factor that turns the counter into
    bytes for a copy of known size."""
    tot = _counter_totals(folder)[counter]
    cands = [v for k, v in tot.items() if "elementwise" in k or "Mul" in k]
    vals = max(cands, key=lambda v: np.mean(v))
    return nbytes / (float(np.median(vals)) * 1024.0)


def utilization(counters, by_k, calls):
    """Busy fractions of the main kernel of each call (the one with the most
    time), from the mean-per-dispatch counters, or {} without them."""
    need = ("GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
            "TD_TD_BUSY_sum", "TA_BUSY_avr", "TCC_HIT_sum", "TCC_MISS_sum")
    if any(c not in counters for c in need):
        return {}
    out = {}
    for c in ("fw_a_columns", "fw_b_argmin"):
        ks = [k for k in by_k if _call_of(k) == c and all(k in counters[x] for x in need)]
        if not ks:
            continue
        k = max(ks, key=lambda x: sum(by_k[x]))
        m = {x: float(np.mean(counters[x][k])) for x in need}
        cyc = m["GRBM_GUI_ACTIVE"] / 8.0
        if cyc <= 0:
            continue
        out[c] = {"kernel": k, "valu": m["SQ_INSTS_VALU"] * 4.0 / (1024.0 * cyc),
                  "lds": m["SQ_LDS_IDX_ACTIVE"] / (256.0 * cyc),
                  "lds_conflict_share": m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_LDS_IDX_ACTIVE"], 1.0),
                  "td": m["TD_TD_BUSY_sum"] / (256.0 * cyc), "ta": m["TA_BUSY_avr"] / cyc,
                  "l2_hit": m["TCC_HIT_sum"] / max(m["TCC_HIT_sum"] + m["TCC_MISS_sum"], 1.0)}
    return out


def limiter_from_profile(call, workload, sha):
    """The busiest unit of the call's main kernel in the committed counter
    record (None when absent or the sources changed)."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        rec = json.load(f)
    e = rec.get(call, {}).get(workload)
    if not e or e.get("source_sha") != sha or "utilization" not in e:
        return None
    u = e["utilization"]
    busy = {x: u[x] for x in ("valu", "lds", "td", "ta")}
    top = max(busy, key=busy.get)
    return {"unit": top, "busy": busy, "lds_conflict_share": u["lds_conflict_share"],
            "l2_hit": u["l2_hit"], "kernel": u["kernel"]}


def summarize_profile(args):
    """rocprofv3 folders -> markdown summary and the per-call traffic record."""
    name = args.config
    disp = _dispatches(args.trace)
    by_k = {}
    for k, t0, t1 in disp:
        by_k.setdefault(k, []).append((t1 - t0) / 1000.0)
    calls = _calls_in(by_k)
    lines = ["# rocprofv3 summary: %s, workload %s" % (
        ", ".join(sorted({c for c in map(_call_of, by_k) if c})), name), "",
        "Commands (each a separate run on one MI355X, from the repository root; `<out>` is a "
        "scratch folder):", ""]
    for cmd in args.command.split(";;"):
        if cmd.strip():
            lines.append("    " + cmd.strip())
    lines += ["", "## Kernel time (`--kernel-trace --stats`)", "",
              "Calls in the traced run: %s." % ", ".join("%s %d" % kv for kv in calls.items()), "",
              "| kernel | call | dispatches | per call | avg us | min us | max us |",
              "|---|---|---|---|---|---|---|"]
    per_call_us = {}
    for k in sorted(by_k, key=lambda k: -sum(by_k[k])):
        v = by_k[k]
        c = _call_of(k)
        m = len(v) / calls[c] if c and calls.get(c) else 0
        lines.append("| %s | %s | %d | %s | %.1f | %.1f | %.1f |" % (
            k, c or "-", len(v), ("%.0f" % m) if m else "-", np.mean(v), np.min(v), np.max(v)))
        if c:
            per_call_us[c] = per_call_us.get(c, 0.0) + sum(v) / max(calls[c], 1)
    # kernels dispatched several times per call: one row per pass
    passes = []
    for k, v in by_k.items():
        c = _call_of(k)
        if c and calls.get(c) and len(v) % calls[c] == 0 and len(v) // calls[c] > 1:
            m = len(v) // calls[c]
            for j in range(m):
                pv = v[j::m]
                passes.append("| %s | pass %d of %d | %.1f | %.1f | %.1f |" % (
                    k, j + 1, m, np.mean(pv), np.min(pv), np.max(pv)))
    if passes:
        lines += ["", "Kernels launched more than once per call, by pass (dispatch order within "
                  "the call):", "", "| kernel | pass | avg us | min us | max us |",
                  "|---|---|---|---|---|"] + passes
    lines += ["", "Sum of a call's kernel times, per call: " + ", ".join(
        "%s %.1f us" % kv for kv in sorted(per_call_us.items())) + "."]
    rec = None
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        nbytes = 1024 * 1024 * 1024
        fs = _copy_scale(args.copy_fetch, "FETCH_SIZE", nbytes)
        ws = _copy_scale(args.copy_write, "WRITE_SIZE", nbytes)
        fetch = _counter_totals(args.fetch)["FETCH_SIZE"]
        write = _counter_totals(args.write)["WRITE_SIZE"]
        cf, cw = _calls_in(fetch), _calls_in(write)
        lines += ["", "## Bytes beyond L2 (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)", "",
                  "The counters count the L2's requests to memory: HBM, and also reads the 256 MB "
                  "MALL serves (an upper bound on HBM bytes). A plain 1 GiB device copy "
                  "(`bench.py --copy-calibration 1024`) counts FETCH_SIZE and WRITE_SIZE such "
                  "that bytes = FETCH_SIZE x %.4f + WRITE_SIZE x %.4f (KiB); every figure "
                  "below is scaled by those factors." % (fs, ws), "",
                  "| kernel | call | FETCH_SIZE KiB | WRITE_SIZE KiB | MB per dispatch |",
                  "|---|---|---|---|---|"]
        tot = {}
        for k in sorted(set(fetch) | set(write)):
            c = _call_of(k)
            f = fetch.get(k, [0.0])
            wv = write.get(k, [0.0])
            mb = (np.mean(f) * fs + np.mean(wv) * ws) * 1024.0 / 1e6
            lines.append("| %s | %s | %.1f | %.1f | %.1f |" % (k, c or "-", np.mean(f),
                                                               np.mean(wv), mb))
            if c and cf.get(c) and cw.get(c):
                tot.setdefault(c, 0.0)
                tot[c] += (sum(f) * fs / cf[c] + sum(wv) * ws / cw[c]) * 1024.0
        lines += ["", "Bytes beyond L2 per call: " + ", ".join(
            "%s %.4g GB" % (c, b / 1e9) for c, b in sorted(tot.items())) + "."]
        rec = {}
        for c, b in tot.items():
            if c in CALL_SOURCES:
                rec[c] = {"source_sha": source_sha(*CALL_SOURCES[c]), "bytes_per_call": b,
                          "us_per_call_trace": per_call_us.get(c),
                          "kernels": sorted(k for k in fetch if _call_of(k) == c),
                          "fetch_scale": fs, "write_scale": ws}
    all_counters = {}
    for folder in args.counters:
        for c, ks in _counter_totals(folder).items():
            all_counters[c] = ks
    util = utilization(all_counters, by_k, calls)
    if util:
        lines += ["", "## Utilization of the main kernel of each call (from the counters below)", "",
                  "Cycles = GRBM_GUI_ACTIVE / 8 (one per XCD). VALU: SQ_INSTS_VALU x 4 cycles per "
                  "wave64 instruction over 1024 SIMDs; LDS: SQ_LDS_IDX_ACTIVE over 256 CUs (bank "
                  "conflict cycles are part of it); TD: TD_TD_BUSY_sum over 256 CUs; TA: "
                  "TA_BUSY_avr.", "",
                  "| call | kernel | VALU | LDS | LDS conflicts | TD | TA | L2 hit |",
                  "|---|---|---|---|---|---|---|---|"]
        for c, u in sorted(util.items()):
            lines.append("| %s | %s | %.0f%% | %.0f%% | %.0f%% | %.0f%% | %.0f%% | %.0f%% |" % (
                c, u["kernel"], 100 * u["valu"], 100 * u["lds"], 100 * u["lds_conflict_share"],
                100 * u["td"], 100 * u["ta"], 100 * u["l2_hit"]))
            if rec is not None and c in rec:
                rec[c]["utilization"] = u
    for folder in args.counters:
        tots = _counter_totals(folder)
        names = sorted(tots)
        lines += ["", "## Counters: %s (mean per dispatch)" % ", ".join(names), "",
                  "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
        ks = sorted({k for c in names for k in tots[c] if _call_of(k)})
        for k in ks:
            lines.append("| %s | " % k + " | ".join(
                "%.4g" % np.mean(tots[c][k]) if k in tots[c] else "-" for c in names) + " |")
    with open(args.summarize_profile, "w") as f:
        f.write("\n".join(lines) + "\n")
    if rec:
        allrec = {}
        if os.path.exists(TRAFFIC_JSON):
            with open(TRAFFIC_JSON) as f:
                allrec = json.load(f)
        for c, e in rec.items():
            allrec.setdefault(c, {})[name] = e
        with open(TRAFFIC_JSON, "w") as f:
            json.dump(allrec, f, indent=1, sort_keys=True)
    print("wrote %s" % args.summarize_profile)


def _median(xs):
    return float(np.median(np.asarray(xs, np.float64)))


class HotPath:
    """Device operands, outputs and workspaces of one workload, allocated
    once; call() runs one step of the hot path on `stream`."""

    def __init__(self, saa, W, w, prune=None, cap_b_extra=64):
        import torch
        self.saa, self.w, self.prune = saa, w, prune
        dev = torch.device("cuda:0")
        D = saa.DeviceCSR.from_scipy
        self.t1, self.k2b, self.ap, self.aat, self.k2at, self.bm = (
            D(w.t1), D(w.k2b), D(w.a_prev_t), D(w.aat), D(w.k2at), D(w.b))
        n, k, T, cap = w.n, w.k, w.T, w.cap
        cap_b = int(np.diff(w.b.tocsc().indptr).max()) + cap_b_extra
        bi, bv, bc = W.bt_padded(w.b, cap_b)
        self.bt_idx = torch.from_numpy(bi.astype(np.int32)).to(dev)
        self.bt_val = torch.from_numpy(bv).to(dev)
        self.bt_cnt = torch.from_numpy(bc.astype(np.int32)).to(dev)
        self.atom_idx = torch.empty((n, cap), dtype=torch.int32, device=dev)
        self.atom_val = torch.empty((n, cap), dtype=torch.float32, device=dev)
        self.atom_cnt = torch.empty(n, dtype=torch.int32, device=dev)
        ws_a = saa.seacells_fw_a_columns_workspace(n, k, T, cap, w.t1.nnz)
        self.ws_a = torch.empty(max(ws_a, 1), dtype=torch.uint8, device=dev)
        self.out_val = torch.empty(k, dtype=torch.float32, device=dev)
        self.out_idx = torch.empty(k, dtype=torch.int32, device=dev)
        self.gap = torch.empty(1, dtype=torch.float32, device=dev)
        self.ws_b = torch.empty(saa.seacells_fw_b_argmin_workspace(n, k, w.aat.nnz),
                                dtype=torch.uint8, device=dev)
        self.st_a, self.st_b, self.st_p = (saa.new_status(dev) for _ in range(3))

    def a_update(self, stream, trace=None):
        w = self.w
        kw = dict(atom_idx=self.atom_idx, atom_val=self.atom_val, atom_cnt=self.atom_cnt,
                  trace=trace, workspace=self.ws_a, status=self.st_a, stream=stream)
        if self.prune is None:
            self.saa.seacells_fw_a_columns(self.t1, self.k2b, self.ap, w.n, w.k, w.T, w.cap, **kw)
        else:
            self.saa.seacells_fw_a_columns_pruned(self.t1, self.k2b, self.ap, w.n, w.k, w.T,
                                                  w.cap, self.prune, **kw)

    def b_argmin(self, stream):
        w = self.w
        self.saa.seacells_fw_b_argmin(self.k2b, self.aat, self.k2at, self.bm, w.n, w.k,
                                      out_val=self.out_val, out_idx=self.out_idx, gap=self.gap,
                                      workspace=self.ws_b, status=self.st_b, stream=stream)

    def b_apply(self, stream, t):
        # the B loop's step index continues after the workload's s_B prior steps
        gamma, _ = self.saa.seacells_fw_step_size(self.w.cfg.s_b + 1 + t)
        self.saa.seacells_fw_b_apply(self.bt_idx, self.bt_val, self.bt_cnt, self.w.n,
                                     self.out_idx, gamma, status=self.st_p, stream=stream)

    def raise_on_status(self):
        for st in (self.st_a, self.st_b, self.st_p):
            self.saa.raise_on_status(st)

    def traced_bytes(self):
        """One traced A update (outside any timing) for the byte models: the
        trace is deterministic, so the timed calls take the same picks."""
        import torch
        w = self.w
        trace = torch.empty((w.n, w.T), dtype=torch.int32, device="cuda")
        self.a_update(torch.cuda.current_stream(), trace=trace)
        torch.cuda.synchronize()
        self.saa.raise_on_status(self.st_a)
        tr, cnt = trace.cpu().numpy(), self.atom_cnt.cpu().numpy()
        return {"fw_a_columns": algorithmic_bytes_a(w, tr, cnt),
                "fw_b_argmin": algorithmic_bytes_b(w)}, \
               {"fw_a_columns": compulsory_bytes_a(w, cnt), "fw_b_argmin": compulsory_bytes_b(w)}


def call_roofline(call, ms, alg, comp, traffic):
    """Rates and fractions of HBM peak for one call: algorithmic bytes (the
    headline), bytes the counters saw beyond L2, and compulsory bytes."""
    sec = ms * 1e-3
    r = {"ms": ms, "achieved": alg / sec / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
         "frac": alg / sec / 1e9 / PEAK_HBM_GBPS, "bytes_per_launch": alg,
         "compulsory_bytes": comp, "frac_compulsory": comp / sec / 1e9 / PEAK_HBM_GBPS,
         "traffic": traffic}
    r["beyond_l2_gbps"] = None if traffic is None else traffic / sec / 1e9
    r["frac_beyond_l2"] = None if traffic is None else traffic / sec / 1e9 / PEAK_HBM_GBPS
    return r


def cpu_table_row(name, w, threads):
    """The oracle's t_A and t_B on the same workload: every cell and row up to
    n = 100k, else a sample scaled to n (stated)."""
    import oracle
    import scipy.sparse as sp
    out = {"threads": threads}
    rng = np.random.default_rng(0)
    if w.n <= 100_000:
        t0 = time.time()
        oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, n_threads=threads)
        out["t_a_s"] = time.time() - t0
        t0 = time.time()
        oracle.fw_b_argmin(w.k2b, w.aat, w.k2at, w.b, w.n, w.k, n_threads=threads)
        out["t_b_s"] = time.time() - t0
        out["sample"] = "all cells and rows"
    else:
        m = 2000 if w.n <= 500_000 else 400
        cells = rng.choice(w.n, size=m, replace=False)
        t0 = time.time()
        oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells,
                            n_threads=threads)
        out["t_a_s"] = (time.time() - t0) * w.n / m
        r = min(w.n, 200_000)
        rows = lambda x: sp.csr_matrix(x[:r])  # noqa: E731
        t0 = time.time()
        oracle.fw_b_argmin(rows(w.k2b), w.aat, rows(w.k2at), rows(w.b), r, w.k,
                           n_threads=threads)
        out["t_b_s"] = (time.time() - t0) * w.n / r
        out["sample"] = "A on %d random cells, B on the first %d rows, scaled to n" % (m, r)
    out["cells_per_s"] = w.n / (out["t_a_s"] + out["t_b_s"])
    return out


def run_table(args):
    """The A update and the B argmin alone on each workload, with the
    oracle's times beside them; one JSON line per workload."""
    import torch
    import sparse_archetypal_analysis_amd as saa
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    for name in args.table_configs.split(","):
        w = W.make(name, log=lambda m: print(m, file=sys.stderr, flush=True))
        hp = HotPath(saa, W, w)
        alg, comp = hp.traced_bytes()
        reps = 20 if w.n <= 100_000 else 5
        res = {}
        for call, fn in (("fw_a_columns", hp.a_update), ("fw_b_argmin", hp.b_argmin)):
            for _ in range(3):
                fn(stream)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record(stream)
                fn(stream)
                e1.record(stream)
            torch.cuda.synchronize()
            ms = [e0.elapsed_time(e1) for e0, e1 in ev]
            sha = source_sha(*CALL_SOURCES[call])
            res[call] = call_roofline(call, _median(ms), alg[call], comp[call],
                                      traffic_from_profile(call, name, sha))
            res[call]["reps"] = reps
        hp.raise_on_status()
        rec = {"workload": "%s: %s" % (name, W.DESCRIPTIONS.get(name, "")), "n": w.n, "k": w.k,
               "nnz": w.meta.get("nnz"), "calls": res,
               "cells_per_s": w.n / ((res["fw_a_columns"]["ms"] + res["fw_b_argmin"]["ms"]) * 1e-3)}
        if not args.no_cpu_baseline:
            rec["oracle"] = cpu_table_row(name, w, threads)
            if w.n <= 20_000:
                rec["oracle_1_thread"] = cpu_table_row(name, w, 1)
        print(json.dumps(rec), flush=True)
        del hp
        torch.cuda.empty_cache()


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
    ap.add_argument("--table", action="store_true",
                    help="time the A update and the B argmin on every workload, with the oracle")
    ap.add_argument("--table-configs", default="c1,c2,c3,c4,c5")
    ap.add_argument("--summarize-profile", metavar="OUT_MD", default=None,
                    help="write a rocprofv3 summary (CPU only; see the module doc)")
    for opt in ("--trace", "--fetch", "--write", "--copy-fetch", "--copy-write"):
        ap.add_argument(opt, default=None)
    ap.add_argument("--counters", nargs="*", default=[])
    ap.add_argument("--command", default="", help="the profiled command, for the summary")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path's multi-GPU sharding is a design, "
              "not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.table:
        run_table(args)
        return

    import torch
    import sparse_archetypal_analysis_amd as saa
    import workloads as W

    t_gen = time.time()
    w = W.make(args.config, log=lambda m: print(m, file=sys.stderr, flush=True))
    t_gen = time.time() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n, k, T, cap = w.n, w.k, w.T, w.cap
    steps, warm = args.steps, args.warmup
    prune = args.prune
    hp = HotPath(saa, W, w, prune=prune, cap_b_extra=steps + warm + 2)
    stream = torch.cuda.current_stream()
    alg, comp = hp.traced_bytes()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(t, marks=None):
        if marks:
            marks[0].record(stream)
        hp.a_update(stream)
        if marks:
            marks[1].record(stream)
        hp.b_argmin(stream)
        if marks:
            marks[2].record(stream)
        hp.b_apply(stream, t)
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
    hp.raise_on_status()

    per = {c: [e[j].elapsed_time(e[j + 1]) for e in ev]
           for j, c in enumerate(("fw_a_columns", "fw_b_argmin", "fw_b_apply"))}
    ms_step = wall * 1000.0 / steps
    calls = {}
    for c in ("fw_a_columns", "fw_b_argmin"):
        sha = source_sha(*CALL_SOURCES[c])
        traffic = None if prune is not None else traffic_from_profile(c, args.config, sha)
        calls[c] = call_roofline(c, float(np.mean(per[c])), alg[c], comp[c], traffic)
        calls[c]["ms_median"] = _median(per[c])
    dominant = max(calls, key=lambda c: calls[c]["ms"])
    d = calls[dominant]
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
                   "b_init": w.meta.get("b_init"), "prune_threshold": prune},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": d["achieved"],
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": d["frac"],
                     "traffic": d["traffic"], "bytes_per_launch": d["bytes_per_launch"],
                     "frac_beyond_l2": d["frac_beyond_l2"],
                     "compulsory_bytes": d["compulsory_bytes"],
                     "frac_compulsory": d["frac_compulsory"],
                     "limiter": None if prune is not None else limiter_from_profile(
                         dominant, args.config, source_sha(*CALL_SOURCES[dominant])),
                     "note": "achieved = algorithmic bytes (every sparse entry the method "
                             "touches, re-reads counted) / mean call time, so frac > 1 means "
                             "re-reads served on chip; frac_beyond_l2 = rocprofv3 FETCH_SIZE + "
                             "WRITE_SIZE per call (HBM and MALL) / time / peak; frac_compulsory "
                             "= every input read once / time / peak; limiter = the busiest unit "
                             "of the call's main kernel in the committed counters"},
        "calls": calls,
        "kernels_ms": {c: float(np.mean(v)) for c, v in per.items()},
        "kernels_ms_median": {c: _median(v) for c, v in per.items()},
        "a_cells_per_s": n / (calls["fw_a_columns"]["ms"] * 1e-3),
        "b_cells_per_s": n / (calls["fw_b_argmin"]["ms"] * 1e-3),
        "generation_s": t_gen,
        "device": torch.cuda.get_device_name(dev),
    }
    if not args.no_operands:
        rec["operands"] = time_operands(saa, W, w, stream)
    if args.b_loop_steps > 0:
        rec["b_loop"] = time_b_loop(saa, W, w, args.b_loop_steps, calls["fw_b_argmin"]["ms"],
                                    stream)
    if args.iteration_b_steps > 0:
        rec["iteration"] = time_iteration(saa, W, w, args.iteration_b_steps, stream)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
