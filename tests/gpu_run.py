"""Run the HIP entry points on host-side workloads (GPU test helper)."""
import numpy as np
import torch

import sparse_archetypal_analysis_amd as saa


def dev(m):
    return saa.DeviceCSR.from_scipy(m)


def host(d, rows=None):
    """A DeviceCSR back as a scipy CSR (f32 values, int64 indices); with
    ``rows``, only those rows (copied slice by slice)."""
    import scipy.sparse as sp
    ptr = d.row_ptr.cpu().numpy().astype(np.int64)
    if rows is None:
        idx = d.col_idx.cpu().numpy().astype(np.int64)
        val = d.val.cpu().numpy()
        out = sp.csr_matrix((val, idx, ptr), shape=d.shape)
    else:
        rows = np.asarray(rows, np.int64)
        lo, hi = ptr[rows], ptr[rows + 1]
        idx = [d.col_idx[a:b].cpu().numpy().astype(np.int64) for a, b in zip(lo, hi)]
        val = [d.val[a:b].cpu().numpy() for a, b in zip(lo, hi)]
        p = np.zeros(rows.size + 1, np.int64)
        np.cumsum(hi - lo, out=p[1:])
        out = sp.csr_matrix((np.concatenate(val) if val else np.zeros(0, np.float32),
                             np.concatenate(idx) if idx else np.zeros(0, np.int64), p),
                            shape=(rows.size, d.shape[1]))
    out.has_sorted_indices = True
    return out


def run_a(w, T=None, cap=None, gamma=None, trace=True, ops=None, prune=None, gap_out=None):
    """A update on the GPU; the five outputs as numpy. ``gap_out`` (a list)
    receives the per-cell Frank-Wolfe gap when given."""
    T = w.T if T is None else T
    cap = w.cap if cap is None else cap
    g = None if gamma is None else torch.tensor(np.asarray(gamma, np.float32), device="cuda")
    t1, k2b, ap = ops if ops is not None else (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    fg = None
    if gap_out is not None:
        fg = torch.full((w.n,), float("nan"), dtype=torch.float32, device="cuda")
    if prune is None:
        ai, av, ac, tr, st = saa.seacells_fw_a_columns(t1, k2b, ap, w.n, w.k, T, cap, gamma=g,
                                                       trace=trace, fw_gap=fg)
    else:
        ai, av, ac, tr, st = saa.seacells_fw_a_columns_pruned(t1, k2b, ap, w.n, w.k, T, cap,
                                                              prune, gamma=g, trace=trace,
                                                              fw_gap=fg)
    torch.cuda.synchronize()
    if gap_out is not None:
        gap_out.append(fg.cpu().numpy())
    return (ai.cpu().numpy(), av.cpu().numpy(), ac.cpu().numpy(),
            tr.cpu().numpy() if tr is not None else None, saa.status_flags(st))


def run_b(w, with_b=True, ops=None, gap_out=None):
    """B argmin on the GPU: (min values, rows, gap, flags). ``gap_out`` (a
    list) receives the full Frank-Wolfe gap when given."""
    k2b, aat, k2at, b = ops if ops is not None else (dev(w.k2b), dev(w.aat), dev(w.k2at),
                                                     dev(w.b) if with_b else None)
    fg = None
    if gap_out is not None:
        fg = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    v, i, g, st = saa.seacells_fw_b_argmin(k2b, aat, k2at, b, w.n, w.k, fw_gap=fg)
    torch.cuda.synchronize()
    if gap_out is not None:
        gap_out.append(float(fg.cpu().numpy()[0]))
    return v.cpu().numpy(), i.cpu().numpy(), float(g.cpu().numpy()[0]), saa.status_flags(st)


def run_b_dense(k2b, t1, t2, b):
    """B argmin on dense page-style fixtures (converted to CSR)."""
    import workloads as W
    n, k = k2b.shape
    cfg = W.Config("fixture", n, 0, 0, 0, k, 0, 0)
    w = W.Workload(cfg, 0, t1=W.dense_to_csr(t1), k2b=W.dense_to_csr(k2b),
                   a_prev_t=W.dense_to_csr(np.zeros((n, k))), aat=W.dense_to_csr(t1),
                   k2at=W.dense_to_csr(t2), b=W.dense_to_csr(b), init_cells=np.zeros(0, np.int64))
    return w, run_b(w)


def run_a_as_timed(w, ops=None, calls=3):
    """The A update exactly as the benchmark times it: outputs, workspace and
    status allocated once, no trace, no gap, the call repeated on them.
    Returns the last call's (atom_idx, atom_val, atom_cnt, flags)."""
    n, k, T, cap = w.n, w.k, w.T, w.cap
    t1, k2b, ap = ops if ops is not None else (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    ai = torch.empty((n, cap), dtype=torch.int32, device="cuda")
    av = torch.empty((n, cap), dtype=torch.float32, device="cuda")
    ac = torch.empty(n, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(saa.seacells_fw_a_columns_workspace(n, k, T, cap, t1.nnz), 1),
                     dtype=torch.uint8, device="cuda")
    st = saa.new_status()
    for _ in range(calls):
        saa.seacells_fw_a_columns(t1, k2b, ap, n, k, T, cap, atom_idx=ai, atom_val=av,
                                  atom_cnt=ac, workspace=ws, status=st)
    torch.cuda.synchronize()
    return ai.cpu().numpy(), av.cpu().numpy(), ac.cpu().numpy(), saa.status_flags(st)


def run_b_as_timed(w, ops=None, calls=3):
    """The B argmin exactly as the benchmark times it: B given for the gap,
    no full gap, outputs and workspace allocated once, the call repeated.
    Returns (out_val, out_idx, gap, flags) of the last call."""
    k2b, aat, k2at, b = ops if ops is not None else (dev(w.k2b), dev(w.aat), dev(w.k2at),
                                                     dev(w.b))
    v = torch.empty(w.k, dtype=torch.float32, device="cuda")
    i = torch.empty(w.k, dtype=torch.int32, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(saa.seacells_fw_b_argmin_workspace(w.n, w.k, aat.nnz), dtype=torch.uint8,
                     device="cuda")
    st = saa.new_status()
    for _ in range(calls):
        saa.seacells_fw_b_argmin(k2b, aat, k2at, b, w.n, w.k, out_val=v, out_idx=i, gap=g,
                                 workspace=ws, status=st)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy(), float(g.cpu().numpy()[0]), saa.status_flags(st)


def assert_same_atoms(traced, timed):
    """The timed call's atoms equal the traced call's bit for bit."""
    ai0, av0, ac0 = traced[0], traced[1], traced[2]
    ai1, av1, ac1 = timed[0], timed[1], timed[2]
    np.testing.assert_array_equal(ac0, ac1)
    mask = np.arange(ai0.shape[1])[None, :] < ac0[:, None]
    np.testing.assert_array_equal(ai0[mask], ai1[mask])
    np.testing.assert_array_equal(av0[mask].view(np.uint32), av1[mask].view(np.uint32))
