"""B-gradient argmin and B step on the GPU against the f64 oracle."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_archetypal_analysis_amd as saa
import workloads as W
from tests import parity
from tests.gpu_run import dev, run_b, run_b_dense

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_fixtures.json")


def page_problem(n, k):
    fx = json.load(open(GOLDEN))["fixture"]["operands"]
    return (W.page_fixture(n * k, *fx["k2b"]).reshape(n, k),
            W.page_fixture(k * k, *fx["t1"]).reshape(k, k),
            W.page_fixture(n * k, *fx["t2"]).reshape(n, k),
            W.page_fixture(n * k, *fx["b"]).reshape(n, k))


@pytest.mark.parametrize("n,k", [(40, 7), (257, 33), (1000, 130), (3000, 300), (300, 1100)])
def test_page_fixtures(n, k):
    # signed values and a non-symmetric t1: the row-scatter form is still the
    # page's G[i, c] = sum_m K2B[i, m] t1[m, c] - t2[i, c]
    w, (v, i, g, flags) = run_b_dense(*page_problem(n, k))
    assert flags == []
    rep = parity.check_b(w, v, i, g)
    assert rep.near_tie * 50 <= k


def test_page_empty_rows_exact():
    cfg = json.load(open(GOLDEN))["empty_rows"]
    k2b, t1, t2, b = page_problem(cfg["n"], cfg["k"])
    k2b[::cfg["blank_every"]] = 0.0
    w, (v, i, g, flags) = run_b_dense(k2b, t1, t2, b)
    assert flags == []
    res = oracle.fw_b_argmin(w.k2b, w.aat, w.k2at, w.b, w.n, w.k)
    np.testing.assert_array_equal(i, res.row)
    parity.check_b(w, v, i, g, res=res)


def test_page_tie_breaks_on_lowest_row():
    cfg = json.load(open(GOLDEN))["tie_break"]
    n, k = cfg["n"], cfg["k"]
    k2b = np.tile(-1.0 - np.arange(k, dtype=np.float32), (n, 1))
    w, (v, i, g, flags) = run_b_dense(k2b, np.eye(k, dtype=np.float32),
                                      np.zeros((n, k), np.float32), np.zeros((n, k), np.float32))
    assert flags == []
    np.testing.assert_array_equal(i, np.zeros(k))
    np.testing.assert_array_equal(v, -1.0 - np.arange(k))


def test_identity_kernel_worked_example():
    n, k = 4, 2
    B = np.zeros((n, k), np.float32)
    B[0, 0] = B[1, 1] = 1.0
    aat = np.ones((k, k), np.float32)
    k2at = np.full((n, k), 0.5, np.float32)
    w, (v, i, g, flags) = run_b_dense(B, aat, k2at, B)
    assert flags == []
    np.testing.assert_array_equal(i, [2, 2])
    np.testing.assert_array_equal(v, [-0.5, -0.5])
    assert g == 1.0


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_configs_all_columns(name):
    w = W.make(name)
    v, i, g, flags = run_b(w)
    assert flags == []
    rep = parity.check_b(w, v, i, g)
    print("\n%s: %s" % (name, rep))


@pytest.mark.parametrize("n,k", [(3000, 2100), (500, 5000), (2, 9000)])
def test_column_slices(n, k):
    w = W.random_workload(n, k, aat_per_row=30, k2b_per_row=12, k2at_per_row=10, seed=n + k)
    v, i, g, flags = run_b(w)
    assert flags == []
    parity.check_b(w, v, i, g)


def test_one_slice_long_aat_runs():
    # k <= 2048 (one slice, padded AAt copy): symmetric AAt rows of ~200 to
    # ~680 entries, so a gathered run spans 4 to 11 chunks (the first three are
    # loaded together with those of the neighbouring runs, the rest one by one)
    w = W.random_workload(2000, 1500, aat_per_row=250, k2b_per_row=20, k2at_per_row=15, seed=77)
    chunks = (np.diff(w.aat.indptr) + 63) // 64
    assert chunks.min() >= 4 and chunks.max() >= 10
    v, i, g, flags = run_b(w)
    assert flags == []
    parity.check_b(w, v, i, g)


def test_single_row_single_column_and_no_b():
    w = W.random_workload(1, 1, seed=2)
    v, i, g, flags = run_b(w)
    assert flags == [] and i.tolist() == [0]
    parity.check_b(w, v, i, g)
    w = W.make("c1")
    v, i, g, flags = run_b(w, with_b=False)
    assert flags == [] and g == 0.0
    parity.check_b(w, v, i, None, b=False)


def test_deterministic_bitwise():
    w = W.make("c2")
    ops = (dev(w.k2b), dev(w.aat), dev(w.k2at), dev(w.b))
    r1, r2 = run_b(w, ops=ops), run_b(w, ops=ops)
    for a, b in zip(r1[:3], r2[:3]):
        np.testing.assert_array_equal(a, b)


def _apply(bt_idx, bt_val, bt_cnt, n, arg, gam):
    ti = torch.from_numpy(bt_idx.astype(np.int32)).cuda()
    tv = torch.from_numpy(bt_val.astype(np.float32)).cuda()
    tc = torch.from_numpy(bt_cnt.astype(np.int32)).cuda()
    ta = torch.from_numpy(np.asarray(arg, np.int32)).cuda()
    _, _, _, st = saa.seacells_fw_b_apply(ti, tv, tc, n, ta, gam)
    torch.cuda.synchronize()
    return ti.cpu().numpy(), tv.cpu().numpy(), tc.cpu().numpy(), saa.status_flags(st)


def test_b_step_after_argmin():
    w = W.make("c2")
    v, i, g, flags = run_b(w)
    cap_b = int(np.diff(w.b.tocsc().indptr).max()) + 2
    bi, bv, bc = W.bt_padded(w.b, cap_b)
    gam = 2.0 / 5.0
    gi, gv, gc, fl = _apply(bi, bv, bc, w.n, i, gam)
    assert fl == []
    oi, ov, oc = oracle.fw_b_apply(bi, bv, bc, i, gam)
    np.testing.assert_array_equal(gc, oc)
    for c in range(w.k):
        np.testing.assert_array_equal(gi[c, :gc[c]], oi[c, :oc[c]])
    err = max(float(np.max(np.abs(gv[c, :gc[c]] - ov[c, :oc[c]]))) for c in range(w.k))
    assert err <= parity.B_ABS


def test_b_step_overflow_and_bad_index_flags():
    k, cap_b, n = 5, 3, 50
    bi = np.tile(np.array([1, 4, 9], np.uint32), (k, 1))
    bv = np.full((k, cap_b), 1.0 / 3, np.float32)
    bc = np.full(k, 3, np.uint32)
    arg = np.array([4, 4, 4, 4, 4])          # present: fine
    *_, fl = _apply(bi, bv, bc, n, arg, 0.5)
    assert fl == []
    arg = np.array([4, 7, 4, 4, 4])          # column 1 would need a 4th slot
    gi, gv, gc, fl = _apply(bi, bv, bc, n, arg, 0.5)
    assert fl == ["B_CAP_OVERFLOW"] and gc[1] == 3
    np.testing.assert_array_equal(gv[1], bv[1])         # row left unchanged
    arg = np.array([4, 4, 4, 4, 50])         # row index out of range
    *_, fl = _apply(bi, bv, bc, n, arg, 0.5)
    assert fl == ["BAD_INDEX"]


def test_nonfinite_minimum_raises_flag():
    import dataclasses
    w = W.random_workload(300, 40, seed=73)
    # K2At[i, c] = +inf makes G[i, c] = -inf: a non-finite column minimum
    k2at = w.k2at.toarray()
    k2at[17, 5] = np.inf
    v, i, g, flags = run_b(dataclasses.replace(w, k2at=W.dense_to_csr(k2at)))
    assert flags == ["NONFINITE"]
    assert int(i[5]) == 17 and np.isneginf(v[5])
    # a column that is NaN at every row: no row range sees a finite value
    k2at = w.k2at.toarray()
    k2at[:, 9] = np.nan
    v, i, g, flags = run_b(dataclasses.replace(w, k2at=W.dense_to_csr(k2at)))
    assert flags == ["NONFINITE"]
    # the other columns are those of the clean run
    v0, i0, _, f0 = run_b(w)
    assert f0 == []
    cols = np.arange(w.k) != 9
    np.testing.assert_array_equal(i[cols], i0[cols])


def test_large_k_many_slices():
    # k = 300,000 needs 296 column slices of 1016 columns (the plan has no
    # slice ceiling); a few hundred rows keep the oracle quick
    import scipy.sparse as sp
    rng = np.random.default_rng(79)
    n, k = 200, 300_000

    def rand(rows, cols, per_row):
        nnz = rows * per_row
        r = np.repeat(np.arange(rows), per_row)
        c = rng.integers(0, cols, size=nnz)
        m = sp.csr_matrix((rng.uniform(0.05, 1.0, size=nnz), (r, c)), shape=(rows, cols))
        m.sum_duplicates()
        return m

    a = rand(k, k, 3)
    cfg = W.Config("large_k", n, 0, 0, 0, k, 0, 0)
    w = W.Workload(cfg, 0, t1=W._f32(a, symmetric=True), k2b=W._f32(rand(n, k, 40)),
                   a_prev_t=W._f32(rand(n, k, 1)), aat=W._f32(a, symmetric=True),
                   k2at=W._f32(rand(n, k, 30)), b=W._f32(rand(n, k, 2)),
                   init_cells=np.zeros(0, np.int64))
    lay = saa.seacells_debug_b_layout(n, k, w.aat.nnz)
    assert lay["n_slices"] > 128 and lay["slice_w"] <= 2048
    v, i, g, flags = run_b(w)
    assert flags == []
    rep = parity.check_b(w, v, i, g)
    print("\nk=300000: %s" % (rep,))


def test_sliced_copy_flags_a_repeated_aat_column():
    # the narrow-slice copy ranks each run's entries by accumulator position;
    # a column that appears twice in an AAt row (its indices must be
    # strictly ascending) is reported instead of being dropped silently
    w = W.random_workload(300, 5000, aat_per_row=30, k2b_per_row=12, k2at_per_row=10,
                          b_per_col=3, seed=62)
    assert saa.seacells_debug_b_layout(w.n, w.k, w.aat.nnz)["n_slices"] > 1
    ops = (dev(w.k2b), dev(w.aat), dev(w.k2at), dev(w.b))
    *_, flags = run_b(w, ops=ops)
    assert flags == []
    lo = int(w.aat.indptr[7])
    assert int(w.aat.indptr[8]) - lo >= 2
    ops[1].col_idx[lo + 1] = ops[1].col_idx[lo]
    *_, flags = run_b(w, ops=ops)
    assert flags == ["BAD_INDEX"]


@pytest.mark.parametrize("k", [3000, 9000])
def test_sliced_long_k2b_rows_empty_and_long_aat_rows(k):
    # K2B rows of ~250 entries put several hundred chunks of every slice in a
    # row (several staging windows, chunks carried from one batch to the
    # next); every 11th AAt row and column is empty; three AAt rows of 1500
    # entries give runs of many chunks; every 7th K2B row is empty. k = 3000
    # takes 4 slices, k = 9000 16 (dealt to the XCDs by work).
    import dataclasses
    import scipy.sparse as sp
    w = W.random_workload(300, k, k2b_per_row=250, aat_per_row=120, k2at_per_row=40,
                          b_per_col=3, seed=83 + k, empty_k2b_every=7)
    rng = np.random.default_rng(k)
    coo = w.aat.tocoo()
    keep = (coo.row % 11 != 0) & (coo.col % 11 != 0)
    rows, cols = [coo.row[keep]], [coo.col[keep]]
    vals = [coo.data[keep].astype(np.float64)]
    for m in (5, 1234, k - 1):
        c = rng.choice(k, size=1500, replace=False)
        c = c[(c % 11 != 0) & (c != m)]
        v = rng.uniform(0.05, 1.0, size=c.size)
        rows += [np.full(c.size, m), c]
        cols += [c, np.full(c.size, m)]
        vals += [v, v]
    a = sp.csr_matrix((np.concatenate(vals), (np.concatenate(rows), np.concatenate(cols))),
                      shape=(k, k))
    a.sum_duplicates()
    w = dataclasses.replace(w, aat=W._f32(a, symmetric=True))
    lay = saa.seacells_debug_b_layout(w.n, k, w.aat.nnz)
    assert lay["n_slices"] == (4 if k == 3000 else 16)
    assert np.diff(w.aat.indptr)[::11].max() == 0 and np.diff(w.aat.indptr).max() >= 1000
    v, i, g, flags = run_b(w)
    assert flags == []
    rep = parity.check_b(w, v, i, g)
    print("\nk=%d: %s" % (k, rep))
