"""A update on the GPU against the f64 oracle (trace replay)."""
import numpy as np
import pytest

import workloads as W
from tests import parity
from tests.gpu_run import assert_same_atoms, dev, run_a, run_a_as_timed

pytestmark = pytest.mark.gpu


def assert_same_result(r0, r1):
    """Bitwise equality of trace, counts and the valid atom slots."""
    ai0, av0, ac0, tr0, _ = r0
    ai1, av1, ac1, tr1, _ = r1
    np.testing.assert_array_equal(tr0, tr1)
    np.testing.assert_array_equal(ac0, ac1)
    mask = np.arange(ai0.shape[1])[None, :] < ac0[:, None]
    np.testing.assert_array_equal(ai0[mask], ai1[mask])
    np.testing.assert_array_equal(av0[mask].view(np.uint32), av1[mask].view(np.uint32))


def identity_workload():
    n, k = 4, 2
    B = np.zeros((n, k), np.float32)
    B[0, 0] = B[1, 1] = 1.0
    cfg = W.Config("identity", n, 0, 0, 0, k, 2, 0, T=50)
    return W.Workload(cfg, 0, t1=W.dense_to_csr(np.eye(2)), k2b=W.dense_to_csr(B),
                      a_prev_t=W.dense_to_csr(np.full((n, k), 0.5)), aat=W.dense_to_csr(np.eye(2)),
                      k2at=W.dense_to_csr(B), b=W.dense_to_csr(B), init_cells=np.zeros(0, np.int64))


def test_identity_kernel_worked_example_exact_ties():
    w = identity_workload()
    ai, av, ac, tr, flags = run_a(w)
    assert flags == []
    T = 50
    # exact ties in f32 as in f64: the lowest index must win, bit for bit
    assert tr[0].tolist() == [0] * T
    assert tr[1].tolist() == [1, 0] + [1] * (T - 2)
    assert tr[2].tolist() == [t % 2 for t in range(T)]
    assert tr[3].tolist() == [t % 2 for t in range(T)]
    dense = parity.dense_atoms(ai, av, ac, 2)
    want = np.array([[1, 0], [4 / 2550, 1 - 4 / 2550], [25 / 51, 26 / 51], [25 / 51, 26 / 51]])
    np.testing.assert_allclose(dense, want, rtol=0, atol=parity.A_ABS)
    assert ac.tolist() == [2, 2, 2, 2]            # the two seeds, no appends


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_config_all_cells(name):
    w = W.make(name)
    ai, av, ac, tr, flags = run_a(w)
    assert flags == []
    rep = parity.check_a(w, tr, ai, av, ac, np.arange(w.n))
    print("\n%s: %s" % (name, rep))
    assert rep.near_tie <= 1e-3 * rep.steps


def test_c3_full_size_all_cells():
    # every one of the 100,000 cells replayed by the oracle (about 12 s of
    # the f64 oracle on 16 host cores)
    w = W.make("c3")
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    gaps = []
    ai, av, ac, tr, flags = run_a(w, ops=ops, gap_out=gaps)
    assert flags == []
    cells = np.arange(w.n)
    rep = parity.check_a(w, tr, ai, av, ac, cells)
    print("\nc3 all cells: %s" % (rep,))
    assert rep.near_tie <= 1e-3 * rep.steps
    # the call the benchmark times (no trace, no gap, outputs and workspace
    # reused over repeated calls) gives the same atoms bit for bit
    timed = run_a_as_timed(w, ops=ops)
    assert timed[3] == []
    assert_same_atoms((ai, av, ac), timed)
    # properties that hold for every cell at any size
    assert np.all(ac >= np.diff(w.a_prev_t.indptr)) and np.all(ac <= w.cap)
    assert np.all((tr >= 0) & (tr < w.k))
    dense_sum = np.zeros(w.n)
    for s in range(ai.shape[1]):
        dense_sum += np.where(s < ac, av[:, s], 0.0)
    np.testing.assert_allclose(dense_sum, 1.0, atol=1e-5)


def test_ragged_signed_operands_dense_path():
    w = W.random_workload(1237, 333, t1_per_row=12, k2b_per_row=9, s_a=7, seed=5, signed=True)
    ai, av, ac, tr, flags = run_a(w)
    assert flags == []
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n))


@pytest.mark.parametrize("support", ["0", "default"])
def test_large_k_state_in_workspace(support, a_options):
    # k * 4 bytes exceeds the 160 KB LDS of a compute unit: the dense state
    # lives in workspace (support "0"); by default the compact state takes
    # the cells, with fewer waves per CU
    import sparse_archetypal_analysis_amd as saa
    if support == "0":
        a_options.set(support=0)
    w = W.random_workload(37, 45_000, t1_per_row=6, k2b_per_row=20, s_a=5, seed=7, T=30)
    assert saa.seacells_fw_a_columns_workspace(w.n, w.k, 30, w.cap, w.t1.nnz) > 0
    ai, av, ac, tr, flags = run_a(w, T=30)
    assert flags == []
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), T=30)


def test_empty_rows_and_columns():
    # empty K2B rows (g = t1 . a), empty A_prev columns (g = -t2), and both
    w = W.random_workload(300, 40, s_a=3, seed=9, empty_k2b_every=3, empty_ap_every=4)
    ai, av, ac, tr, flags = run_a(w)
    assert flags == []
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n))
    both = [j for j in range(w.n) if j % 12 == 0]
    # g is identically 0 at step 0 when both are empty: the lowest column wins
    assert all(tr[j, 0] == 0 for j in both)


def test_single_archetype_and_single_step():
    w = W.random_workload(65, 1, s_a=1, seed=11)
    ai, av, ac, tr, flags = run_a(w)
    assert flags == [] and np.all(tr == 0)
    np.testing.assert_array_equal(parity.dense_atoms(ai, av, ac, 1), np.ones((65, 1)))
    w = W.make("c1")
    ai, av, ac, tr, flags = run_a(w, T=1, cap=w.cap - w.T + 1)
    assert flags == []
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), T=1)


def test_step_size_table_and_scale_folding():
    w = W.make("c1")
    T = 120
    # gamma_0 = 1 then 0.55 per step: the running scale (0.45^t) drops below
    # 2^-64 and is folded back into the state
    gam = np.full(T, 0.55, np.float32)
    gam[0] = 1.0
    ai, av, ac, tr, flags = run_a(w, T=T, cap=w.cap - w.T + T, gamma=gam)
    assert flags == []
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), gamma=gam.astype(np.float64), T=T)
    # the default schedule passed as an explicit f32 table matches NULL
    tab = (2.0 / (np.arange(w.T) + 2.0)).astype(np.float32)
    assert_same_result(run_a(w), run_a(w, gamma=tab))


def test_cap_overflow_is_reported():
    w = W.make("c1")
    ai, av, ac, tr, flags = run_a(w)
    need = int(ac.max())
    _, _, ac2, _, flags2 = run_a(w, cap=need - 1)
    assert "CAP_OVERFLOW" in flags2
    assert int(ac2.max()) <= need - 1


def test_bad_step_size_is_reported():
    w = W.make("c1")
    gam = np.full(w.T, 0.5, np.float32)
    gam[3] = 1.5
    *_, flags = run_a(w, gamma=gam)
    assert "BAD_GAMMA" in flags


def test_deterministic_bitwise():
    w = W.make("c2")
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    assert_same_result(run_a(w, ops=ops), run_a(w, ops=ops))


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "empty"])
def test_support_argmin_equals_dense_scan(name, a_options):
    # On non-negative data the argmin is taken from the minimum over supp(t2)
    # and the touched-column bitmap; it must give the very index a dense scan
    # of the same f32 state gives, at every step of every cell.
    if name == "empty":
        w = W.random_workload(300, 40, s_a=3, seed=9, empty_k2b_every=3, empty_ap_every=4)
    else:
        w = W.make(name)
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    a_options.set(dense_argmin=True)
    dense = run_a(w, ops=ops)
    a_options.clear("dense_argmin")
    fast = run_a(w, ops=ops)
    assert dense[4] == [] and fast[4] == []
    assert_same_result(dense, fast)


def test_large_capacity_keeps_atoms_in_lds():
    # cap > 128: the atom list moves from registers to LDS
    w = W.make("c1")
    T = 200
    ai, av, ac, tr, flags = run_a(w, T=T, cap=w.cap - w.T + T)
    assert flags == []
    cells = np.arange(0, w.n, 5)
    parity.check_a(w, tr[cells], ai[cells], av[cells], ac[cells], cells, T=T)


def test_large_k_and_large_capacity():
    # state in workspace and atoms in LDS together
    w = W.random_workload(37, 45_000, t1_per_row=6, k2b_per_row=20, s_a=5, seed=17, T=140)
    ai, av, ac, tr, flags = run_a(w, T=140)
    assert flags == []
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), T=140)


def test_lane_group_widths_agree_bitwise(a_options):
    # 16, 32 or 64 lanes per cell only changes which lanes carry a cell; each
    # column sees the same operations in the same order, so the results must
    # be bit-identical (and match the oracle)
    w = W.random_workload(777, 300, t1_per_row=14, k2b_per_row=10, s_a=6, seed=23)
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    res = {}
    for g in ("16", "32", "64"):
        a_options.set(group=int(g))
        res[g] = run_a(w, ops=ops)
        assert res[g][4] == []
    a_options.clear("group")
    assert_same_result(res["16"], res["32"])
    assert_same_result(res["16"], res["64"])
    parity.check_a(w, res["32"][3], res["32"][0], res["32"][1], res["32"][2], np.arange(w.n))


def _support_case(name):
    if name in ("c1", "c2", "c3"):
        return W.make(name), {}
    if name == "empty":
        return W.random_workload(300, 40, s_a=3, seed=9, empty_k2b_every=3, empty_ap_every=4), {}
    if name == "signed":      # every cell leaves the support path at its first negative product
        return W.random_workload(400, 333, t1_per_row=12, k2b_per_row=9, s_a=7, seed=5,
                                 signed=True), {}
    if name == "long_t1_rows":  # t1 rows of 0 to 10 chunks: full batches and every tail size
        return W.random_workload(300, 2500, t1_per_row=300, k2b_per_row=40, s_a=6, seed=41), {}
    if name == "long_rows":   # K2B rows from 0 to 1600 entries: some exceed the first pass
        return W.random_workload(200, 3000, t1_per_row=40, k2b_per_row=800, s_a=6, seed=29), {}
    if name == "very_long_rows":  # up to 12000 entries: some exceed the long-row pass too
        return W.random_workload(40, 12000, t1_per_row=60, k2b_per_row=3000, s_a=6, seed=31,
                                 T=20), {"T": 20}
    if name == "fold":        # the running scale is folded back: those cells go to the dense kernel
        w = W.make("c1")
        gam = np.full(120, 0.55, np.float32)
        gam[0] = 1.0
        return w, {"T": 120, "cap": w.cap - w.T + 120, "gamma": gam}
    if name == "restarts":    # gamma = 1 every 7 steps: support state and marks restart
        w = W.make("c2")
        gam = (2.0 / (np.arange(60) % 7 + 2.0)).astype(np.float32)
        return w, {"T": 60, "cap": w.cap - w.T + 60, "gamma": gam}
    if name == "bad_gamma":
        w = W.make("c1")
        gam = np.full(w.T, 0.5, np.float32)
        gam[3] = 1.5
        return w, {"gamma": gam}
    if name == "cap_overflow":
        return W.make("c1"), {"cap": 12}
    raise KeyError(name)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "empty", "signed", "long_t1_rows", "long_rows",
                                  "very_long_rows", "fold", "restarts", "bad_gamma",
                                  "cap_overflow"])
def test_support_state_equals_dense_kernel(name, a_options):
    # The support state (h kept on supp(t2) only, plus bitmaps) must give the
    # dense kernel's results bit for bit; cells it cannot settle are redone by
    # the dense kernel. Forced on here for every k, with one cell per wave.
    w, kw = _support_case(name)
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    a_options.set(group=64)
    a_options.set(support=0)
    dense = run_a(w, ops=ops, **kw)
    a_options.set(support=1)
    for waves in ("20", "32"):    # two support capacities
        a_options.set(support_waves=int(waves))
        sup = run_a(w, ops=ops, **kw)
        assert sup[4] == dense[4]
        assert_same_result(dense, sup)
    if name in ("c1", "c2", "empty", "long_t1_rows", "long_rows"):
        parity.check_a(w, sup[3], sup[0], sup[1], sup[2], np.arange(w.n))


def test_support_state_is_the_default_for_large_k():
    import sparse_archetypal_analysis_amd as saa
    # the workspace then carries the queue of cells left to the dense kernel
    big = saa.seacells_fw_a_columns_workspace(1000, 6700, 50, 62, 10)
    assert big >= 2 * 1000 * 4 + saa.seacells_fw_a_columns_workspace(1000, 1000, 50, 60, 10)


@pytest.mark.parametrize("group", [16, 64])
def test_nan_state_raises_nonfinite(group, a_options):
    # A cell whose K2B row holds NaN in every column has no gradient entry
    # below +inf: the argmin finds no minimum, NONFINITE is raised, and the
    # other cells (independent) are exactly those of the run without it.
    import dataclasses
    a_options.set(group=group)
    w = W.random_workload(40, 24, t1_per_row=4, k2b_per_row=5, s_a=3, seed=71)
    k2b = w.k2b.toarray()
    k2b[7, :] = np.nan
    bad = dataclasses.replace(w, k2b=W.dense_to_csr(k2b))
    clean = run_a(w)
    got = run_a(bad)
    assert clean[4] == [] and got[4] == ["NONFINITE"]
    keep = np.arange(w.n) != 7
    assert_same_result(tuple(x[keep] for x in clean[:4]) + (None,),
                       tuple(x[keep] for x in got[:4]) + (None,))
