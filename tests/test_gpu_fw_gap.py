"""The full Frank-Wolfe duality gap outputs on the GPU against the f64 oracle.

A update: the gap <g, a> - min g of each returned column, checked on the
oracle's replay of the GPU's own trajectory. B argmin:
sum(B * G) - sum_c min_i G[i, c]. The page computes only the B side's
sum(B * G) half; the full gaps are the certificates the method's stopping
test needs (the oracle's pins fix both against the objective itself).
"""
import numpy as np
import pytest
import torch

import sparse_archetypal_analysis_amd as saa
import workloads as W
from tests import parity
from tests.gpu_run import dev, run_a, run_b, run_b_dense
from tests.test_gpu_a_update import _support_case, identity_workload

pytestmark = pytest.mark.gpu


def a_with_gap(w, **kw):
    gaps = []
    res = run_a(w, gap_out=gaps, **kw)
    assert res[4] == []
    assert not np.any(np.isnan(gaps[0])), "a cell's gap was not written"
    return res, gaps[0]


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_a_gap_all_cells(name):
    w = W.make(name)
    (ai, av, ac, tr, _), gap = a_with_gap(w)
    rep = parity.check_a(w, tr, ai, av, ac, np.arange(w.n), fw_gap=gap)
    print("\n%s: %s" % (name, rep))


def test_a_gap_c3_sampled_cells():
    w = W.make("c3")
    (ai, av, ac, tr, _), gap = a_with_gap(w)
    rng = np.random.default_rng(30)
    cells = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, size=300, replace=False)]))
    rep = parity.check_a(w, tr[cells], ai[cells], av[cells], ac[cells], cells, fw_gap=gap[cells])
    print("\nc3 sampled: %s" % (rep,))


def test_a_gap_identity_closed_form():
    # g = a - B[j, :] (t1 = I). Cells 2, 3 alternate picks: after 50 steps
    # a = (25/51, 26/51), gap (50+2)/(2*51^2) = 26/2601; cell 0 sits at its
    # optimum e_0 (gap 0)
    w = identity_workload()
    (ai, av, ac, tr, _), gap = a_with_gap(w)
    np.testing.assert_allclose(gap[2:], 26 / 2601, rtol=0, atol=1e-7)
    assert abs(gap[0]) <= 1e-7
    # cell 1: a_0 = x = 4 / (50 * 51) after 50 steps, g = (x, -x), gap 2 x^2
    assert abs(gap[1] - 2 * (4 / 2550) ** 2) <= 1e-7
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), fw_gap=gap)


@pytest.mark.parametrize("thr", [0.0213, 2.0])
def test_a_gap_pruned(thr):
    w = W.make("c1")
    (ai, av, ac, tr, _), gap = a_with_gap(w, prune=thr)
    rep = parity.check_a(w, tr, ai, av, ac, np.arange(w.n), prune=thr, fw_gap=gap)
    print("\nthr=%g: %s" % (thr, rep))


def test_a_gap_without_a_step_table_and_with_folds():
    # T > 256: the kernels compute the step schedule as they go; and a
    # schedule whose running scale is folded back into the state
    w = W.make("c1")
    T = 260
    (ai, av, ac, tr, _), gap = a_with_gap(w, T=T, cap=w.cap - w.T + T)
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), T=T, fw_gap=gap)
    T = 120
    gam = np.full(T, 0.55, np.float32)
    gam[0] = 1.0
    (ai, av, ac, tr, _), gap = a_with_gap(w, T=T, cap=w.cap - w.T + T, gamma=gam)
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), gamma=gam.astype(np.float64), T=T,
                   fw_gap=gap)


def test_a_gap_large_k_state_in_workspace(a_options):
    a_options.set(support=0)
    w = W.random_workload(37, 45_000, t1_per_row=6, k2b_per_row=20, s_a=5, seed=7, T=30)
    (ai, av, ac, tr, _), gap = a_with_gap(w, T=30)
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), T=30, fw_gap=gap)


def test_a_gap_large_capacity_atoms_in_lds():
    w = W.make("c1")
    cap = 200
    (ai, av, ac, tr, _), gap = a_with_gap(w, cap=cap)
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), fw_gap=gap)


@pytest.mark.parametrize("name", ["c2", "empty", "long_rows", "restarts", "fold"])
@pytest.mark.parametrize("prune", [None, 1e-6])
def test_a_gap_support_state_equals_dense_kernel(name, prune, a_options):
    # the compact state computes the gap from the same values in the same
    # order as the dense kernel: equal bit for bit (cells it cannot price go
    # to the dense kernel)
    w, kw = _support_case(name)
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    a_options.set(group=64)
    a_options.set(support=0)
    dense, gd = a_with_gap(w, ops=ops, prune=prune, **kw)
    a_options.set(support=1)
    sup, gs = a_with_gap(w, ops=ops, prune=prune, **kw)
    np.testing.assert_array_equal(dense[3], sup[3])
    np.testing.assert_array_equal(gd.view(np.uint32), gs.view(np.uint32))


def test_a_gap_lane_groups_agree(a_options):
    # 16 / 32 / 64 lanes per cell sum <g, a> in different orders: equal to
    # rounding, and each within the oracle's tolerance
    w = W.random_workload(777, 300, t1_per_row=14, k2b_per_row=10, s_a=6, seed=23)
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    for g in ("16", "32", "64"):
        a_options.set(group=int(g))
        (ai, av, ac, tr, _), gap = a_with_gap(w, ops=ops)
        parity.check_a(w, tr, ai, av, ac, np.arange(w.n), fw_gap=gap)


def test_a_gap_large_k_default_path():
    # k >= 2048: the compact state takes the cells by default
    w = W.random_workload(500, 4000, t1_per_row=30, k2b_per_row=60, s_a=8, seed=41)
    (ai, av, ac, tr, _), gap = a_with_gap(w)
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), fw_gap=gap)


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_b_full_gap(name):
    w = W.make(name)
    gl = []
    v, i, g, flags = run_b(w, gap_out=gl)
    assert flags == []
    rep = parity.check_b(w, v, i, g, fw_gap=gl[0])
    print("\n%s: %s, fw_gap %.9g" % (name, rep, gl[0]))


def test_b_full_gap_identity_exact():
    # sum(B * G) = 1 and both column minima are -1/2: the gap is 2, exactly
    n, k = 4, 2
    B = np.zeros((n, k), np.float32)
    B[0, 0] = B[1, 1] = 1.0
    w, _ = run_b_dense(B, np.ones((k, k), np.float32), np.full((n, k), 0.5, np.float32), B)
    gl = []
    run_b(w, gap_out=gl)
    assert gl[0] == 2.0


def test_b_full_gap_needs_b():
    w = W.make("c1")
    fg = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(saa.SeacellsError):
        saa.seacells_fw_b_argmin(dev(w.k2b), dev(w.aat), dev(w.k2at), None, w.n, w.k, fw_gap=fg)
