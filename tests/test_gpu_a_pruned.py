"""The A update's pruning + renormalisation variant on the GPU (the page's
`fw_columns_a_gpu` with `pruning`) against the f64 oracle, by trace replay."""
import numpy as np
import pytest

import workloads as W
from tests import parity
from tests.gpu_run import dev, run_a

pytestmark = pytest.mark.gpu


def weights_invariants(av, ac, thr):
    slot = np.arange(av.shape[1])[None, :] < ac[:, None]
    a = np.where(slot, av, 0.0)
    assert np.all(a >= 0.0)
    assert not np.any((a > 0.0) & (a <= thr)), "a weight at or below the threshold survived"
    s = a.sum(axis=1)
    assert np.all((np.abs(s - 1.0) < 1e-5) | (s == 0.0))


@pytest.mark.parametrize("name,thr", [("c1", 0.0), ("c1", 0.0213), ("c1", 0.0871),
                                      ("c2", 0.0213), ("c2", 0.0047)])
def test_small_configs_all_cells(name, thr):
    w = W.make(name)
    ai, av, ac, tr, flags = run_a(w, prune=thr)
    assert flags == []
    weights_invariants(av, ac, thr)
    rep = parity.check_a(w, tr, ai, av, ac, np.arange(w.n), prune=thr)
    print("\n%s thr=%g: %s" % (name, thr, rep))
    assert rep.skipped <= 0.1 * w.n


def test_threshold_above_one_drops_everything():
    # every weight is <= 1: each step ends with a = 0, so from step 1 on the
    # gradient is -t2 and the pick is the lowest column of the row's maximum
    # (each drop takes a row back out of the f32 state, leaving rounding-level
    # residue: the closed form is exact where the row's maximum is clearly
    # unique; elsewhere, e.g. empty rows with g == 0, the replay decides)
    w = W.make("c1")
    ai, av, ac, tr, flags = run_a(w, prune=2.0)
    assert flags == []
    t2 = np.asarray(w.k2b.todense())
    srt = np.sort(t2, axis=1)
    clear = srt[:, -1] - srt[:, -2] > 1e-4 * np.maximum(srt[:, -1], 1e-30)
    assert clear.mean() > 0.5
    np.testing.assert_array_equal(tr[clear, 1:], np.repeat(np.argmin(-t2[clear], axis=1)[:, None],
                                                            w.T - 1, axis=1))
    slot = np.arange(av.shape[1])[None, :] < ac[:, None]
    assert np.all(np.where(slot, av, 0.0) == 0.0)
    parity.check_a(w, tr, ai, av, ac, np.arange(w.n), prune=2.0)


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_large_configs_sampled_cells(name):
    # c3: the dense kernel; c4: the support state, whose cells that drop an
    # atom are finished by the dense kernel
    w = W.make(name)
    thr = 0.0213
    ai, av, ac, tr, flags = run_a(w, prune=thr)
    assert flags == []
    weights_invariants(av, ac, thr)
    rng = np.random.default_rng(17)
    cells = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, size=200, replace=False)]))
    rep = parity.check_a(w, tr[cells], ai[cells], av[cells], ac[cells], cells, prune=thr)
    print("\n%s thr=%g: %s" % (name, thr, rep))
    assert rep.skipped <= 0.1 * cells.shape[0]


@pytest.mark.parametrize("thr", [1e-6, 0.0213])
def test_support_state_equals_dense_kernel(thr, a_options):
    # 1e-6: nothing drops, the support state renormalises every step exactly
    # as the dense kernel does; 0.0213: cells drop atoms and are handed over
    w = W.random_workload(300, 3000, t1_per_row=40, k2b_per_row=60, s_a=6, seed=61)
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    a_options.set(support=0)
    dense = run_a(w, ops=ops, prune=thr)
    a_options.set(support=1)
    sup = run_a(w, ops=ops, prune=thr)
    assert dense[4] == [] and sup[4] == []
    np.testing.assert_array_equal(dense[3], sup[3])
    np.testing.assert_array_equal(dense[2], sup[2])
    slot = np.arange(dense[0].shape[1])[None, :] < dense[2][:, None]
    np.testing.assert_array_equal(dense[0][slot], sup[0][slot])
    np.testing.assert_array_equal(dense[1][slot].view(np.uint32), sup[1][slot].view(np.uint32))
    rep = parity.check_a(w, sup[3], sup[0], sup[1], sup[2], np.arange(w.n), prune=thr)
    print("\nthr=%g: %s" % (thr, rep))


def test_plain_and_pruned_agree_while_nothing_drops():
    # at a threshold below every weight the pruned run only renormalises (a
    # factor 1 +- rounding): the picks and weights stay those of the plain run
    w = W.make("c2")
    plain = run_a(w)
    pruned = run_a(w, prune=1e-9)
    same = (plain[3] == pruned[3]).all(axis=1)
    assert same.mean() > 0.99
    slot = np.arange(plain[0].shape[1])[None, :] < plain[2][:, None]
    d = np.abs(np.where(slot, plain[1] - pruned[1], 0.0))[same]
    assert d.max() <= 1e-5
