"""The two largest kNN-kernel workloads (n = 500k, k = 6700 and n = 1M,
k = 10000) at full size on the GPU, against the f64 oracle.

A update: trace replay on a random sample of cells (the oracle redoes each
sampled cell exactly, with its Frank-Wolfe gap), properties that hold for
every cell, and the compact per-cell state against the dense kernel bit for
bit on every cell. B argmin: every column and the full gap against the full
oracle.

Each workload is generated once per module (about 12 s and 60 s on the GPU
machine; kNN on the GPU, products on the host cores).
"""
import sys

import numpy as np
import pytest

import workloads as W
from tests import parity
from tests.gpu_run import dev, run_a, run_b

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", params=["c4", "c5"])
def big(request):
    w = W.make(request.param, log=_log)
    ops_a = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    yield request.param, w, ops_a


def test_a_update_sampled_cells_and_invariants(big):
    name, w, ops = big
    gaps = []
    ai, av, ac, tr, flags = run_a(w, ops=ops, gap_out=gaps)
    assert flags == []
    rng = np.random.default_rng(4 if name == "c4" else 5)
    cells = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, size=160, replace=False)]))
    rep = parity.check_a(w, tr[cells], ai[cells], av[cells], ac[cells], cells,
                         fw_gap=gaps[0][cells])
    assert not np.any(np.isnan(gaps[0]))
    print("\n%s sampled: %s" % (name, rep))
    parity.check_atom_layout(ai[cells], ac[cells], tr[cells], w.a_prev_t, cells)
    # every cell: counts within [seeds, cap], picks in range, weights on the simplex
    assert np.all(ac >= np.diff(w.a_prev_t.indptr)) and np.all(ac <= w.cap)
    assert np.all((tr >= 0) & (tr < w.k))
    slot = np.arange(ai.shape[1])[None, :] < ac[:, None]
    sums = np.where(slot, av, 0.0).sum(axis=1)
    np.testing.assert_allclose(sums, 1.0, atol=1e-5)
    assert np.all(np.where(slot, av, 0.0) >= 0.0)


def test_compact_state_equals_dense_kernel(big, monkeypatch):
    # large k takes the compact per-cell state by default; the dense kernel
    # must give the same picks and weights bit for bit on every cell
    name, w, ops = big
    fast = run_a(w, ops=ops)
    monkeypatch.setenv("SEACELLS_A_SUPPORT", "0")
    dense = run_a(w, ops=ops)
    assert fast[4] == [] and dense[4] == []
    np.testing.assert_array_equal(fast[3], dense[3])
    np.testing.assert_array_equal(fast[2], dense[2])
    slot = np.arange(fast[0].shape[1])[None, :] < fast[2][:, None]
    np.testing.assert_array_equal(fast[0][slot], dense[0][slot])
    np.testing.assert_array_equal(fast[1][slot].view(np.uint32), dense[1][slot].view(np.uint32))


def test_b_argmin_all_columns(big):
    name, w, _ = big
    gl = []
    v, i, g, flags = run_b(w, gap_out=gl)
    assert flags == []
    rep = parity.check_b(w, v, i, g, fw_gap=gl[0])
    print("\n%s: %s" % (name, rep))
