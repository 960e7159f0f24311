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
import scipy.sparse as sp
import torch

import sparse_archetypal_analysis_amd as saa
import workloads as W
from oracle import sparse as S
from tests import parity
from tests.gpu_run import assert_same_atoms, dev, host, run_a, run_a_as_timed, run_b, run_b_as_timed

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
    # the f64 oracle recomputes every gradient from scratch: ~270 cells/s at
    # n = 500k, k = 6700 and ~40 cells/s at n = 1M, k = 10000 on 16 cores
    size = 2000 if name == "c4" else 400
    cells = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, size=size, replace=False)]))
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
    # the call the benchmark times (no trace, no gap, outputs and workspace
    # reused over repeated calls) gives the same atoms bit for bit
    timed = run_a_as_timed(w, ops=ops)
    assert timed[3] == []
    assert_same_atoms((ai, av, ac), timed)


def test_compact_state_equals_dense_kernel(big, a_options):
    # large k takes the compact per-cell state by default; the dense kernel
    # must give the same picks and weights bit for bit on every cell
    name, w, ops = big
    fast = run_a(w, ops=ops)
    a_options.set(support=0)
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
    ops = (dev(w.k2b), dev(w.aat), dev(w.k2at), dev(w.b))
    v, i, g, flags = run_b(w, ops=ops, gap_out=gl)
    assert flags == []
    rep = parity.check_b(w, v, i, g, fw_gap=gl[0])
    print("\n%s: %s" % (name, rep))
    # the call the benchmark times (no full gap, reused workspace and
    # outputs) and a call without B: the same minima and rows bit for bit
    tv, ti, tg, tflags = run_b_as_timed(w, ops=ops)
    assert tflags == []
    np.testing.assert_array_equal(ti, i)
    np.testing.assert_array_equal(tv.view(np.uint32), v.view(np.uint32))
    assert np.float32(tg).view(np.uint32) == np.float32(g).view(np.uint32)
    nv, ni, _, nflags = run_b(w, ops=ops[:3] + (None,))
    assert nflags == []
    np.testing.assert_array_equal(ni, i)
    np.testing.assert_array_equal(nv.view(np.uint32), v.view(np.uint32))


def _place_rows(prod, rows, n):
    """An n-row CSR holding the oracle rows ``prod`` at positions ``rows``
    (ascending) and nothing elsewhere."""
    counts = np.zeros(n, np.int64)
    counts[rows] = np.diff(prod.indptr)
    ptr = np.zeros(n + 1, np.int64)
    np.cumsum(counts, out=ptr[1:])
    return sp.csr_matrix((prod.value, prod.indices, ptr), shape=(n, prod.shape[1]))


def _chain_rows(K, X, rows):
    """Rows ``rows`` (ascending) of K (K X) by the oracle: the rows of K X
    that K's rows reach, then the product with them. Returns the product and
    the most terms in a first-level sum."""
    nb = np.unique(K[rows].indices)
    first = S.matmul_rows(K, X, nb)
    second = S.matmul_rows(K, _place_rows(first, nb, K.shape[0]), rows)
    return second, int(first.terms.max()) if first.terms.size else 0


def test_device_operands_full_size(big):
    name, w, _ = big
    K = W.kernel_matrix(w)
    st = saa.new_status()
    dK, dAt = dev(K), dev(w.a_prev_t)
    ops = saa.device_operands(dK, dev(w.b), dAt, status=st)
    acc, _ = saa.rss(dK, ops["k2b"], dAt, ops["t1"], ops["aat"], status=st)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    _log("%s: device operands built" % name)
    # every entry against the generator's operands (f64 products of the f64
    # kernel, rounded to f32; t1 and A A^T symmetrised)
    for nm in ("k2b", "t1", "aat", "k2at"):
        ref, d = getattr(w, nm), ops[nm]
        assert d.nnz == ref.nnz, nm
        assert torch.equal(d.row_ptr.cpu(), torch.from_numpy(ref.indptr.astype(np.int32))), nm
        assert torch.equal(d.col_idx, torch.from_numpy(ref.indices.astype(np.int32)).cuda()), nm
        rv = torch.from_numpy(ref.data).cuda().double()
        rel = ((d.val.double() - rv).abs() / rv.abs()).max().item()
        del rv
        assert rel <= 2e-5, (nm, rel)
    _log("%s: generator operands matched" % name)
    # sampled rows against the oracle
    rng = np.random.default_rng(40 if name == "c4" else 50)
    rows = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, size=100, replace=False)]))
    parity.check_product(host(ops["kb"], rows), S.matmul_rows(K, w.b, rows), what="K B")
    parity.check_product(host(ops["kat"], rows), S.matmul_rows(K, w.a_prev_t, rows),
                         what="K A^T")
    want, l1 = _chain_rows(K, w.b, rows)
    parity.check_product(host(ops["k2b"], rows), want, extra_terms=l1 + 1, what="K^2 B")
    want, l1 = _chain_rows(K, w.a_prev_t, rows)
    parity.check_product(host(ops["k2at"], rows), want, extra_terms=l1 + 1, what="K^2 A^T")
    arch = np.unique(np.concatenate([[0, w.k - 1], rng.choice(w.k, size=30, replace=False)]))
    bt = S.transpose(w.b)
    cells = np.unique(bt[arch].indices)
    k2b_cells, l1 = _chain_rows(K, w.b, cells)
    t1_rows = S.matmul(bt[arch], _place_rows(k2b_cells, cells, w.n))
    l2 = int(k2b_cells.terms.max()) if k2b_cells.terms.size else 0
    parity.check_product(host(ops["t1"], arch), t1_rows, extra_terms=l1 + l2 + 2, what="t1")
    a = S.transpose(w.a_prev_t)
    parity.check_product(host(ops["aat"], arch), S.matmul_rows(a, w.a_prev_t, arch),
                         what="A A^T")
    # transposes bit for bit
    for nm, ref in (("bt", bt), ("a", a)):
        got = host(ops[nm])
        assert np.array_equal(got.indptr, ref.indptr) and np.array_equal(got.indices, ref.indices)
        assert np.array_equal(got.data.view(np.uint32), ref.data.astype(np.float32).view(np.uint32))
    _log("%s: sampled rows matched" % name)
    # RSS: the expansion on the generator's operands
    val, scale = S.rss_of_operands(K, w.k2b, w.a_prev_t, w.t1, w.aat)
    assert abs(float(acc.item()) - val) <= 1e-5 * scale, (float(acc.item()), val, scale)
    print("\n%s: rss %.6e (oracle on generator operands %.6e, scale %.3e)" % (
        name, float(acc.item()), val, scale))
