"""The B update as a loop of Frank-Wolfe steps on the device, and its two
new pieces (include/seacells_sparse.h): the sparse sum alpha X + beta Y and
the vertex matrix of the B argmin's picks.

Sum: the pattern bit for bit against oracle.sparse.add (the union of the
stored patterns), every value within 2.02 * 2^-24 * (|alpha x| + |beta y|)
(two roundings of the products, one of the sum). Vertex matrix: bit for bit.

Loop (oracle.b_loop.fw_b_loop, K^2 B recomputed from B in f64 at every
step): the oracle replays the GPU's picks; every pick must be the oracle's or
within the tie rule of the B argmin (G at the pick within 1e-5 of the term
scale of the minimum); the minimum values and gaps follow the B argmin's
policy; B after the loop within 1e-5 absolute; K^2 B after the loop within
5e-5 relative (its updates accumulate f32 rounding of the products
K (K S) and of the sums, decaying with the step weights).
"""
import zlib

import numpy as np
import pytest
import scipy.sparse as sp
import torch

import sparse_archetypal_analysis_amd as saa
import workloads as W
from oracle import b_loop as BL
from oracle import sparse as S
from tests import parity
from tests.gpu_run import dev, host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def rand_csr(rng, m, q, density, signed=True, zeros=0.05, empty_rows=()):
    mask = rng.random((m, q)) < density
    mask[list(empty_rows), :] = False
    rows, cols = np.nonzero(mask)
    vals = rng.uniform(0.1, 1.0, size=rows.size)
    if signed:
        vals *= rng.choice([-1.0, 1.0], size=rows.size)
    vals[rng.random(rows.size) < zeros] = 0.0
    out = sp.csr_matrix((vals.astype(np.float32), (rows, cols)), shape=(m, q))
    out.sort_indices()
    return out


ADD_CASES = {
    # name: (m, q, density x, density y, alpha, beta)
    "small": (30, 20, 0.2, 0.15, 0.75, -1.5),
    "scale_only": (50, 40, 0.3, 0.0, np.float32(1.0 / 3.0), 2.0),
    "disjoint_heavy": (200, 3000, 0.05, 0.02, 1.0, 1.0),
    "alpha_zero": (40, 30, 0.3, 0.3, 0.0, 1.0),
    "long_rows": (8, 20000, 0.3, 0.01, 0.5, 0.5),
}


@pytest.mark.parametrize("case", sorted(ADD_CASES))
def test_sparse_add_matches_oracle(case):
    m, q, dx, dy, alpha, beta = ADD_CASES[case]
    alpha, beta = float(np.float32(alpha)), float(np.float32(beta))
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    x = rand_csr(rng, m, q, dx, empty_rows=(0,))
    y = rand_csr(rng, m, q, dy, empty_rows=(0, m - 1))
    st = saa.new_status()
    got = host(saa.csr_add(alpha, dev(x), beta, dev(y), status=st))
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    want = S.add(alpha, x, beta, y)
    scale = S.add(abs(alpha), abs(x), abs(beta), abs(y))
    assert np.array_equal(got.indptr, want.indptr)
    assert np.array_equal(got.indices, want.indices)
    err = np.abs(got.data.astype(np.float64) - want.data)
    assert np.all(err <= 2.02 * U * scale.data), float(np.max(err - 2.02 * U * scale.data))


def test_sparse_add_keeps_cancelled_sums_and_flags_unsorted_rows():
    x = sp.csr_matrix(np.array([[2.0, 0.0, 1.0]], np.float32))
    y = sp.csr_matrix(np.array([[-2.0, 3.0, 0.0]], np.float32))
    got = host(saa.csr_add(1.0, dev(x), 1.0, dev(y)))
    assert list(got.indices) == [0, 1, 2] and list(got.data) == [0.0, 3.0, 1.0]
    # a row whose columns are not ascending is flagged
    bad = sp.csr_matrix((np.array([1.0, 1.0], np.float32), np.array([2, 1]), np.array([0, 2])),
                        shape=(1, 3))
    st = saa.new_status()
    saa.seacells_csr_add_rows(dev(bad), dev(x), status=st)
    torch.cuda.synchronize()
    assert "BAD_INDEX" in saa.status_flags(st)


def test_sparse_add_flags_a_row_pointer_past_the_entries():
    # rows of one operand whose range runs past its entries or backwards:
    # each operand's range is checked on its own, the bad ones count as
    # empty, the other operand's rows stay in bounds, and the call reports it
    x = sp.csr_matrix(np.array([[2.0, 0.0, 1.0], [0.0, 4.0, 0.0], [1.0, 1.0, 1.0]], np.float32))
    y = sp.csr_matrix(np.array([[1.0, 1.0, 0.0], [0.0, 0.0, 5.0], [0.0, 2.0, 0.0]], np.float32))
    for bad_first in (True, False):
        xd, yd = dev(x), dev(y)
        (xd if bad_first else yd).row_ptr[2] = 9  # row 1: (2, 9) past nnz; row 2: (9, 6)
        st = saa.new_status()
        ptr, _ = saa.seacells_csr_add_rows(xd, yd, status=st) if bad_first else \
            saa.seacells_csr_add_rows(yd, xd, status=st)
        torch.cuda.synchronize()
        assert saa.status_flags(st) == ["BAD_INDEX"]
        # row 0 is the plain sum; rows 1 and 2 keep the good operand's entries
        counts = np.diff(ptr.cpu().numpy().astype(np.int64))
        good = y if bad_first else x
        assert counts[0] == 3 and list(counts[1:]) == list(np.diff(good.indptr)[1:])


@pytest.mark.parametrize("n,k", [(1, 5), (7, 30), (100_000, 1300), (1_000_000, 10_000)])
def test_vertex_matrix_bit_exact(n, k):
    rng = np.random.default_rng(n + k)
    picks = rng.integers(0, n, size=k)
    if k > 3:
        picks[1] = picks[3]  # two columns on one row
    st = saa.new_status()
    got = host(saa.seacells_fw_b_vertex(torch.from_numpy(picks.astype(np.int32)).cuda(), n, 0.5,
                                        status=st))
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    want = S.picks(picks, n, 0.5)
    assert np.array_equal(got.indptr, want.indptr)
    assert np.array_equal(got.indices, want.indices)
    assert np.all(got.data == 0.5)


@pytest.mark.parametrize("name,T", [("c1", 12), ("c2", 8), ("c3", 3)])
def test_b_loop_against_oracle_replay(name, T):
    w = W.make(name)
    K = W.kernel_matrix(w)
    st = saa.new_status()
    res = saa.fw_b_loop(dev(K), dev(w.k2b), dev(w.aat), dev(w.k2at), dev(w.b), T, status=st)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    flips, krel = parity.check_b_loop(K, w.b, w.aat, w.k2at, T, res)
    print("\n%s: %d steps, %d picks differ within the tie rule, K^2B max rel err %.2e"
          % (name, T, flips, krel))


def test_b_loop_with_a_step_size_table():
    w = W.make("c1")
    K = W.kernel_matrix(w)
    gam = [0.5, 0.25, 0.125, 0.6]
    res = saa.fw_b_loop(dev(K), dev(w.k2b), dev(w.aat), dev(w.k2at), dev(w.b), len(gam),
                        gammas=gam)
    torch.cuda.synchronize()
    picks = res[2].cpu().numpy().astype(np.int64)
    orc = BL.fw_b_loop(K, w.b, w.aat, w.k2at, len(gam), gammas=gam, force=picks)
    assert np.max(np.abs(host(res[0]).toarray() - orc.b)) <= 1e-5
    kd = host(res[1]).toarray().astype(np.float64)
    assert np.all(np.abs(kd - orc.k2b) <= 5e-5 * np.abs(orc.k2b) + 1e-6 * np.max(np.abs(orc.k2b)))


def test_b_loop_on_a_tiny_problem():
    # n = 7 cells, k = 3 archetypes, every operand formed here in f64 from a
    # random symmetric K, column-stochastic B and A, then cast to f32
    rng = np.random.default_rng(77)
    n, k, T = 7, 3, 6
    Kd = rng.uniform(0, 1, size=(n, n)) * (rng.random((n, n)) < 0.5)
    Kd = (Kd + Kd.T) / 2 + np.eye(n)
    Bd = np.zeros((n, k))
    for c in range(k):
        sup = rng.choice(n, size=2, replace=False)
        Bd[sup, c] = rng.dirichlet(np.ones(2))
    Ad = rng.dirichlet(np.ones(k), size=n).T
    f32 = lambda m: sp.csr_matrix(np.asarray(m, np.float32))
    K, B = f32(Kd), f32(Bd)
    Kf, Bf, Af = (np.asarray(M.toarray() if sp.issparse(M) else M, np.float64)
                  for M in (K, B, f32(Ad)))
    k2b, aat, k2at = f32(Kf @ Kf @ Bf), f32(Af @ Af.T), f32(Kf @ Kf @ Af.T)
    res = saa.fw_b_loop(dev(K), dev(k2b), dev(aat), dev(k2at), dev(B), T)
    torch.cuda.synchronize()
    flips, krel = parity.check_b_loop(K, B, aat, k2at, T, res)
    assert krel <= 5e-5
