"""Pins of the f64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: brute-force differences of
the objective, enumeration of simplex vertices, a closed form, a worked
example with K = I, a special case that reduces to a library routine, or the
independent dense implementation. The method is the one on the source page
(bixverse-rs 0.6.4, seacells_kernels.rs): the `fw_columns_a_gpu` recurrence,
the `fw_argmin_b` gradient and argmin, and the tests of that page.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.sparse as sp

import oracle
from oracle import dense
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers: operands from dense K, B, A (test side, plain numpy)
# --------------------------------------------------------------------------

def operands(K, B, A):
    K2 = K @ K
    t1 = B.T @ K2 @ B
    t1 = (t1 + t1.T) / 2
    k2b = K2 @ B
    aat = A @ A.T
    k2at = K2 @ A.T
    return {nm: W.dense_to_csr(v.astype(np.float32)) for nm, v in
            dict(t1=t1, k2b=k2b, a_prev_t=A.T, aat=aat, k2at=k2at, b=B).items()}


def dyadic_problem(n, k, rng):
    """K, B, A with dyadic entries so every operand is exact in f32."""
    K = rng.integers(0, 5, size=(n, n)) / 4.0
    K = np.triu(K, 1)
    K = K + K.T + np.eye(n)
    B = np.zeros((n, k))
    cells = rng.choice(n, size=k, replace=False)
    for c in range(k):
        B[cells[c], c] = 0.5
        B[rng.integers(n), c] += 0.25
        B[rng.integers(n), c] += 0.25
    A = np.zeros((k, n))
    for j in range(n):
        A[rng.integers(k), j] += 0.5
        A[rng.integers(k), j] += 0.25
        A[rng.integers(k), j] += 0.25
    return K, B, A


def random_problem(n, k, rng):
    K = rng.uniform(0, 1, size=(n, n))
    K = (K + K.T) / 2
    np.fill_diagonal(K, 1.0)
    B = rng.dirichlet(np.ones(n), size=k).T
    A = rng.dirichlet(np.ones(k), size=n).T
    return K, B, A


def oracle_g_vector(ops, n, k, j):
    """The oracle's g for cell j at A_prev, one entry per forced index."""
    g = np.empty(k)
    for c in range(k):
        tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, 1, cells=[j],
                                 force=np.array([[c]]))
        g[c] = tr.g_taken[0, 0]
    return g


# --------------------------------------------------------------------------
# P1: brute-force central differences of the objective
# --------------------------------------------------------------------------

def test_p1_a_gradient_matches_objective_differences():
    rng = np.random.default_rng(11)
    n, k = 7, 3
    K, B, A = dyadic_problem(n, k, rng)
    ops = operands(K, B, A)
    h = 1e-3
    for j in range(n):
        g = oracle_g_vector(ops, n, k, j)
        for m in range(k):
            E = np.zeros_like(A)
            E[m, j] = h
            fd = (dense.objective(K, B, A + E) - dense.objective(K, B, A - E)) / (2 * h)
            # f is quadratic in A, so the central difference is exact up to rounding
            assert abs(2 * g[m] - fd) <= 1e-8 * max(1.0, abs(fd)), (j, m, 2 * g[m], fd)


def test_p1_b_gradient_matches_objective_differences():
    rng = np.random.default_rng(12)
    n, k = 8, 3
    K, B, A = dyadic_problem(n, k, rng)
    ops = operands(K, B, A)
    rows, cols = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    G, _ = oracle.fw_b_grad_at(ops["k2b"], ops["aat"], ops["k2at"], n, k, rows.ravel(), cols.ravel())
    G = G.reshape(n, k)
    h = 1e-3
    for i in range(n):
        for c in range(k):
            E = np.zeros_like(B)
            E[i, c] = h
            # f is quartic in B; a 4-point stencil is exact for quartics up to
            # rounding, and the closed form 2(K^2 B A A^T - K^2 A^T) is
            # independent of this stencil.
            f = lambda s: dense.objective(K, B + s * E, A)
            fd = (-f(2) + 8 * f(1) - 8 * f(-1) + f(-2)) / (12 * h)
            assert abs(2 * G[i, c] - fd) <= 1e-7 * max(1.0, abs(fd)), (i, c, 2 * G[i, c], fd)
    # the oracle's column minimum is the minimum of those entries
    res = oracle.fw_b_argmin(ops["k2b"], ops["aat"], ops["k2at"], ops["b"], n, k)
    np.testing.assert_allclose(res.val, G.min(axis=0), rtol=0, atol=1e-12)
    # and the gap is sum(B * G)
    assert abs(res.gap - float(np.sum(B * G))) < 1e-12


def test_p1_closed_form_gradients_match_differences():
    rng = np.random.default_rng(13)
    K, B, A = random_problem(6, 3, rng)
    h = 1e-5
    ga, gb = dense.grad_a(K, B, A), dense.grad_b(K, B, A)
    for (m, j) in [(0, 0), (2, 5), (1, 3)]:
        E = np.zeros_like(A)
        E[m, j] = h
        fd = (dense.objective(K, B, A + E) - dense.objective(K, B, A - E)) / (2 * h)
        assert abs(ga[m, j] - fd) < 1e-6 * max(1, abs(fd))
    for (i, c) in [(0, 0), (5, 2), (3, 1)]:
        E = np.zeros_like(B)
        E[i, c] = h
        fd = (dense.objective(K, B + E, A) - dense.objective(K, B - E, A)) / (2 * h)
        assert abs(gb[i, c] - fd) < 1e-6 * max(1, abs(fd))


# --------------------------------------------------------------------------
# P2: the FW vertex by enumerating every simplex vertex through the objective
# --------------------------------------------------------------------------

def test_p2_a_pick_is_best_vertex():
    rng = np.random.default_rng(21)
    n, k = 9, 4
    K, B, A = random_problem(n, k, rng)
    ops = operands(K, B, A)
    tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, 1)
    h = 1e-4
    A32 = ops["a_prev_t"].toarray().T.astype(np.float64)
    for j in range(n):
        dd = np.empty(k)
        for c in range(k):
            D = np.zeros_like(A32)
            D[:, j] = -A32[:, j]
            D[c, j] += 1.0
            dd[c] = (dense.objective(K, B, A32 + h * D) - dense.objective(K, B, A32 - h * D)) / (2 * h)
        order = np.argsort(dd, kind="stable")
        if dd[order[1]] - dd[order[0]] > 1e-5:
            assert tr.pick[j, 0] == order[0], (j, dd)


def test_p2_b_pick_is_best_vertex():
    rng = np.random.default_rng(22)
    n, k = 10, 3
    K, B, A = random_problem(n, k, rng)
    ops = operands(K, B, A)
    res = oracle.fw_b_argmin(ops["k2b"], ops["aat"], ops["k2at"], ops["b"], n, k)
    h = 1e-4
    B32 = ops["b"].toarray().astype(np.float64)
    A32 = ops["a_prev_t"].toarray().T.astype(np.float64)
    for c in range(k):
        dd = np.empty(n)
        for i in range(n):
            D = np.zeros_like(B32)
            D[:, c] = -B32[:, c]
            D[i, c] += 1.0
            dd[i] = (dense.objective(K, B32 + h * D, A32) - dense.objective(K, B32 - h * D, A32)) / (2 * h)
        order = np.argsort(dd, kind="stable")
        if dd[order[1]] - dd[order[0]] > 1e-5:
            assert res.row[c] == order[0], (c, dd)


# --------------------------------------------------------------------------
# P3: invariants
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c1():
    return W.make("c1")


def test_p3_columns_stay_on_simplex_and_match_step_weights(c1):
    w = c1
    cells = np.arange(0, w.n, 7)
    tr = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells)
    assert np.all(tr.a >= 0)
    np.testing.assert_allclose(tr.a.sum(axis=1), 1.0, atol=1e-12)
    # closed form of the recurrence: gamma_0 = 1 wipes the seeds, and the
    # weight of step t survives the later scalings as 2 (t + 1) / (T (T + 1))
    T = w.T
    for r in range(cells.shape[0]):
        want = np.zeros(w.k)
        for t in range(T):
            want[tr.pick[r, t]] += 2.0 * (t + 1) / (T * (T + 1))
        np.testing.assert_allclose(tr.a[r], want, rtol=0, atol=1e-13)


def test_p3_one_hot_after_first_step(c1):
    w = c1
    tr = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, 1, cells=np.arange(50))
    for r in range(50):
        e = np.zeros(w.k)
        e[tr.pick[r, 0]] = 1.0
        assert np.array_equal(tr.a[r], e)


def test_p3_fw_gap_nonnegative_and_line_search_descends():
    rng = np.random.default_rng(31)
    n, k, T = 8, 4, 6
    K, B, _ = random_problem(n, k, rng)
    A0 = rng.dirichlet(np.ones(k), size=n).T
    ops = operands(K, B, A0)
    t1 = ops["t1"].toarray().astype(np.float64)
    t2 = ops["k2b"].toarray().astype(np.float64)
    Bf = ops["b"].toarray().astype(np.float64)
    for j in range(n):
        for t in range(T):
            # state a_t from the oracle itself (t steps), pick from step t
            tr_t = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, t + 1,
                                       cells=[j])
            a = ops["a_prev_t"].toarray()[j].astype(np.float64) if t == 0 else \
                oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, t,
                                    cells=[j]).a[0]
            idx = tr_t.pick[0, t]
            g = t1 @ a - t2[j]
            gap = float(g @ a - g[idx])
            assert gap >= -1e-12
            assert gap >= float(np.max(g @ a - g)) - 1e-12       # the best vertex
            d = -a.copy()
            d[idx] += 1.0
            curv = float(d @ t1 @ d)
            if curv <= 0:
                continue
            gam = min(1.0, max(0.0, gap / curv))
            Acur = A0.copy()
            Acur[:, j] = a
            Anew = Acur.copy()
            Anew[:, j] = a + gam * d
            f0, f1 = dense.objective(K, Bf, Acur), dense.objective(K, Bf, Anew)
            assert f1 <= f0 + 1e-12
            if gap > 1e-9:
                assert f1 < f0


# --------------------------------------------------------------------------
# P4: the RSS without forming K B A
# --------------------------------------------------------------------------

def test_p4_rss_closed_form():
    rng = np.random.default_rng(41)
    for n, k in [(5, 2), (12, 4), (30, 7)]:
        K, B, A = random_problem(n, k, rng)
        assert abs(dense.rss_closed_form(K, B, A) - dense.objective(K, B, A)) <= \
            1e-12 * max(1.0, dense.objective(K, B, A))


# --------------------------------------------------------------------------
# P5: worked example, K = I (n = 4, k = 2, T = 50)
# --------------------------------------------------------------------------

def identity_example():
    n, k = 4, 2
    K = np.eye(n)
    B = np.zeros((n, k))
    B[0, 0] = 1.0
    B[1, 1] = 1.0
    A = np.full((k, n), 0.5)
    return K, B, A, operands(K, B, A)


def test_p5_identity_kernel_a_update():
    K, B, A, ops = identity_example()
    T = 50
    tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], 4, 2, T)
    # t1 = I and t2_j = B[j, :], so g = a - B[j, :].
    # cell 0: picks 0 and stays e_0 (every later step is the 0-0 tie -> 0)
    assert tr.pick[0].tolist() == [0] * T
    np.testing.assert_array_equal(tr.a[0], [1.0, 0.0])
    # cell 1: picks 1, then the exact 0-0 tie goes to 0, then 1 forever;
    # a_0 = (2/3) prod_{u=2}^{t} u/(u+2) = 4 / ((t+1)(t+2)) after step t
    assert tr.pick[1].tolist() == [1, 0] + [1] * (T - 2)
    a0 = Fraction(4, T * (T + 1))
    np.testing.assert_allclose(tr.a[1], [float(a0), float(1 - a0)], rtol=0, atol=1e-15)
    # cells 2, 3: B row is zero, g = a; step 0 is the exact tie (1/2, 1/2) -> 0,
    # then the picks alternate, giving 25/51 and 26/51
    for j in (2, 3):
        assert tr.pick[j].tolist() == [t % 2 for t in range(T)]
        np.testing.assert_allclose(tr.a[j], [25 / 51, 26 / 51], rtol=0, atol=1e-15)
    # step 0 of cells 2, 3 is an exact tie: runner-up equals the minimum
    assert tr.g_min[2, 0] == tr.g_second[2, 0] == 0.5


def test_p5_identity_kernel_b_argmin():
    K, B, A, ops = identity_example()
    res = oracle.fw_b_argmin(ops["k2b"], ops["aat"], ops["k2at"], ops["b"], 4, 2)
    # AA^T = [[1, 1], [1, 1]], so G rows are (1/2, 1/2), (1/2, 1/2), (-1/2, -1/2), (-1/2, -1/2)
    np.testing.assert_array_equal(res.val, [-0.5, -0.5])
    np.testing.assert_array_equal(res.row, [2, 2])         # exact tie between rows 2, 3
    np.testing.assert_array_equal(res.second, [-0.5, -0.5])
    assert res.gap == 1.0


# --------------------------------------------------------------------------
# P6: special cases that reduce to a library routine
# --------------------------------------------------------------------------

def test_p6_single_archetype():
    n, k = 6, 1
    t1 = W.dense_to_csr(np.array([[2.0]]))
    k2b = W.dense_to_csr(np.arange(1, n + 1, dtype=np.float32)[:, None])
    ap = W.dense_to_csr(np.ones((n, 1)))
    tr = oracle.fw_a_columns(t1, k2b, ap, n, k, 5)
    assert np.all(tr.pick == 0)
    np.testing.assert_array_equal(tr.a, np.ones((n, 1)))
    assert np.all(np.isinf(tr.g_second))


def test_p6_single_step_is_sparse_matvec_then_argmin(c1):
    w = c1
    tr = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, 1)
    # scipy sparse product + numpy argmin (first minimum)
    G = (w.t1.astype(np.float64) @ w.a_prev_t.astype(np.float64).T).toarray() \
        - w.k2b.astype(np.float64).toarray().T
    want = np.argmin(G, axis=0)
    mins = G[want, np.arange(w.n)]
    np.testing.assert_allclose(tr.g_min[:, 0], mins, rtol=0, atol=1e-12)
    # indices agree wherever the minimum is not an f64-rounding near tie
    srt = np.sort(G, axis=0)
    clear = (srt[1] - srt[0]) > 1e-12 * np.maximum(1, np.abs(srt[0]))
    assert np.array_equal(tr.pick[clear, 0], want[clear])
    # exact ties in G (structural zeros) must resolve to the lowest index
    exact = srt[1] == srt[0]
    assert np.array_equal(tr.pick[exact, 0], want[exact])
    for j in range(w.n):
        e = np.zeros(w.k)
        e[want[j]] = 1.0
        if clear[j] or exact[j]:
            assert np.array_equal(tr.a[j], e)


def test_p6_page_identity_tie_breaks_to_row_zero():
    cfg = json.load(open(os.path.join(GOLDEN, "page_fixtures.json")))["tie_break"]
    n, k = cfg["n"], cfg["k"]
    t1 = np.eye(k, dtype=np.float32)
    k2b = np.tile(-1.0 - np.arange(k, dtype=np.float32), (n, 1))
    zero = sp.csr_matrix((n, k), dtype=np.float32)
    res = oracle.fw_b_argmin(W.dense_to_csr(k2b), W.dense_to_csr(t1), zero, zero, n, k)
    np.testing.assert_array_equal(res.row, np.zeros(k))
    np.testing.assert_array_equal(res.val, -1.0 - np.arange(k))


def page_problem(n, k):
    fx = json.load(open(os.path.join(GOLDEN, "page_fixtures.json")))["fixture"]["operands"]
    k2b = W.page_fixture(n * k, *fx["k2b"]).reshape(n, k)
    t1 = W.page_fixture(k * k, *fx["t1"]).reshape(k, k)
    t2 = W.page_fixture(n * k, *fx["t2"]).reshape(n, k)
    b = W.page_fixture(n * k, *fx["b"]).reshape(n, k)
    return k2b, t1, t2, b


def test_p6_page_empty_rows_keep_competing():
    cfg = json.load(open(os.path.join(GOLDEN, "page_fixtures.json")))["empty_rows"]
    n, k = cfg["n"], cfg["k"]
    k2b, t1, t2, b = page_problem(n, k)
    k2b[::cfg["blank_every"]] = 0.0
    res = oracle.fw_b_argmin(W.dense_to_csr(k2b), W.dense_to_csr(t1), W.dense_to_csr(t2),
                             W.dense_to_csr(b), n, k)
    G = k2b.astype(np.float64) @ t1.astype(np.float64) - t2.astype(np.float64)
    np.testing.assert_array_equal(res.row, np.argmin(G, axis=0))
    np.testing.assert_allclose(res.val, G.min(axis=0), rtol=0, atol=1e-12)
    # a blanked row still has a gradient: exactly -t2
    rows = np.repeat(np.arange(0, n, cfg["blank_every"]), k)
    cols = np.tile(np.arange(k), rows.shape[0] // k)
    g, _ = oracle.fw_b_grad_at(W.dense_to_csr(k2b), W.dense_to_csr(t1), W.dense_to_csr(t2), n, k,
                               rows, cols)
    np.testing.assert_array_equal(g, -t2[rows, cols].astype(np.float64))


# --------------------------------------------------------------------------
# P7: the page's fixtures and shapes, against the dense form of its CPU scan
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(40, 7), (257, 33), (1000, 130), (3000, 300), (300, 1100)])
def test_p7_page_fixtures(n, k):
    k2b, t1, t2, b = page_problem(n, k)
    res = oracle.fw_b_argmin(W.dense_to_csr(k2b), W.dense_to_csr(t1), W.dense_to_csr(t2),
                             W.dense_to_csr(b), n, k)
    val, idx, gap, G = dense.fw_b_argmin(k2b, t1, t2, b)
    np.testing.assert_allclose(res.val, val, rtol=1e-12, atol=1e-12)
    srt = np.sort(G, axis=0)
    tie = (srt[1] - srt[0]) <= 1e-12 * np.maximum(1.0, np.abs(srt[0]))
    assert np.array_equal(res.row[~tie], idx[~tie])
    assert np.all(G[res.row[tie], np.flatnonzero(tie)] - srt[0][tie] <= 1e-12 * np.maximum(1.0, np.abs(srt[0][tie])))
    np.testing.assert_allclose(res.second, srt[1], rtol=1e-12, atol=1e-12)
    assert abs(res.gap - gap) <= 1e-9 * max(1.0, abs(gap))
    # row scale: max |(K2B t1)[i, :]| and |t2[i, :]|
    P = k2b.astype(np.float64) @ t1.astype(np.float64)
    want_scale = np.maximum(np.abs(P).max(axis=1), np.abs(t2).max(axis=1))
    np.testing.assert_allclose(res.row_scale, want_scale, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P8: C oracle against the dense numpy form on a whole workload
# --------------------------------------------------------------------------

def test_p8_a_update_matches_dense_on_c1(c1):
    w = c1
    tr = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T)
    A, picks = dense.fw_a_columns(w.t1.toarray(), w.k2b.toarray(), w.a_prev_t.toarray().T, w.T)
    same = np.all(tr.pick == picks, axis=1)
    # every cell whose trajectory never met a rounding-level near tie agrees
    near = np.any((tr.g_second - tr.g_min) <= 1e-12 * np.maximum(1.0, tr.g_scale), axis=1) & \
        ~np.all(tr.g_second == tr.g_min, axis=1)
    assert np.all(same | near)
    assert same.mean() > 0.99
    np.testing.assert_allclose(tr.a[same], A.T[same], rtol=0, atol=1e-12)


def test_p8_b_argmin_matches_dense_on_c2():
    w = W.make("c2")
    res = oracle.fw_b_argmin(w.k2b, w.aat, w.k2at, w.b, w.n, w.k)
    val, idx, gap, G = dense.fw_b_argmin(w.k2b.toarray(), w.aat.toarray(), w.k2at.toarray(),
                                         w.b.toarray())
    np.testing.assert_allclose(res.val, val, rtol=1e-12, atol=1e-14)
    srt = np.sort(G, axis=0)
    clear = (srt[1] - srt[0]) > 1e-12 * np.maximum(1.0, np.abs(srt[0]))
    assert np.array_equal(res.row[clear], idx[clear])
    assert abs(res.gap - gap) <= 1e-10 * max(1.0, abs(gap))


# --------------------------------------------------------------------------
# trace replay and the B step
# --------------------------------------------------------------------------

def test_force_replays_own_trajectory_and_reports_taken_value(c1):
    w = c1
    cells = np.arange(0, 200, 3)
    tr = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells)
    rep = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells,
                              force=tr.pick.astype(np.int64))
    np.testing.assert_array_equal(rep.a, tr.a)
    np.testing.assert_array_equal(rep.g_taken, tr.g_min)
    # forcing another index changes the state and g_taken is g at that index
    alt = tr.pick.astype(np.int64).copy()
    alt[:, 0] = (alt[:, 0] + 1) % w.k
    r2 = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, 1, cells=cells, force=alt[:, :1])
    t1 = w.t1.toarray().astype(np.float64)
    for r, j in enumerate(cells):
        a = w.a_prev_t.toarray()[j].astype(np.float64)
        g = t1 @ a - w.k2b.toarray()[j].astype(np.float64)
        assert abs(r2.g_taken[r, 0] - g[alt[r, 0]]) < 1e-12
        e = np.zeros(w.k)
        e[alt[r, 0]] = 1.0
        assert np.array_equal(r2.a[r], e)


def test_b_apply_matches_convex_step():
    rng = np.random.default_rng(71)
    n, k, cap_b = 40, 6, 5
    B = np.zeros((n, k), np.float32)
    for c in range(k):
        sup = rng.choice(n, size=rng.integers(1, 4), replace=False)
        B[sup, c] = rng.dirichlet(np.ones(sup.shape[0]))
    idx, val, cnt = W.bt_padded(W.dense_to_csr(B), cap_b)
    arg = rng.integers(0, n, size=k).astype(np.uint32)
    arg[0] = idx[0, 0]                               # one column re-selects a present cell
    gam = 2.0 / 7.0
    oi, ov, oc = oracle.fw_b_apply(idx, val, cnt, arg, gam)
    want = (1 - gam) * B.astype(np.float64)
    want[arg, np.arange(k)] += gam
    for c in range(k):
        got = np.zeros(n)
        got[oi[c, :oc[c]]] = ov[c, :oc[c]]
        np.testing.assert_allclose(got, want[:, c], rtol=0, atol=1e-15)
        assert np.all(np.diff(oi[c, :oc[c]].astype(np.int64)) > 0)      # still ascending
        assert abs(ov[c, :oc[c]].sum() - 1.0) < 1e-6
    # a full row is an error, not a silent drop
    full_idx = np.tile(np.arange(cap_b, dtype=np.uint32), (k, 1))
    full_val = np.full((k, cap_b), 1.0 / cap_b)
    with pytest.raises(RuntimeError):
        oracle.fw_b_apply(full_idx, full_val, np.full(k, cap_b, np.uint32),
                          np.full(k, n - 1, np.uint32), gam)


# --------------------------------------------------------------------------
# P9: the pruning + renormalisation variant of the A update (the page's
# `fw_columns_a_gpu` with `pruning`, and `A_RENORM_FLOOR`)
# --------------------------------------------------------------------------

def _dense(m):
    return np.asarray(m.todense(), np.float64)


def _prune_ref(a, thr):
    """Drop-and-renormalise written out on one dense column (numpy)."""
    a = a.copy()
    drop = (a != 0.0) & (np.abs(a) <= thr)
    a[drop] = 0.0
    tot = a.sum()
    if tot > 1e-15:
        a = a * (1.0 / tot)
    return a, int(drop.sum())


def test_p9_threshold_zero_only_renormalises(c1):
    # nothing can drop at threshold 0 (the weights are >= 0 and 0 is exempt),
    # and a column that sums to 1 is renormalised by a factor 1 +- rounding
    w = c1
    r0 = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T)
    r1 = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, prune=0.0)
    assert r1.drops.sum() == 0
    np.testing.assert_array_equal(r0.pick, r1.pick)
    np.testing.assert_allclose(r1.a, r0.a, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", ["c1", "empty"])
def test_p9_threshold_above_one_drops_everything(case, c1):
    # every weight is <= 1, so every step ends with a = 0 (the sum is 0 and the
    # renormalisation is skipped); the gradient from step 1 on is -t2_j, whose
    # lowest argmin is the lowest column holding the row's maximum (column 0
    # for an empty K2B row)
    if case == "c1":
        w = c1
    else:
        w = W.random_workload(90, 9, s_a=3, seed=41, empty_k2b_every=4)
    r = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, prune=2.0)
    r0 = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, 1)
    np.testing.assert_array_equal(r.pick[:, 0], r0.pick[:, 0])
    t2 = _dense(w.k2b)
    want = np.argmin(-t2, axis=1)   # numpy's argmin returns the first minimum
    for t in range(1, w.T):
        np.testing.assert_array_equal(r.pick[:, t], want)
    assert np.all(r.a == 0.0)
    assert np.all(r.drops >= 1)


def _first_drop_cases():
    rng = np.random.default_rng(9)
    out = []
    for seed in range(8):
        w = W.random_workload(16, 6, t1_per_row=4, k2b_per_row=3, s_a=3, seed=100 + seed, T=24)
        out.append((w, 0.0371 + 0.01 * rng.random()))
    return out


def test_p9_drops_and_renormalisation_follow_the_unpruned_state():
    # Up to the first step whose updated weights include one at or below the
    # threshold, the pruned run is the plain run (renormalised by 1 +- eps);
    # at that step exactly those weights drop and the rest is divided by its
    # sum; the next pick is the argmin of the dense gradient of that column.
    checked = 0
    for w, thr in _first_drop_cases():
        t1, t2 = _dense(w.t1), _dense(w.k2b)
        for j in range(w.n):
            cells = np.array([j])
            prev = _dense(w.a_prev_t)[j]
            # unpruned weights after every step, from runs of length 1..T
            states = [oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, t + 1,
                                          cells=cells).a[0] for t in range(w.T)]
            rp = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells,
                                     prune=thr)
            td = next((t for t, a in enumerate(states)
                       if np.any((a != 0) & (np.abs(a) <= thr))), None)
            if td is None or td + 1 >= w.T:
                continue
            a = states[td]
            nz = a[a != 0]
            if np.min(np.abs(np.abs(nz) - thr)) < 1e-9:
                continue  # a decision on the threshold itself: not a fair case
            ru = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells)
            np.testing.assert_array_equal(rp.pick[0, :td + 1], ru.pick[0, :td + 1])
            assert np.all(rp.drops[0, :td] == 0)
            want_a, nd = _prune_ref(a, thr)
            assert rp.drops[0, td] == nd >= 1
            got = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, td + 1, cells=cells,
                                      prune=thr).a[0]
            np.testing.assert_allclose(got, want_a, rtol=0, atol=1e-12)
            g = t1 @ want_a - t2[j]
            srt = np.sort(g)
            if srt.shape[0] > 1 and srt[1] - srt[0] < 1e-9:
                continue  # tie: the order of rounding decides
            assert rp.pick[0, td + 1] == int(np.argmin(g))
            checked += 1
    assert checked >= 12


def test_p9_invariants_after_every_prefix(c1):
    # after any number of steps: weights >= 0, none in (0, threshold], and the
    # column sums to 1 unless everything was dropped
    w = c1
    thr = 0.0213
    cells = np.arange(0, w.n, 37)
    for T in (1, 2, 7, 19, 50):
        r = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, T, cells=cells, prune=thr)
        assert np.all(r.a >= 0.0)
        assert not np.any((r.a > 0.0) & (r.a <= thr))
        s = r.a.sum(axis=1)
        assert np.all((np.abs(s - 1.0) < 1e-12) | (s == 0.0))


# --------------------------------------------------------------------------
# P10: the full Frank-Wolfe duality gap of both updates (g and G without the
# factor 2, as on the page): <g, a> - min_c g[c] for an A column, and
# sum(B * G) - sum_c min_i G[i, c] for B
# --------------------------------------------------------------------------

def test_p10_identity_kernel_gaps_closed_form():
    K, B, A, ops = identity_example()
    T = 50
    tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], 4, 2, T)
    gap = tr.fw_gap
    # g = a - B[j, :]. Cell 0: a_prev = (1/2, 1/2) gives g = (-1/2, 1/2) and
    # gap 1/2; after step 0, a = e_0 is optimal and every gap is 0.
    np.testing.assert_allclose(gap[0], [0.5] + [0.0] * (T - 1), rtol=0, atol=1e-15)
    # Cell 1: 1/2, then 0 at e_1, then 8/9 at (2/3, 1/3); from step 2 on
    # a_0 = x = 4/(t(t+1)) and g = (x, -x), so the gap is 2 x^2.
    want1 = [0.5, 0.0] + [2.0 * (4.0 / (t * (t + 1))) ** 2 for t in range(2, T)]
    np.testing.assert_allclose(gap[1], want1, rtol=1e-13, atol=1e-15)
    assert abs(gap[1, 2] - 8 / 9) < 1e-15
    # Cells 2, 3: g = a. Step 0 is the optimum (1/2, 1/2): gap 0. After an
    # odd number m of steps a = ((m+1)/(2m), (m-1)/(2m)), gap (m+1)/(2m^2);
    # after an even m >= 2, a = (m/(2(m+1)), (m+2)/(2(m+1))), gap
    # (m+2)/(2(m+1)^2).
    want = [0.0] + [(m + 1) / (2 * m * m) if m % 2 else (m + 2) / (2 * (m + 1) ** 2)
                    for m in range(1, T)]
    for j in (2, 3):
        np.testing.assert_allclose(gap[j], want, rtol=1e-13, atol=1e-15)
    assert abs(gap[2, T - 1] - 25 / 2401) < 1e-15
    # B: G rows (1/2, 1/2) x 2 and (-1/2, -1/2) x 2, B = [e_0, e_1]:
    # sum(B * G) = 1 and each column's minimum is -1/2, so the full gap is 2
    res = oracle.fw_b_argmin(ops["k2b"], ops["aat"], ops["k2at"], ops["b"], 4, 2)
    assert res.fw_gap == 2.0


def test_p10_a_gap_is_the_steepest_vertex_descent_of_the_objective():
    # gap = max over vertices e_v of -d/de f(A with column j moved towards e_v),
    # halved (the page drops the factor 2), from central differences of
    # ||K - K B A||^2 itself (exact up to rounding: f is quadratic in A)
    rng = np.random.default_rng(101)
    n, k, T = 7, 4, 5
    K, B, A0 = dyadic_problem(n, k, rng)
    ops = operands(K, B, A0)
    Bf = ops["b"].toarray().astype(np.float64)
    tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, T)
    h = 1e-3
    checked = 0
    for j in range(n):
        for t in range(T):
            a = ops["a_prev_t"].toarray()[j].astype(np.float64) if t == 0 else \
                oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, t,
                                    cells=[j]).a[0]
            Acur = ops["a_prev_t"].toarray().T.astype(np.float64)
            Acur[:, j] = a
            best = -np.inf
            for v in range(k):
                d = -a.copy()
                d[v] += 1.0
                Ap, Am = Acur.copy(), Acur.copy()
                Ap[:, j] += h * d
                Am[:, j] -= h * d
                slope = (dense.objective(K, Bf, Ap) - dense.objective(K, Bf, Am)) / (2 * h)
                best = max(best, -0.5 * slope)
            assert abs(tr.fw_gap[j, t] - best) <= 1e-8 * max(1.0, abs(best)), (j, t)
            checked += 1
    assert checked == n * T


def _simplex_qp_min(Q, c):
    """min 0.5 a^T Q a - c^T a over the simplex, Q positive semidefinite, by
    enumerating supports: on each support the KKT system is linear; every
    feasible solution is a candidate and the minimiser is one of them."""
    import itertools
    k = Q.shape[0]
    best = np.inf
    for r in range(1, k + 1):
        for S in itertools.combinations(range(k), r):
            S = list(S)
            M = np.zeros((r + 1, r + 1))
            M[:r, :r] = Q[np.ix_(S, S)]
            M[:r, r] = 1.0
            M[r, :r] = 1.0
            rhs = np.concatenate([c[S], [1.0]])
            sol = np.linalg.lstsq(M, rhs, rcond=None)[0]
            aS = sol[:r]
            if np.any(aS < -1e-12) or abs(aS.sum() - 1.0) > 1e-9:
                continue
            a = np.zeros(k)
            a[S] = np.maximum(aS, 0.0)
            a /= a.sum()
            best = min(best, 0.5 * a @ Q @ a - c @ a)
    return best


def test_p10_a_gap_bounds_the_suboptimality():
    # weak duality: q(a_t) - min_simplex q <= gap_t with q(a) = a^T t1 a / 2 -
    # t2_j^T a, whose gradient is the page's g; t1 = B^T K^2 B is PSD
    rng = np.random.default_rng(102)
    n, k, T = 9, 5, 12
    K, B, A0 = random_problem(n, k, rng)
    ops = operands(K, B, A0)
    t1 = ops["t1"].toarray().astype(np.float64)
    t2 = ops["k2b"].toarray().astype(np.float64)
    tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, T)
    for j in range(n):
        qstar = _simplex_qp_min(t1, t2[j])
        for t in range(T):
            a = ops["a_prev_t"].toarray()[j].astype(np.float64) if t == 0 else \
                oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, t,
                                    cells=[j]).a[0]
            sub = 0.5 * a @ t1 @ a - t2[j] @ a - qstar
            assert sub >= -1e-12
            assert tr.fw_gap[j, t] >= sub - 1e-12, (j, t, tr.fw_gap[j, t], sub)


def test_p10_a_gap_vertex_optimum_is_zero():
    # t1 = I, t2 = 5 e_0: from e_0 the gradient is -4 e_0 (gap 0); from e_1 it
    # is e_1 - 5 e_0 (gap 1 - (-5) = 6)
    k = 3
    t1 = sp.identity(k, format="csr", dtype=np.float32)
    k2b = sp.csr_matrix(np.array([[5.0, 0, 0], [5.0, 0, 0]], np.float32))
    ap = sp.csr_matrix(np.array([[1.0, 0, 0], [0, 1.0, 0]], np.float32))
    tr = oracle.fw_a_columns(t1, k2b, ap, 2, k, 3)
    np.testing.assert_array_equal(tr.fw_gap[0], [0.0, 0.0, 0.0])
    assert tr.fw_gap[1, 0] == 6.0


def test_p10_b_full_gap_by_vertex_enumeration():
    # max over every vertex matrix S (one-hot columns) of <G, B - S>, with G
    # from the closed form 2 (K^2 B A A^T - K^2 A^T) / 2 of the dense module
    import itertools
    rng = np.random.default_rng(103)
    for n, k in ((4, 2), (5, 3), (6, 2)):
        K, B, A = random_problem(n, k, rng)
        ops = operands(K, B, A)
        Bf = ops["b"].toarray().astype(np.float64)
        # the operands are f32: G from the f32-rounded products, as the oracle sees them
        G = (ops["k2b"].toarray().astype(np.float64) @ ops["aat"].toarray().astype(np.float64)
             - ops["k2at"].toarray().astype(np.float64))
        best = -np.inf
        for rows in itertools.product(range(n), repeat=k):
            S = np.zeros((n, k))
            S[list(rows), list(range(k))] = 1.0
            best = max(best, float(np.sum(G * (Bf - S))))
        res = oracle.fw_b_argmin(ops["k2b"], ops["aat"], ops["k2at"], ops["b"], n, k)
        assert abs(res.fw_gap - best) <= 1e-12 * max(1.0, abs(best)), (n, k, res.fw_gap, best)
        assert res.fw_gap >= 0.0
        # and G itself agrees with half the closed-form gradient of the objective
        # on the exact (f64) problem up to the f32 rounding of the operands
        np.testing.assert_allclose(G, dense.grad_b(K, B, A) / 2, rtol=0, atol=1e-5)


def test_p10_a_gap_on_a_forced_trajectory_uses_the_true_minimum():
    # trace replay: the update follows forced (non-optimal) picks, and the
    # gap at each iterate is still measured against its best vertex
    rng = np.random.default_rng(104)
    n, k, T = 5, 4, 6
    K, B, A0 = dyadic_problem(n, k, rng)
    ops = operands(K, B, A0)
    Bf = ops["b"].toarray().astype(np.float64)
    force = np.array([[(t + j) % k for t in range(T)] for j in range(n)], np.int64)
    tr = oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, T, force=force)
    assert np.any(tr.pick != force)
    h = 1e-3
    for j in range(n):
        for t in range(T):
            a = ops["a_prev_t"].toarray()[j].astype(np.float64) if t == 0 else \
                oracle.fw_a_columns(ops["t1"], ops["k2b"], ops["a_prev_t"], n, k, t, cells=[j],
                                    force=force[j:j + 1, :t]).a[0]
            Acur = ops["a_prev_t"].toarray().T.astype(np.float64)
            Acur[:, j] = a
            best = -np.inf
            for v in range(k):
                d = -a.copy()
                d[v] += 1.0
                Ap, Am = Acur.copy(), Acur.copy()
                Ap[:, j] += h * d
                Am[:, j] -= h * d
                slope = (dense.objective(K, Bf, Ap) - dense.objective(K, Bf, Am)) / (2 * h)
                best = max(best, -0.5 * slope)
            assert abs(tr.fw_gap[j, t] - best) <= 1e-8 * max(1.0, abs(best)), (j, t)
