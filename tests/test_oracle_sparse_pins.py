"""Pins of oracle/sparse.py (the operand construction and the RSS) to things
other than itself: brute-force loops over tiny matrices, dense numpy
products, the brute-force objective ||K - K B A||^2, closed forms, and the
workload generator's own f64 products (C, in workloads/_spgemm.c).

The method (bixverse-rs 0.6.4, ``seacells_kernels.rs``, module doc): the
objective f(A, B) = ||K - K B A||_F^2 and its operands K^2 B, B^T K^2 B,
A A^T, K^2 A^T; the host routines ``csr_matmul_csr`` and
``transpose_sparse`` named in the ``lower_bound`` doc.
"""
import numpy as np
import pytest
import scipy.sparse as sp

from oracle import dense
from oracle import sparse as S
import workloads as W


def rand_csr(rng, m, q, density, signed=True, zeros=0.1, empty_rows=(), dtype=np.float32):
    """Random CSR with explicit zero entries and chosen empty rows."""
    mask = rng.random((m, q)) < density
    mask[list(empty_rows), :] = False
    vals = rng.uniform(0.1, 1.0, size=(m, q))
    if signed:
        vals *= rng.choice([-1.0, 1.0], size=(m, q))
    vals[rng.random((m, q)) < zeros] = 0.0
    rows, cols = np.nonzero(mask)
    out = sp.csr_matrix((vals[rows, cols].astype(dtype), (rows, cols)), shape=(m, q))
    out.sort_indices()
    return out


def brute_product(a, b):
    """{(i, c): (sum, sum of |.|, count)} by three plain loops."""
    a, b = sp.csr_matrix(a), sp.csr_matrix(b)
    out = {}
    for i in range(a.shape[0]):
        for e in range(a.indptr[i], a.indptr[i + 1]):
            j, av = int(a.indices[e]), float(a.data[e])
            for t in range(b.indptr[j], b.indptr[j + 1]):
                c, bv = int(b.indices[t]), float(b.data[t])
                s, sa, n = out.get((i, c), (0.0, 0.0, 0))
                out[(i, c)] = (s + av * bv, sa + abs(av * bv), n + 1)
    return out


def as_dict(p: S.Product):
    out = {}
    for i in range(p.shape[0]):
        for e in range(p.indptr[i], p.indptr[i + 1]):
            out[(i, int(p.indices[e]))] = (p.value[e], p.abs_value[e], int(p.terms[e]))
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matmul_equals_brute_force_loops(seed):
    rng = np.random.default_rng(seed)
    a = rand_csr(rng, 9, 7, 0.4, empty_rows=(2,))
    b = rand_csr(rng, 7, 11, 0.35, empty_rows=(4,))
    got, want = as_dict(S.matmul(a, b)), brute_product(a, b)
    assert got.keys() == want.keys()
    for key, (s, sa, n) in want.items():
        gs, gsa, gn = got[key]
        assert gn == n
        assert abs(gs - s) <= 1e-15 * sa
        assert abs(gsa - sa) <= 1e-15 * sa
    p = S.matmul(a, b)
    for i in range(p.shape[0]):  # ascending columns in every row
        assert np.all(np.diff(p.indices[p.indptr[i]:p.indptr[i + 1]]) > 0)


def test_matmul_matches_dense_numpy_product():
    rng = np.random.default_rng(7)
    a = rand_csr(rng, 60, 80, 0.1, empty_rows=(0, 59))
    b = rand_csr(rng, 80, 70, 0.1, empty_rows=(3,))
    p = S.matmul(a, b)
    d = a.toarray().astype(np.float64) @ b.toarray().astype(np.float64)
    got = p.csr().toarray()
    np.testing.assert_allclose(got, d, rtol=0, atol=1e-14)
    # the pattern is the product of the patterns: where no product meets, no entry
    reach = (a.toarray() != 0) | _explicit(a)
    reach_b = (b.toarray() != 0) | _explicit(b)
    meets = (reach.astype(np.int64) @ reach_b.astype(np.int64)) > 0
    stored = np.zeros_like(meets)
    rows = np.repeat(np.arange(p.shape[0]), np.diff(p.indptr))
    stored[rows, p.indices] = True
    assert np.array_equal(stored, meets)


def _explicit(m):
    """Dense mask of the stored positions (explicit zeros included)."""
    out = np.zeros(m.shape, bool)
    rows = np.repeat(np.arange(m.shape[0]), np.diff(m.indptr))
    out[rows, m.indices] = True
    return out


def test_matmul_keeps_cancelled_sums_and_explicit_zeros():
    a = sp.csr_matrix(np.array([[1.0, -1.0], [0.0, 2.0]]))
    b = sp.csr_matrix(np.array([[3.0], [3.0]]))
    p = S.matmul(a, b)
    assert list(p.indptr) == [0, 1, 2] and list(p.indices) == [0, 0]
    assert list(p.value) == [0.0, 6.0] and list(p.terms) == [2, 1]
    assert list(p.abs_value) == [6.0, 6.0]
    # an explicitly stored zero still reaches its columns
    z = sp.csr_matrix((np.array([0.0]), np.array([1]), np.array([0, 1])), shape=(1, 2))
    q = S.matmul(z, sp.csr_matrix(np.array([[1.0, 0.0], [0.0, 5.0]])))
    assert list(q.indices) == [1] and list(q.value) == [0.0] and list(q.terms) == [1]


def test_matmul_rows_is_a_row_slice():
    rng = np.random.default_rng(3)
    a = rand_csr(rng, 30, 20, 0.2)
    b = rand_csr(rng, 20, 25, 0.2)
    full = S.matmul(a, b).csr().toarray()
    rows = [0, 5, 29, 5]
    np.testing.assert_array_equal(S.matmul_rows(a, b, rows).csr().toarray(), full[rows])


@pytest.mark.parametrize("seed", [0, 1])
def test_transpose_equals_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    a = rand_csr(rng, 13, 9, 0.3, empty_rows=(0, 6))
    t = S.transpose(a)
    assert t.shape == (9, 13) and t.nnz == a.nnz  # explicit zeros kept
    want = [[] for _ in range(9)]
    for i in range(13):  # rows in ascending order, so every list comes out sorted
        for e in range(a.indptr[i], a.indptr[i + 1]):
            want[int(a.indices[e])].append((i, float(a.data[e])))
    for c in range(9):
        got = [(int(t.indices[e]), float(t.data[e])) for e in range(t.indptr[c], t.indptr[c + 1])]
        assert got == want[c]
    np.testing.assert_array_equal(t.toarray(), a.toarray().T)
    back = S.transpose(t)
    assert np.array_equal(back.indptr, a.indptr) and np.array_equal(back.indices, a.indices)
    assert np.array_equal(back.data, a.data)


def test_dot_matches_dense_sum_and_closed_forms():
    rng = np.random.default_rng(5)
    x = rand_csr(rng, 40, 30, 0.2, dtype=np.float64)
    y = rand_csr(rng, 40, 30, 0.2, dtype=np.float64)
    assert abs(S.dot(x, y) - float(np.sum(x.toarray() * y.toarray()))) <= 1e-14
    assert abs(S.dot(x, x) - float(np.sum(x.toarray() ** 2))) <= 1e-14
    assert abs(S.dot_abs(x, y) - float(np.sum(np.abs(x.toarray() * y.toarray())))) <= 1e-14
    # disjoint patterns
    e = sp.csr_matrix(np.array([[1.0, 0.0]]))
    f = sp.csr_matrix(np.array([[0.0, 1.0]]))
    assert S.dot(e, f) == 0.0
    with pytest.raises(ValueError):
        S.dot(e, sp.csr_matrix(np.ones((2, 1))))


def random_problem(rng, n, k, knn=4):
    """Symmetric non-negative K with unit diagonal, column-stochastic B (n x k)
    and A (k x n, returned as A^T)."""
    W_ = np.zeros((n, n))
    for i in range(n):
        nb = rng.choice(np.delete(np.arange(n), i), size=knn, replace=False)
        W_[i, nb] = rng.uniform(0.1, 1.0, size=knn)
    K = (W_ + W_.T) / 2 + np.eye(n)
    B = np.zeros((n, k))
    for c in range(k):
        sup = rng.choice(n, size=3, replace=False)
        B[sup, c] = rng.dirichlet(np.ones(3))
    A = np.zeros((k, n))
    for j in range(n):
        sup = rng.choice(k, size=min(2, k), replace=False)
        A[sup, j] = rng.dirichlet(np.ones(sup.size))
    return sp.csr_matrix(K), sp.csr_matrix(B), sp.csr_matrix(A.T)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rss_equals_brute_force_objective(seed):
    rng = np.random.default_rng(20 + seed)
    K, B, At = random_problem(rng, 30, 5)
    brute = dense.objective(K.toarray(), B.toarray(), At.toarray().T)
    assert abs(S.rss(K, B, At) - brute) <= 1e-12 * S.rss_scale(K, B, At)
    assert S.rss(K, B, At) > 0


def test_rss_of_operands_equals_brute_force():
    rng = np.random.default_rng(31)
    K, B, At = random_problem(rng, 25, 4)
    Kd, Bd, Ad = K.toarray(), B.toarray(), At.toarray().T
    k2b = sp.csr_matrix(Kd @ Kd @ Bd)
    t1 = sp.csr_matrix(Bd.T @ Kd @ Kd @ Bd)
    aat = sp.csr_matrix(Ad @ Ad.T)
    val, scale = S.rss_of_operands(K, k2b, At, t1, aat)
    assert abs(val - dense.objective(Kd, Bd, Ad)) <= 1e-12 * scale
    assert abs(scale - S.rss_scale(K, B, At)) <= 1e-12 * scale


def test_rss_closed_forms():
    n = 6
    K = sp.identity(n, format="csr")
    # B = A = I reconstructs K exactly
    I = sp.identity(n, format="csr")
    assert abs(S.rss(K, I, I)) <= 1e-15
    # K = I, one archetype = cell 0, every cell assigned to it: K B A = e_0 1^T,
    # so the residual I - e_0 1^T holds n - 1 entries -1 (row 0 past column 0)
    # and n - 1 diagonal ones (rows 1 ..): squared norm 2 (n - 1)
    B = sp.csr_matrix(([1.0], ([0], [0])), shape=(n, 1))
    At = sp.csr_matrix(np.ones((n, 1)))
    assert abs(S.rss(K, B, At) - 2.0 * (n - 1)) <= 1e-12
    assert abs(dense.objective(K.toarray(), B.toarray(), At.toarray().T) - 2.0 * (n - 1)) <= 1e-12


def test_operands_match_the_generators_products():
    """The generator forms K^2 B, t1, A A^T and K^2 A^T with its own f64
    products (C) from the f64 kernel and rounds them to f32; the oracle
    rebuilds them from the f32 K, B, A^T. They agree to f32 rounding."""
    w = W.make("c1")
    K = W.kernel_matrix(w)
    ops = S.operands(K, w.b, w.a_prev_t)
    for nm, got in (("k2b", ops.k2b), ("t1", ops.t1), ("aat", ops.aat), ("k2at", ops.k2at)):
        ref = getattr(w, nm)
        g = got.csr()
        assert g.shape == ref.shape
        # same pattern (no cancellation: every operand is non-negative)
        assert np.array_equal(g.indptr, ref.indptr) and np.array_equal(g.indices, ref.indices), nm
        rel = np.abs(g.data - ref.data.astype(np.float64)) / got.abs_value
        assert rel.max() <= 2e-6, (nm, rel.max())
    assert np.array_equal(ops.bt.toarray(), w.b.toarray().T)
    assert np.array_equal(ops.a.toarray(), w.a_prev_t.toarray().T)


# --------------------------------------------------------------------------
# sparse add and the vertex matrix
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_add_equals_brute_force(seed):
    rng = np.random.default_rng(60 + seed)
    x = rand_csr(rng, 11, 9, 0.3, empty_rows=(3,))
    y = rand_csr(rng, 11, 9, 0.3, empty_rows=(3, 5))
    alpha, beta = 0.75, -1.5
    got = S.add(alpha, x, beta, y)
    want = {}
    for m, coef in ((x, alpha), (y, beta)):
        for i in range(m.shape[0]):
            for e in range(m.indptr[i], m.indptr[i + 1]):
                key = (i, int(m.indices[e]))
                want[key] = want.get(key, 0.0) + coef * float(m.data[e])
    seen = {}
    for i in range(11):
        cols = got.indices[got.indptr[i]:got.indptr[i + 1]]
        assert np.all(np.diff(cols) > 0)
        for e in range(got.indptr[i], got.indptr[i + 1]):
            seen[(i, int(got.indices[e]))] = float(got.data[e])
    assert seen.keys() == want.keys()  # union of the stored patterns, zeros included
    for key, v in want.items():
        assert abs(seen[key] - v) <= 1e-15
    np.testing.assert_allclose(got.toarray(), alpha * x.toarray().astype(np.float64)
                               + beta * y.toarray().astype(np.float64),
                               rtol=0, atol=1e-15)
    # a cancelling sum stays stored
    c = S.add(1.0, sp.csr_matrix(np.array([[2.0, 0.0]])), 1.0, sp.csr_matrix(np.array([[-2.0, 1.0]])))
    assert c.nnz == 2 and list(c.data) == [0.0, 1.0]


def test_picks_is_the_vertex_matrix():
    idx = np.array([3, 0, 3, 2])
    P = S.picks(idx, 5, 0.25)
    d = np.zeros((5, 4))
    d[idx, np.arange(4)] = 0.25
    np.testing.assert_array_equal(P.toarray(), d)
    assert P.nnz == 4 and list(P.indices[P.indptr[3]:P.indptr[4]]) == [0, 2]


# --------------------------------------------------------------------------
# the B loop
# --------------------------------------------------------------------------

from oracle import b_loop as BL  # noqa: E402


def loop_problem(rng, n, k):
    K, B, At = random_problem(rng, n, k)
    Kd, Bd, Ad = K.toarray(), B.toarray(), At.toarray().T
    aat = Ad @ Ad.T
    k2at = Kd @ Kd @ Ad.T
    return K, B, Ad, sp.csr_matrix(aat), sp.csr_matrix(k2at)


@pytest.mark.parametrize("seed", [0, 1])
def test_b_loop_gradient_is_half_the_objective_gradient(seed):
    rng = np.random.default_rng(70 + seed)
    n, k = 7, 3
    K, B, Ad, aat, k2at = loop_problem(rng, n, k)
    grad = dense.grad_b(K.toarray(), B.toarray(), Ad)  # 2 (K^2 B AA^T - K^2 A^T)
    for r in range(n):
        res = BL.fw_b_loop(K, B, aat, k2at, 1, force=np.full((1, k), r))
        np.testing.assert_allclose(res.g_used[0], grad[r] / 2.0, rtol=0, atol=1e-12)
    res = BL.fw_b_loop(K, B, aat, k2at, 1)
    np.testing.assert_array_equal(res.pick[0], np.argmin(grad, axis=0))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_b_loop_direction_derivative_of_the_objective(seed):
    # f(B) = ||K - K B A||^2 is quadratic in B: the central difference along
    # the Frank-Wolfe direction S - B is exact up to rounding and equals
    # 2 <G, S - B> = 2 (sum_c min_i G[i, c] - sum B * G)
    rng = np.random.default_rng(80 + seed)
    n, k = 8, 3
    K, B, Ad, aat, k2at = loop_problem(rng, n, k)
    res = BL.fw_b_loop(K, B, aat, k2at, 1)
    Kd, Bd = K.toarray(), B.toarray()
    Sv = np.zeros((n, k))
    Sv[res.pick[0], np.arange(k)] = 1.0
    d = Sv - Bd
    eps = 1e-3
    fd = (dense.objective(Kd, Bd + eps * d, Ad) - dense.objective(Kd, Bd - eps * d, Ad)) / (2 * eps)
    want = 2.0 * (res.gmin[0].sum() - res.gap[0])
    assert abs(fd - want) <= 1e-8 * max(1.0, abs(want))
    assert want <= 0.0  # a descent direction (the vertex minimises the linear model)


def test_b_loop_step_weights_closed_form():
    # with gamma_t = 2/(t+2), B_T = sum_t 2(t+1)/(T(T+1)) S(used_t), whatever B_0
    rng = np.random.default_rng(90)
    n, k, T = 9, 4, 7
    K, B, Ad, aat, k2at = loop_problem(rng, n, k)
    res = BL.fw_b_loop(K, B, aat, k2at, T)
    want = np.zeros((n, k))
    for t in range(T):
        want[res.used[t], np.arange(k)] += 2.0 * (t + 1) / (T * (T + 1))
    np.testing.assert_allclose(res.b, want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(res.b.sum(axis=0), 1.0, rtol=0, atol=1e-14)
    Kd = K.toarray()
    np.testing.assert_allclose(res.k2b, Kd @ Kd @ res.b, rtol=0, atol=1e-12)
    # replaying its own picks reproduces the run
    rep = BL.fw_b_loop(K, B, aat, k2at, T, force=res.pick)
    np.testing.assert_array_equal(rep.b, res.b)
    np.testing.assert_array_equal(rep.g_used, res.gmin)


def test_b_loop_identity_kernel_trajectory():
    # K = I, A = 1/2 everywhere (n = 4, k = 2): A A^T = 1, K^2 A^T = 1/2, so
    # G[i, c] = (row sum of B at i) - 1/2 and every step picks the row with
    # the smallest row sum, the lowest on a tie: 2, 0, 1, 3; then
    # B_4 = (2/20, 4/20, 6/20, 8/20) on rows (2, 0, 1, 3) in both columns
    n, k = 4, 2
    K = sp.identity(n, format="csr")
    B = np.zeros((n, k))
    B[0, 0] = B[1, 1] = 1.0
    A = np.full((k, n), 0.5)
    res = BL.fw_b_loop(K, B, sp.csr_matrix(A @ A.T), sp.csr_matrix(A.T), 4)
    assert res.pick.tolist() == [[2, 2], [0, 0], [1, 1], [3, 3]]
    np.testing.assert_array_equal(res.gmin, np.full((4, 2), -0.5))
    np.testing.assert_allclose(res.b, np.array([[0.2, 0.2], [0.3, 0.3], [0.1, 0.1], [0.4, 0.4]]),
                               rtol=0, atol=1e-15)
    # gap at step 0: sum(B * G) = 1 * (1 - 1/2) + 1 * (1 - 1/2) = 1
    assert res.gap[0] == 1.0


def test_b_loop_orientation_with_a_non_symmetric_middle_matrix():
    # the page's G[i, c] = sum_m K^2B[i, m] t1[m, c] - K^2A^T[i, c] holds for
    # any t1 (its own fixtures are not symmetric): brute-force loops
    rng = np.random.default_rng(95)
    n, k = 6, 3
    K, B, Ad, _, k2at = loop_problem(rng, n, k)
    mid = rng.uniform(-1, 1, size=(k, k))
    Kd, Bd, T2 = K.toarray(), B.toarray(), k2at.toarray()
    K2B = Kd @ Kd @ Bd
    for r in range(n):
        res = BL.fw_b_loop(K, B, sp.csr_matrix(mid), k2at, 1, force=np.full((1, k), r))
        for c in range(k):
            g = sum(K2B[r, m] * mid[m, c] for m in range(k)) - T2[r, c]
            assert abs(res.g_used[0, c] - g) <= 1e-12


def test_atoms_to_csr_equals_dense_scatter():
    rng = np.random.default_rng(99)
    n, k, cap = 12, 9, 6
    idx = np.zeros((n, cap), np.int32)
    val = np.zeros((n, cap), np.float32)
    cnt = rng.integers(0, cap + 1, size=n)
    dense_a = np.zeros((n, k))
    for j in range(n):
        cols = rng.choice(k, size=cnt[j], replace=False)  # unique atoms, any order
        w = rng.uniform(0, 1, size=cnt[j]).astype(np.float32)
        w[rng.random(cnt[j]) < 0.3] = 0.0                   # zero weights are dropped
        idx[j, :cnt[j]], val[j, :cnt[j]] = cols, w
        idx[j, cnt[j]:] = 7                                 # slots past the count are ignored
        val[j, cnt[j]:] = 5.0
        dense_a[j, cols] = w
    got = S.atoms_to_csr(idx, val, cnt, k)
    np.testing.assert_array_equal(got.toarray(), dense_a)
    assert got.nnz == int(np.count_nonzero(dense_a))
    for j in range(n):
        assert np.all(np.diff(got.indices[got.indptr[j]:got.indptr[j + 1]]) > 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_b_loop_rows_and_the_a_change_bound(seed):
    # keep_rows returns the rows of K (K B_t) that G_t was read at; a change
    # of every A entry by at most d_a moves those G values by at most the
    # bound the B-loop check adds (brute force on perturbed A)
    from tests import parity
    rng = np.random.default_rng(110 + seed)
    n, k, T = 9, 4, 3
    K, B, Ad, aat, k2at = loop_problem(rng, n, k)
    res = BL.fw_b_loop(K, B, aat, k2at, T, keep_rows=True)
    Kd = K.toarray()
    Bt = B.toarray()
    for t in range(T):
        np.testing.assert_allclose(res.k2b_used[t], (Kd @ Kd @ Bt)[res.used[t]], rtol=0,
                                   atol=1e-12)
        Bt = Bt * (1.0 - 2.0 / (t + 2.0))
        Bt[res.used[t], np.arange(k)] += 2.0 / (t + 2.0)
    d_a = 1e-3
    bound = parity.a_change_bound(K, sp.csr_matrix(Ad.T), res.used, res.k2b_used, d_a)
    worst = 0.0
    for _ in range(20):
        A2 = np.clip(Ad + rng.uniform(-d_a, d_a, size=Ad.shape), 0.0, None)
        rep = BL.fw_b_loop(K, B, sp.csr_matrix(A2 @ A2.T), sp.csr_matrix(Kd @ Kd @ A2.T), T,
                           force=res.used)
        worst = max(worst, float(np.max(np.abs(rep.g_used - res.g_used) / bound)))
    assert worst <= 1.0 + 1e-6
