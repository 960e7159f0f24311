"""Device operand construction (include/seacells_sparse.h) against the f64
oracle (oracle/sparse.py).

Products: the stored pattern must equal the oracle's structural pattern
exactly (integer work), and every value must lie within the rounding bound
of an f32 sum of fused multiply-adds, |c - c*| <= 1.01 * t * 2^-24 * sum|a b|
with t the number of products in the sum (a chained product adds the bound
of its first factor). Transposes are bit-exact. Inner products are f64 sums
of exact f64 products: within 1e-12 of the sum of |x y|. The RSS from device
operands is within 1e-5 of the scale of its cancelling terms.

Shapes cover several column windows (16384 columns each), rows with more
than 2048 outputs (several value windows), rows of a with 2048 entries or
more (split over a block of waves), empty rows on both sides,
explicit zeros and exact cancellation, a ragged last window, one-column and
zero-row operands, and the kNN-kernel workloads (n = 2000, 20000, 100000).
"""
import zlib

import numpy as np
import pytest
import scipy.sparse as sp
import torch

import sparse_archetypal_analysis_amd as saa
from oracle import sparse as S
import workloads as W
from tests.gpu_run import dev, host
from tests.parity import check_product

pytestmark = pytest.mark.gpu


def rand_csr(rng, m, q, per_row, signed=True, zeros=0.05, empty_every=0, dense_rows=()):
    """m x q with about per_row entries per row, explicit zeros, every
    empty_every-th row empty and the rows in dense_rows full."""
    rows, cols = [], []
    for i in range(m):
        if empty_every and i % empty_every == empty_every - 1:
            continue
        if i in dense_rows:
            c = np.arange(q)
        else:
            c = np.unique(rng.integers(0, q, size=per_row))
        rows.append(np.full(c.size, i))
        cols.append(c)
    rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    cols = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    vals = rng.uniform(0.1, 1.0, size=rows.size)
    if signed:
        vals *= rng.choice([-1.0, 1.0], size=rows.size)
    vals[rng.random(rows.size) < zeros] = 0.0
    out = sp.csr_matrix((vals.astype(np.float32), (rows, cols)), shape=(m, q))
    out.sort_indices()
    return out


def product_on_gpu(a, b):
    st = saa.new_status()
    c = saa.csr_matmul(dev(a), dev(b), status=st)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    return host(c)


PRODUCT_CASES = {
    # name: (m, p, q, per_row_a, per_row_b, extra)
    "small": (50, 40, 30, 6, 5, {}),
    "ragged_window": (70, 90, 16384 + 33, 12, 40, {}),
    "three_windows": (40, 300, 40000, 20, 80, {"empty_every_a": 7, "empty_every_b": 5}),
    "wide_rows": (12, 64, 20000, 10, 120, {"dense_rows_a": (0, 5, 11)}),
    "one_column": (100, 30, 1, 5, 1, {}),
    "many_rows": (5000, 300, 700, 4, 6, {"empty_every_a": 11}),
    # one column window (rows pass keeps its bitmaps) and rows of up to 7
    # value windows: their further windows run as units of their own
    "long_rows_kept": (300, 64, 12000, 6, 110, {"dense_rows_a": (0, 7, 150, 299)}),
    # rows of a with 2048 entries or more: a block per row (16 runs of the
    # row's entries) while b has one column window, else one wave per row
    "heavy_rows": (60, 5000, 3000, 20, 8, {"dense_rows_a": (0, 7, 59), "empty_every_b": 9}),
    "heavy_rows_long_outputs": (20, 2500, 16384, 5, 12, {"dense_rows_a": (3, 19)}),
    "heavy_rows_two_windows": (30, 3000, 20000, 10, 6, {"dense_rows_a": (1, 29)}),
}


def test_product_with_more_than_256_scan_tiles():
    # 1.2M rows: the row-pointer scan runs over 293 tiles of 4096 counts
    rng = np.random.default_rng(11)
    m, p, q = 1_200_000, 5000, 300
    nnz_a = 3 * m
    rows = np.repeat(np.arange(m), 3)
    cols = rng.integers(0, p, size=nnz_a)
    a = sp.csr_matrix((rng.uniform(0.1, 1, nnz_a).astype(np.float32), (rows, cols)), shape=(m, p))
    a.sum_duplicates()
    a.sort_indices()
    b = rand_csr(rng, p, q, 2, empty_every=3)
    got = product_on_gpu(a, b)
    check_product(got, S.matmul(a, b), what="1.2M rows")


@pytest.mark.parametrize("case", sorted(PRODUCT_CASES))
def test_product_matches_oracle(case):
    m, p, q, ra, rb, ex = PRODUCT_CASES[case]
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    a = rand_csr(rng, m, p, ra, empty_every=ex.get("empty_every_a", 0),
                 dense_rows=ex.get("dense_rows_a", ()))
    b = rand_csr(rng, p, q, rb, empty_every=ex.get("empty_every_b", 0))
    got = product_on_gpu(a, b)
    want = S.matmul(a, b)
    rel = check_product(got, want, what=case)
    if case in ("wide_rows", "long_rows_kept", "heavy_rows_long_outputs"):
        assert np.diff(got.indptr).max() > 2048  # several value windows per row
    if case.startswith("heavy_rows"):
        assert np.diff(a.indptr).max() >= 2048
    print("\n%s: nnz %d, max error / sum|ab| = %.2e" % (case, got.nnz, rel))


def test_product_rows_at_the_heavy_threshold_and_empty_products():
    # rows of a with 2047 and 2048 entries (one on each side of the
    # block-per-row threshold), a heavy row that meets only empty rows of b,
    # and a heavy row of explicit zeros: the same pattern rule and value bound
    rng = np.random.default_rng(31)
    p, q = 6000, 900
    rows = [np.sort(rng.choice(p - 2100, size=2047, replace=False)),
            np.sort(rng.choice(p - 2100, size=2048, replace=False)),
            np.arange(p - 2100, p),
            np.sort(rng.choice(p, size=3000, replace=False))]
    r = np.concatenate([np.full(c.size, i) for i, c in enumerate(rows)])
    c = np.concatenate(rows)
    v = rng.uniform(0.1, 1.0, size=c.size).astype(np.float32)
    v[r == 3] = 0.0  # products of value 0: their columns stay, as explicit zeros
    a = sp.csr_matrix((v, (r, c)), shape=(4, p))
    a.sort_indices()
    b = rand_csr(rng, p, q, 6, zeros=0.0)
    keep = b.indptr[p - 2100]  # b's last 2100 rows empty
    b = sp.csr_matrix((b.data[:keep], b.indices[:keep],
                       np.minimum(b.indptr, keep)), shape=(p, q))
    assert list(np.diff(a.indptr)) == [2047, 2048, 2100, 3000]
    assert b[p - 2100:].nnz == 0
    got = product_on_gpu(a, b)
    check_product(got, S.matmul(a, b), what="heavy threshold")
    assert got.indptr[3] == got.indptr[2]  # no products: an empty row
    assert got.indptr[4] > got.indptr[3]
    assert np.all(got.data[got.indptr[3]:got.indptr[4]] == 0.0)


@pytest.mark.parametrize("p", [400, 3000])
def test_product_with_kept_bitmaps_equals_recomputed_columns(p):
    # the fill pass reading the rows pass's bitmaps, or marking the columns
    # again, writes the same product bit for bit (p = 3000: the dense rows of
    # a have 3000 entries and go to the heavy-row blocks in both)
    rng = np.random.default_rng(12)
    a = rand_csr(rng, 3000, p, 9, empty_every=7, dense_rows=(3, 1500, 2999))
    b = rand_csr(rng, p, 9000, 30 if p == 400 else 4, empty_every=5)
    da, db = dev(a), dev(b)
    m, q = a.shape[0], b.shape[1]
    outs = []
    for nbytes in (saa.seacells_csr_matmul_workspace(m),
                   saa.seacells_csr_matmul_pattern_workspace(m, q)):
        st = saa.new_status()
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ptr, _ = saa.seacells_csr_matmul_rows(da, db, workspace=ws, status=st)
        torch.cuda.synchronize()
        nnz = int(ptr[-1].item())
        idx = torch.empty(nnz, dtype=torch.int32, device="cuda")
        val = torch.empty(nnz, dtype=torch.float32, device="cuda")
        saa.seacells_csr_matmul_fill(da, db, ptr, idx, val, workspace=ws, status=st)
        torch.cuda.synchronize()
        assert saa.status_flags(st) == []
        outs.append((ptr.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy().view(np.uint32)))
    assert saa.seacells_csr_matmul_pattern_workspace(m, q) > saa.seacells_csr_matmul_workspace(m)
    for x, y in zip(outs[0], outs[1]):
        assert np.array_equal(x, y)
    check_product(host(saa.csr_matmul(da, db)), S.matmul(a, b), what="kept bitmaps")


def test_product_fill_refuses_a_capacity_below_the_true_size():
    rng = np.random.default_rng(13)
    a = rand_csr(rng, 200, 50, 5)
    b = rand_csr(rng, 50, 300, 6)
    da, db = dev(a), dev(b)
    ptr, _ = saa.seacells_csr_matmul_rows(da, db)
    torch.cuda.synchronize()
    nnz = int(ptr[-1].item())
    idx = torch.full((nnz - 1,), -3, dtype=torch.int32, device="cuda")
    val = torch.full((nnz - 1,), 7.0, dtype=torch.float32, device="cuda")
    st = saa.new_status()
    saa.seacells_csr_matmul_fill(da, db, ptr, idx, val, status=st)
    torch.cuda.synchronize()
    assert "OUTPUT_TOO_LARGE" in saa.status_flags(st)
    assert bool((idx == -3).all()) and bool((val == 7.0).all())
    # a bound above the true size is fine (the rows end at the true size)
    st = saa.new_status()
    c = saa.csr_matmul(da, db, status=st, bound=nnz + 50)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    assert c.nnz == nnz + 50 and int(c.row_ptr[-1].item()) == nnz
    exact = saa.csr_trim(c)
    assert exact.nnz == nnz
    check_product(host(exact), S.matmul(a, b), what="bounded output")


def test_product_keeps_cancellation_as_explicit_zero():
    a = sp.csr_matrix((np.array([1.0, -1.0, 2.0], np.float32), np.array([0, 1, 1]),
                       np.array([0, 2, 3])), shape=(2, 2))
    b = sp.csr_matrix((np.array([3.0, 3.0], np.float32), np.array([0, 0]), np.array([0, 1, 2])),
                      shape=(2, 1))
    got = product_on_gpu(a, b)
    assert list(got.indptr) == [0, 1, 2] and list(got.indices) == [0, 0]
    assert list(got.data) == [0.0, 6.0]


def test_product_with_empty_operands():
    rng = np.random.default_rng(1)
    b = rand_csr(rng, 30, 20, 4)
    for a in (sp.csr_matrix((0, 30), dtype=np.float32),  # no rows
              sp.csr_matrix((25, 30), dtype=np.float32)):  # no entries
        got = product_on_gpu(a, b)
        assert got.shape == (a.shape[0], 20) and got.nnz == 0
        assert np.array_equal(got.indptr, np.zeros(a.shape[0] + 1))


def test_product_rows_pass_rejects_pointers_of_another_product():
    # fill with the row pointer of a different product: rows whose size does
    # not match are flagged, nothing is written past the given sizes
    rng = np.random.default_rng(2)
    a = rand_csr(rng, 20, 10, 3)
    b = rand_csr(rng, 10, 15, 3)
    da, db = dev(a), dev(b)
    ptr, st = saa.seacells_csr_matmul_rows(da, db)
    torch.cuda.synchronize()
    nnz = int(ptr[-1].item())
    short = torch.zeros_like(ptr)  # every row claimed empty
    idx = torch.full((nnz + 64,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((nnz + 64,), 5.0, dtype=torch.float32, device="cuda")
    _, _, st2 = saa.seacells_csr_matmul_fill(da, db, short, idx, val)
    torch.cuda.synchronize()
    assert "BAD_INDEX" in saa.status_flags(st2)
    assert bool((idx == -7).all()) and bool((val == 5.0).all())


TRANSPOSE_CASES = {
    "small": (13, 9, 3, 0),
    "tall": (300_000, 50, 2, 3),       # 1024 row blocks, several rows each
    "wide": (10_000, 5_000_000, 3, 4),  # few blocks (table bound)
    "one_row": (1, 1000, 200, 0),
    "one_col": (5000, 1, 1, 0),
    "no_entries": (40, 30, 0, 0),
}


@pytest.mark.parametrize("case", sorted(TRANSPOSE_CASES))
def test_transpose_bit_exact(case):
    m, q, per_row, empty_every = TRANSPOSE_CASES[case]
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if per_row == 0:
        a = sp.csr_matrix((m, q), dtype=np.float32)
    else:
        a = rand_csr(rng, m, q, per_row, empty_every=empty_every)
    st = saa.new_status()
    t, _ = saa.seacells_csr_transpose(dev(a), status=st)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    got = host(t)
    want = S.transpose(a)
    assert got.shape == want.shape
    assert np.array_equal(got.indptr, want.indptr)
    assert np.array_equal(got.indices, want.indices)
    assert np.array_equal(got.data.view(np.uint32), want.data.astype(np.float32).view(np.uint32))


def dot_on_gpu(x, y, alpha, start):
    acc = torch.tensor([start], dtype=torch.float64, device="cuda")
    st = saa.new_status()
    saa.seacells_csr_dot(dev(x), dev(y), alpha, acc, status=st)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    return float(acc.item())


@pytest.mark.parametrize("m,q,per_row", [(1, 10, 5), (500, 300, 20), (200_000, 2000, 8)])
def test_inner_product(m, q, per_row):
    rng = np.random.default_rng(m)
    x = rand_csr(rng, m, q, per_row, empty_every=9)
    y = rand_csr(rng, m, q, per_row, empty_every=4)
    scale = S.dot_abs(x, y)
    got = dot_on_gpu(x, y, 1.0, 0.0)
    assert abs(got - S.dot(x, y)) <= 1e-12 * scale + 1e-300
    # accumulation: acc += alpha * <x, y>
    got2 = dot_on_gpu(x, y, -2.0, 1.5)
    assert abs(got2 - (1.5 - 2.0 * S.dot(x, y))) <= 1e-12 * (2 * scale + 1.5)
    # <x, x>
    assert abs(dot_on_gpu(x, x, 1.0, 0.0) - S.dot(x, x)) <= 1e-12 * S.dot_abs(x, x)


def test_inner_product_of_empty_matrices_leaves_acc():
    z = sp.csr_matrix((0, 7), dtype=np.float32)
    assert dot_on_gpu(z, z, 3.0, 2.25) == 2.25


def chain_terms(first: S.Product):
    return int(first.terms.max()) if first.terms.size else 0


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_operands_from_the_kernel_match_oracle_and_generator(name):
    w = W.make(name)
    K = W.kernel_matrix(w)
    st = saa.new_status()
    ops = saa.device_operands(dev(K), dev(w.b), dev(w.a_prev_t), status=st)
    acc, _ = saa.rss(dev(K), ops["k2b"], dev(w.a_prev_t), ops["t1"], ops["aat"], status=st)
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    want = S.operands(K, w.b, w.a_prev_t)
    got = {nm: host(d) for nm, d in ops.items()}
    # first-level products and transposes
    check_product(got["kb"], want.kb, what="K B")
    check_product(got["kat"], want.kat, what="K A^T")
    for nm, ref in (("bt", want.bt), ("a", want.a)):
        assert np.array_equal(got[nm].indptr, ref.indptr) and np.array_equal(
            got[nm].indices, ref.indices) and np.array_equal(got[nm].data, ref.data), nm
    # chained products: the first factor's rounding is carried through (all
    # operands are non-negative, so sum|.| of the chain is its value)
    rel = {}
    rel["k2b"] = check_product(got["k2b"], want.k2b, extra_terms=chain_terms(want.kb) + 1,
                               what="K^2 B")
    rel["k2at"] = check_product(got["k2at"], want.k2at, extra_terms=chain_terms(want.kat) + 1,
                                what="K^2 A^T")
    l2 = chain_terms(want.kb) + chain_terms(want.k2b) + 2
    rel["t1"] = check_product(got["t1"], want.t1, extra_terms=l2, what="t1")
    rel["aat"] = check_product(got["aat"], want.aat, what="A A^T")
    # the generator's operands (f64 products of the f64 kernel, rounded to f32,
    # t1 and A A^T symmetrised): same patterns, values to f32 accuracy
    for nm in ("k2b", "t1", "aat", "k2at"):
        ref = getattr(w, nm)
        assert np.array_equal(got[nm].indptr, ref.indptr), nm
        assert np.array_equal(got[nm].indices, ref.indices), nm
        d = np.abs(got[nm].data.astype(np.float64) - ref.data) / np.abs(ref.data)
        assert d.max() <= 2e-5, (nm, d.max())
    # RSS through the expansion, from the device operands
    r_want = S.rss(K, w.b, w.a_prev_t)
    r_scale = S.rss_scale(K, w.b, w.a_prev_t)
    r_got = float(acc.item())
    assert abs(r_got - r_want) <= 1e-5 * r_scale, (r_got, r_want, r_scale)
    print("\n%s: max rel error %s; rss %.6e (oracle %.6e, scale %.3e)" % (
        name, {k: "%.1e" % v for k, v in rel.items()}, r_got, r_want, r_scale))
