"""Sparse products, transposes and inner products in f64: the operand
construction of SEACells written from the definitions.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): only the tests, the smoke
check and the bench's CPU baseline use this module; the library never does.

What is computed (bixverse-rs 0.6.4, ``seacells_kernels.rs``): the module
doc leaves kernel construction and the RSS to the host, and the
``lower_bound`` doc names the host's ``csr_matmul_csr`` (a CSR x CSR
product, each output row sorted) and ``transpose_sparse`` (rows of the
transpose in ascending order of the original rows). From the objective
f(A, B) = ||K - K B A||_F^2 (same page, module doc) the operands are

    K^2 B = K (K B),  t1 = B^T K^2 B,  A A^T,  K^2 A^T = K (K A^T),

and, with K symmetric, the RSS expands as
    ||K||_F^2 - 2 <K^2 B, A^T> + <B^T K^2 B, A A^T>
(trace of R^T R with R = K - K B A; <X, Y> = sum of X * Y).

Conventions: operands are scipy CSR matrices (f32 or f64 values, sorted
unique columns per row). Every result is f64. A product's stored pattern is
the set of (i, c) reached by some stored a[i, j] and stored b[j, c], whatever
the values, so a sum that cancels is kept as an explicit 0.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import scipy.sparse as sp


def _f64(m) -> sp.csr_matrix:
    m = sp.csr_matrix(m, dtype=np.float64, copy=True)
    m.sort_indices()
    return m


def _indicator(m: sp.csr_matrix) -> sp.csr_matrix:
    """The stored pattern of m with every value 1 (explicit zeros included)."""
    return sp.csr_matrix((np.ones(m.nnz), m.indices.copy(), m.indptr.copy()), shape=m.shape)


def _keys(m: sp.csr_matrix) -> np.ndarray:
    """Row-major position of every stored entry (sorted for a sorted CSR)."""
    rows = np.repeat(np.arange(m.shape[0], dtype=np.int64), np.diff(m.indptr))
    return rows * np.int64(m.shape[1]) + m.indices.astype(np.int64)


def _on_pattern(pat: sp.csr_matrix, m: sp.csr_matrix) -> np.ndarray:
    """The values of m at the stored positions of pat (0 where m stores
    nothing; m's pattern must lie inside pat's)."""
    pk, mk = _keys(pat), _keys(m)
    at = np.searchsorted(pk, mk)
    if mk.size and (at.max() >= pk.size or not np.array_equal(pk[at], mk)):
        raise AssertionError("value outside the pattern")
    out = np.zeros(pk.size)
    out[at] = m.data
    return out


@dataclass
class Product:
    """C = A B on the structural pattern of the product."""
    indptr: np.ndarray     # [m + 1] int64
    indices: np.ndarray    # [nnz] int64, ascending per row
    value: np.ndarray      # [nnz] f64: sum_j a[i, j] b[j, c]
    abs_value: np.ndarray  # [nnz] f64: sum_j |a[i, j] b[j, c]|
    terms: np.ndarray      # [nnz] int64: number of products in the sum
    shape: tuple

    def csr(self) -> sp.csr_matrix:
        out = sp.csr_matrix((self.value, self.indices, self.indptr), shape=self.shape)
        out.has_sorted_indices = True
        return out


def matmul(a, b) -> Product:
    """A B (the page's ``csr_matmul_csr``) in f64.

    The pattern is the product of the two indicator matrices (its values
    count the products that meet at each output); the values are scipy's
    f64 product, placed on that pattern. Products of f32 inputs are exact in
    f64, so ``value`` carries only f64 summation error.
    """
    A, B = _f64(a), _f64(b)
    if A.shape[1] != B.shape[0]:
        raise ValueError("inner dimensions differ")
    pat = (_indicator(A) @ _indicator(B)).tocsr()
    pat.sort_indices()
    val = (A @ B).tocsr()
    val.sort_indices()
    absval = (abs(A) @ abs(B)).tocsr()
    absval.sort_indices()
    return Product(indptr=pat.indptr.astype(np.int64), indices=pat.indices.astype(np.int64),
                   value=_on_pattern(pat, val), abs_value=_on_pattern(pat, absval),
                   terms=np.rint(pat.data).astype(np.int64), shape=(A.shape[0], B.shape[1]))


def matmul_rows(a, b, rows) -> Product:
    """Rows ``rows`` of A B (the same definition as ``matmul``)."""
    A = _f64(a)[np.asarray(rows, np.int64)]
    return matmul(A, b)


def transpose(a) -> sp.csr_matrix:
    """A^T with every stored entry kept (the page's ``transpose_sparse``):
    row c lists the rows of A that store column c, in ascending order."""
    A = sp.csr_matrix(a, copy=True)
    A.sort_indices()
    m, q = A.shape
    rows = np.repeat(np.arange(m, dtype=np.int64), np.diff(A.indptr))
    cols = A.indices.astype(np.int64)
    order = np.lexsort((rows, cols))  # by column, then by row
    counts = np.bincount(cols, minlength=q)
    ptr = np.zeros(q + 1, np.int64)
    np.cumsum(counts, out=ptr[1:])
    out = sp.csr_matrix((A.data[order], rows[order], ptr), shape=(q, m))
    out.has_sorted_indices = True
    return out


def _dots(x, y):
    """(sum x * y, sum |x * y|) over the positions stored in both, in f64:
    every position of the matrix with fewer entries is looked up among the
    sorted positions of the other."""
    if x.shape != y.shape:
        raise ValueError("shapes differ")
    X, Y = sp.csr_matrix(x), sp.csr_matrix(y)
    if X.nnz < Y.nnz:
        X, Y = Y, X
    X.sort_indices()
    Y.sort_indices()
    kx, ky = _keys(X), _keys(Y)
    at = np.searchsorted(kx, ky)
    hit = at < kx.size
    hit[hit] = kx[at[hit]] == ky[hit]
    prod = X.data[at[hit]].astype(np.float64) * Y.data[hit].astype(np.float64)
    return float(np.sum(prod)), float(np.sum(np.abs(prod)))


def dot(x, y) -> float:
    """<X, Y> = sum over positions stored in both of x * y, in f64."""
    return _dots(x, y)[0]


def dot_abs(x, y) -> float:
    """sum |x * y| over the common positions (the scale of ``dot``'s rounding)."""
    return _dots(x, y)[1]


@dataclass
class Operands:
    """The Frank-Wolfe operands built from K, B and A^T (f64)."""
    kb: Product
    k2b: Product
    bt: sp.csr_matrix
    t1: Product
    a: sp.csr_matrix
    aat: Product
    kat: Product
    k2at: Product


def operands(K, B, At) -> Operands:
    """K B, K^2 B = K (K B), B^T, t1 = B^T K^2 B, A = (A^T)^T, A A^T,
    K A^T and K^2 A^T = K (K A^T), each product from its f64 operands."""
    kb = matmul(K, B)
    k2b = matmul(K, kb.csr())
    bt = transpose(B)
    t1 = matmul(bt, k2b.csr())
    a = transpose(At)
    aat = matmul(a, At)
    kat = matmul(K, At)
    k2at = matmul(K, kat.csr())
    return Operands(kb, k2b, bt, t1, a, aat, kat, k2at)


def rss(K, B, At) -> float:
    """||K - K B A||_F^2 through the expansion above (K symmetric), f64."""
    Kf, Bf, Atf = _f64(K), _f64(B), _f64(At)
    k2b = Kf @ (Kf @ Bf)
    t1 = Bf.T @ k2b
    aat = Atf.T @ Atf
    return dot(Kf, Kf) - 2.0 * dot(k2b, Atf) + dot(t1, aat)


def rss_scale(K, B, At) -> float:
    """||K||^2 + 2 |<K^2 B, A^T>| + |<t1, A A^T>| with absolute values
    throughout: the size of the terms that cancel in ``rss``."""
    Kf, Bf, Atf = abs(_f64(K)), abs(_f64(B)), abs(_f64(At))
    k2b = Kf @ (Kf @ Bf)
    t1 = Bf.T @ k2b
    aat = Atf.T @ Atf
    return dot(Kf, Kf) + 2.0 * dot(k2b, Atf) + dot(t1, aat)


def rss_of_operands(K, k2b, At, t1, aat):
    """The same expansion evaluated on given operands K, K^2 B, A^T,
    B^T K^2 B and A A^T (f64 sums): (value, scale), the scale as in
    ``rss_scale``."""
    (kk, kk_a), (ba, ba_a), (ta, ta_a) = _dots(K, K), _dots(k2b, At), _dots(t1, aat)
    return kk - 2.0 * ba + ta, kk_a + 2.0 * ba_a + ta_a


def add(alpha, x, beta, y) -> sp.csr_matrix:
    """alpha X + beta Y in f64 (the page's ``sparse_add_csr``, named in its
    ``lower_bound`` doc, merges two sorted rows): the pattern is the union of
    the stored patterns (a position stored in either operand stays stored,
    even where the sum is 0), the values are scipy's f64 sum placed on it."""
    X, Y = _f64(x), _f64(y)
    if X.shape != Y.shape:
        raise ValueError("shapes differ")
    pat = (_indicator(X) + _indicator(Y)).tocsr()
    pat.sort_indices()
    val = (float(alpha) * X + float(beta) * Y).tocsr()
    val.sort_indices()
    out = sp.csr_matrix((_on_pattern(pat, val), pat.indices.copy(), pat.indptr.copy()),
                        shape=X.shape)
    out.has_sorted_indices = True
    return out


def picks(idx, n: int, value: float = 1.0) -> sp.csr_matrix:
    """The n x k matrix holding ``value`` at (idx[c], c) for every column c
    (a Frank-Wolfe vertex of the column-stochastic B when value is 1)."""
    idx = np.asarray(idx, np.int64)
    k = idx.shape[0]
    out = sp.csr_matrix((np.full(k, float(value)), (idx, np.arange(k))), shape=(n, k))
    out.sort_indices()
    return out


def atoms_to_csr(atom_idx, atom_val, atom_cnt, k: int) -> sp.csr_matrix:
    """The A update's returned columns as A^T (n x k CSR): row j holds cell
    j's atoms (the first atom_cnt[j] slots of its lists) with a non-zero
    weight, in ascending column order."""
    atom_idx = np.asarray(atom_idx)
    atom_val = np.asarray(atom_val, np.float64)
    n = atom_idx.shape[0]
    rows, cols, vals = [], [], []
    for j in range(n):
        c = int(atom_cnt[j])
        keep = atom_val[j, :c] != 0.0
        order = np.argsort(atom_idx[j, :c][keep], kind="stable")
        rows.append(np.full(int(keep.sum()), j))
        cols.append(atom_idx[j, :c][keep][order].astype(np.int64))
        vals.append(atom_val[j, :c][keep][order])
    out = sp.csr_matrix((np.concatenate(vals) if vals else np.zeros(0),
                         (np.concatenate(rows) if rows else np.zeros(0, np.int64),
                          np.concatenate(cols) if cols else np.zeros(0, np.int64))), shape=(n, k))
    out.sort_indices()
    return out
