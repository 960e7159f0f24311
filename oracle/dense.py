"""Dense numpy forms of the SEACells objective and its Frank-Wolfe updates.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). These work from the dense
matrices K, B, A of the method rather than from the CSR operands, and serve
as an implementation independent of the C oracle for tiny sizes.

Method (bixverse-rs 0.6.4, ``seacells_kernels.rs``, module doc and the
``fw_columns_a_gpu`` / ``fw_argmin_b`` docs): minimise
f(A, B) = ||K - K B A||_F^2 with K symmetric, B (n x k) and A (k x n)
column-stochastic. Its gradients are
    grad_A = 2 (B^T K^2 B A - B^T K^2)
    grad_B = 2 (K^2 B A A^T - K^2 A^T)
and the pages' updates drop the factor 2 (an argmin is unchanged by it).
"""
from __future__ import annotations

import numpy as np


def objective(K, B, A):
    """||K - K B A||_F^2 by brute force."""
    R = K - K @ B @ A
    return float(np.sum(R * R))


def grad_a(K, B, A):
    K2 = K @ K
    return 2.0 * (B.T @ K2 @ B @ A - B.T @ K2)


def grad_b(K, B, A):
    K2 = K @ K
    return 2.0 * (K2 @ B @ A @ A.T - K2 @ A.T)


def rss_closed_form(K, B, A):
    """||K||^2 - 2 <K^2 B, A^T> + <B^T K^2 B, A A^T>, the RSS without K B A."""
    K2 = K @ K
    return float(np.sum(K * K) - 2.0 * np.sum((K2 @ B) * A.T) + np.sum((B.T @ K2 @ B) * (A @ A.T)))


def fw_a_columns(t1, k2b, a_prev, T, gamma=None):
    """A update on dense operands: t1 [k, k], k2b [n, k], a_prev [k, n].

    Returns (A [k, n], picks [n, T]). np.argmin returns the first minimum,
    i.e. the lowest index on a tie.
    """
    t1 = np.asarray(t1, np.float64)
    k2b = np.asarray(k2b, np.float64)
    A = np.array(a_prev, np.float64, copy=True)
    n = k2b.shape[0]
    picks = np.empty((n, T), np.int64)
    for t in range(T):
        gam = 2.0 / (t + 2.0) if gamma is None else float(gamma[t])
        G = t1 @ A - k2b.T                    # column j is g for cell j
        idx = np.argmin(G, axis=0)
        picks[:, t] = idx
        A *= (1.0 - gam)
        A[idx, np.arange(n)] += gam
    return A, picks


def fw_b_argmin(k2b, aat, k2at, b=None):
    """B-gradient argmin on dense operands. Returns (min [k], argmin [k], gap)."""
    G = np.asarray(k2b, np.float64) @ np.asarray(aat, np.float64) - np.asarray(k2at, np.float64)
    idx = np.argmin(G, axis=0)
    val = G[idx, np.arange(G.shape[1])]
    gap = 0.0 if b is None else float(np.sum(np.asarray(b, np.float64) * G))
    return val, idx, gap, G
