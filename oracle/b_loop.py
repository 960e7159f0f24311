"""The B update as a loop of Frank-Wolfe steps, in f64 with dense B.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): only the tests, the smoke
check and the bench's CPU baseline use this module; the library never does.

Source: bixverse-rs 0.6.4, ``seacells_kernels.rs``, the ``fw_argmin_b`` doc
(the gradient G = K^2 B AA^T - K^2 A^T of the B update, its column-wise
argmin with the lowest row winning a tie, and sum(B * G)). The page leaves
the B step itself to the host; the reading taken here is the plain
Frank-Wolfe step on every column of the column-stochastic B,
B <- (1 - gamma_t) B + gamma_t S, with S the vertex matrix holding 1 at
(argmin row of column c, c), and gamma_t = 2 / (t + 2) unless a schedule is
given. A (hence A A^T and K^2 A^T) is fixed during the loop; K^2 B is
recomputed from the current B at every step as K (K B).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import scipy.sparse as sp


@dataclass
class BLoop:
    pick: np.ndarray     # [T, k] the oracle's argmin row per column and step
    used: np.ndarray     # [T, k] the row the step was taken with (pick, or forced)
    gmin: np.ndarray     # [T, k] min over rows of G[:, c]
    second: np.ndarray   # [T, k] second smallest G[:, c] (+inf for n = 1)
    g_used: np.ndarray   # [T, k] G at the used row
    scale: np.ndarray    # [T, k] term scale (|K^2 B| |AA^T| + |K^2 A^T|) at the used row
    gap: np.ndarray      # [T] sum(B_t * G_t)
    b: np.ndarray        # [n, k] B after the last step
    k2b: np.ndarray      # [n, k] K (K B) after the last step
    k2b_used: np.ndarray = None  # [T, k, k] row used[t, c] of K^2 B_t (keep_rows only)


def _dense(m) -> np.ndarray:
    return np.asarray(m.toarray() if sp.issparse(m) else m, np.float64)


def fw_b_loop(K, B0, aat, k2at, T: int, gammas=None, force=None, keep_rows=False) -> BLoop:
    """T Frank-Wolfe steps of the B update from B0 (n x k).

    Step t: K^2 B_t = K (K B_t); G_t = K^2 B_t A A^T - K^2 A^T; the pick of
    column c is the lowest row minimising G_t[:, c]; B_{t+1} =
    (1 - gamma_t) B_t + gamma_t S_t. With ``force`` ([T, k]) the step uses
    force[t] instead of the pick (replaying another trajectory) and reports
    G_t there. ``keep_rows`` also returns the rows of K^2 B_t that G_t was
    read at (how a change of A A^T reaches those values).
    """
    Ks = sp.csr_matrix(K, dtype=np.float64)
    B = _dense(B0).copy()
    AAt = _dense(aat)
    K2At = _dense(k2at)
    n, k = B.shape
    cols = np.arange(k)
    out = {nm: np.zeros((T, k)) for nm in ("gmin", "second", "g_used", "scale")}
    pick = np.zeros((T, k), np.int64)
    used = np.zeros((T, k), np.int64)
    rows = np.zeros((T, k, k)) if keep_rows else None
    gap = np.zeros(T)
    for t in range(T):
        K2B = Ks @ (Ks @ B)
        G = K2B @ AAt - K2At
        p = np.argmin(G, axis=0)  # first (lowest) row on a tie
        pick[t] = p
        out["gmin"][t] = G[p, cols]
        if n > 1:
            out["second"][t] = np.partition(G, 1, axis=0)[1]
        else:
            out["second"][t] = np.inf
        u = p if force is None else np.asarray(force[t], np.int64)
        used[t] = u
        out["g_used"][t] = G[u, cols]
        if keep_rows:
            rows[t] = K2B[u]
        S = np.abs(K2B[u]) @ np.abs(AAt)  # [k, k]: rows u_c of |K^2 B| |AA^T|
        out["scale"][t] = S[cols, cols] + np.abs(K2At[u, cols])
        gap[t] = float(np.sum(B * G))
        g = 2.0 / (t + 2.0) if gammas is None else float(gammas[t])
        B *= 1.0 - g
        B[u, cols] += g
    return BLoop(pick=pick, used=used, gap=gap, b=B, k2b=Ks @ (Ks @ B), k2b_used=rows, **out)
