"""Acceptance rules for GPU results against the f64 oracle (test helper).

Argmin indices: the GPU's pick p at a step (or for a column) is accepted when
it equals the oracle's, or when the oracle's f64 gradient at p lies within
TIE_REL of the minimum, relative to max(|g_min|, |g_second|, S). S is the
size of the terms the gradient is a difference of: in f32 the error of g
scales with S, not with |g|, so a tie window relative to |g| alone would
reject rounding-level disagreements at g ~ 0. Outside such near ties the
index must match exactly.

A values: the oracle replays the GPU's own trajectory (every step forced to
the GPU's pick, after the pick is checked as above). Each entry of the GPU's
A column must then be within A_ABS of the replayed f64 column.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import scipy.sparse as sp

import oracle

TIE_REL = 1e-5   # near-tie window, relative
A_ABS = 1e-5     # A entries after T steps, absolute
B_ABS = 1e-5     # B entries after the B step, absolute
VAL_REL, VAL_ABS = 1e-4, 1e-5   # B minimum values (the page's policy)
GAP_REL = 1e-3                  # sum(B * G) (the page's policy)
# Pruning: a cell whose replayed weights came within this distance of the
# threshold at some step is left out (f32 and f64 weights may fall on either
# side of it: f32 weights of ~0.02 carry ~1e-7 of rounding after 50 steps);
# outside that band both take the same drop decisions.
PRUNE_MARGIN = 1e-6
# Frank-Wolfe gap of the returned column, <g, a> - min g: each g entry
# carries f32 rounding of ~T ulps of the term scale S (T = 50: ~3e-6 S; S is
# the largest over the run, since drops take earlier terms back out), and
# the minimum may sit at a near tie: within 2e-5 S.
GAP_A_REL = 2e-5


def dense_atoms(atom_idx, atom_val, atom_cnt, k):
    """Scatter GPU atom lists [m, cap] into dense [m, k] (f64)."""
    m, cap = atom_idx.shape
    out = np.zeros((m, k), np.float64)
    for r in range(m):
        c = int(atom_cnt[r])
        assert 0 <= c <= cap
        ids = atom_idx[r, :c].astype(np.int64)
        assert np.all((ids >= 0) & (ids < k)), "atom index out of range"
        assert np.unique(ids).shape[0] == c, "duplicate atom in a cell"
        out[r, ids] = atom_val[r, :c]
    return out


@dataclass
class AReport:
    steps: int
    exact: int
    near_tie: int
    zero_tie_mismatch: int
    max_abs_err: float
    worst_window: float
    skipped: int = 0          # cells left out for a drop decision within PRUNE_MARGIN
    gap_err: float = 0.0      # worst |fw_gap - oracle| / scale when the gap was checked


def check_atom_layout(atom_idx, atom_cnt, trace, a_prev_t, cells):
    """Seeds first in A_prev order, then each new pick in order of first pick."""
    for r, j in enumerate(cells):
        s0, s1 = a_prev_t.indptr[j], a_prev_t.indptr[j + 1]
        seeds = list(a_prev_t.indices[s0:s1])
        want = list(seeds)
        for p in trace[r]:
            if int(p) not in want:
                want.append(int(p))
        got = list(atom_idx[r, :atom_cnt[r]].astype(np.int64))
        assert got == want, (j, got[:10], want[:10])


def check_a(w, gpu_trace, atom_idx, atom_val, atom_cnt, cells, gamma=None, T=None,
            strict_zero_ties=True, prune=None, fw_gap=None) -> AReport:
    """Trace replay of the A update for ``cells``; returns counts and errors.

    ``prune`` (a threshold) replays the pruning variant. Its drop steps take
    products back out of the state, so a column can return to an exact 0 in
    f64 but not in f32: the structural zero-tie rule is not applied then."""
    T = w.T if T is None else T
    cells = np.asarray(cells, np.int64)
    trace = np.asarray(gpu_trace, np.int64)
    atom_idx, atom_val, atom_cnt = np.asarray(atom_idx), np.asarray(atom_val), np.asarray(atom_cnt)
    assert trace.shape == (cells.shape[0], T)
    assert np.all((trace >= 0) & (trace < w.k)), "trace index out of range"
    rep = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, T, cells=cells, force=trace,
                              gamma=gamma, prune=prune)
    skipped = 0
    if prune is not None:
        strict_zero_ties = False
        keep = ~np.any(rep.margin < PRUNE_MARGIN, axis=1)
        skipped = int((~keep).sum())
        if skipped:
            cells, trace = cells[keep], trace[keep]
            atom_idx, atom_val, atom_cnt = atom_idx[keep], atom_val[keep], atom_cnt[keep]
            if fw_gap is not None:
                fw_gap = np.asarray(fw_gap)[keep]
            for f in ("a", "pick", "g_min", "g_second", "g_scale", "g_taken", "g_dot"):
                setattr(rep, f, getattr(rep, f)[keep])
    exact = trace == rep.pick
    window = TIE_REL * np.maximum(np.maximum(np.abs(rep.g_min), np.abs(rep.g_second)),
                                  rep.g_scale)
    excess = rep.g_taken - rep.g_min
    ok = exact | (excess <= window)
    bad = np.argwhere(~ok)
    if bad.shape[0]:
        r, t = bad[0]
        raise AssertionError(
            "cell %d step %d: gpu picked %d (g=%.9g), oracle %d (g=%.9g, second %.9g, scale %.3g); "
            "%d bad steps" % (cells[r], t, trace[r, t], rep.g_taken[r, t], rep.pick[r, t],
                              rep.g_min[r, t], rep.g_second[r, t], rep.g_scale[r, t], bad.shape[0]))
    # Structural zeros: with non-negative t1, a column outside supp(t2_j) whose
    # f64 gradient is exactly 0 was never touched by a picked t1 row, so the
    # f32 state holds an exact 0 there as well and the lowest such column must
    # win bit for bit. (A zero reached by cancellation against t2 is only a
    # rounding-level tie and falls under the window above.)
    zero_tie = (rep.g_min == 0.0) & (rep.g_taken == 0.0) & ~exact
    if strict_zero_ties and np.any(zero_tie) and (w.t1.data.min(initial=0.0) >= 0.0):
        rr, tt = np.nonzero(zero_tie)
        t2 = w.k2b[cells[rr]]
        t2_gpu = np.asarray(t2[np.arange(rr.shape[0]), trace[rr, tt]]).ravel()
        t2_orc = np.asarray(t2[np.arange(rr.shape[0]), rep.pick[rr, tt]]).ravel()
        structural = (t2_gpu == 0.0) & (t2_orc == 0.0)
        assert not np.any(structural), "lowest-index rule broken at a structural zero tie"
        zero_tie[rr[~structural], tt[~structural]] = False
    got = dense_atoms(atom_idx, atom_val, atom_cnt, w.k)
    err = float(np.max(np.abs(got - rep.a))) if got.size else 0.0
    assert err <= A_ABS, "A entries differ from the replayed oracle by %.3g" % err
    check_atom_layout(atom_idx, atom_cnt, trace, w.a_prev_t, cells)
    gap_err = 0.0
    if fw_gap is not None and cells.shape[0]:
        # the gap of the returned column a_T: the oracle replays the T steps
        # and reports the gap at the start of one more (free) step; the f32
        # state's rounding is relative to the largest terms it has held
        # (pruning takes whole rows back out of it)
        force1 = np.concatenate([trace, np.full((cells.shape[0], 1), -1, np.int64)], axis=1)
        gam1 = None if gamma is None else np.concatenate([np.asarray(gamma, np.float64), [0.5]])
        rep1 = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, T + 1, cells=cells,
                                   force=force1, gamma=gam1, prune=prune)
        want = rep1.fw_gap[:, T]
        scale = np.maximum(rep1.g_scale.max(axis=1), np.abs(want))
        got = np.asarray(fw_gap, np.float64)
        rel = np.abs(got - want) / np.maximum(scale, 1e-30)
        worst = int(np.argmax(rel))
        assert rel[worst] <= GAP_A_REL, ("cell %d: fw_gap %.9g, oracle %.9g (scale %.3g)"
                                         % (cells[worst], got[worst], want[worst], scale[worst]))
        gap_err = float(rel[worst])
    return AReport(int(trace.size), int(exact.sum()), int((~exact).sum()), int(zero_tie.sum()),
                   err, float(np.max(excess / np.maximum(window, 1e-300))) if excess.size else 0.0,
                   skipped, gap_err)


@dataclass
class BReport:
    exact: int
    near_tie: int
    max_val_rel: float
    gap_rel: float


def check_b(w, out_val, out_idx, gap, n=None, k=None, b=True, res=None, fw_gap=None) -> BReport:
    n = w.n if n is None else n
    k = w.k if k is None else k
    if res is None:
        res = oracle.fw_b_argmin(w.k2b, w.aat, w.k2at, w.b if b else None, n, k)
    out_idx = np.asarray(out_idx, np.int64)
    out_val = np.asarray(out_val, np.float64)
    assert np.all((out_idx >= 0) & (out_idx < n)), "argmin row out of range"
    exact = out_idx == res.row
    mism = np.flatnonzero(~exact)
    if mism.shape[0]:
        g, sc = oracle.fw_b_grad_at(w.k2b, w.aat, w.k2at, n, k, out_idx[mism], mism)
        scale = np.maximum.reduce([np.abs(res.val[mism]), np.abs(res.second[mism]), sc,
                                   res.row_scale[res.row[mism]]])
        over = (g - res.val[mism]) > TIE_REL * scale
        if np.any(over):
            c = mism[np.argmax(over)]
            raise AssertionError("column %d: gpu row %d, oracle row %d (min %.9g, second %.9g)"
                                 % (c, out_idx[c], res.row[c], res.val[c], res.second[c]))
    tol = VAL_ABS + VAL_REL * np.abs(res.val)
    dv = np.abs(out_val - res.val)
    assert np.all(dv <= tol), "min values differ: worst %.3g" % float(np.max(dv - tol))
    grel = 0.0
    if gap is not None and b:
        grel = abs(float(gap) - res.gap) / max(abs(res.gap), 1e-4 / GAP_REL)
        assert grel <= GAP_REL, "gap %.9g vs oracle %.9g" % (float(gap), res.gap)
    if fw_gap is not None:
        # the full gap sum(B * G) - sum_c min G, at the page's relative gap
        # policy, relative to the size of the two sums it is a difference of
        size = abs(res.gap) + float(np.sum(np.abs(res.val)))
        assert abs(float(fw_gap) - res.fw_gap) <= GAP_REL * max(size, 1e-4 / GAP_REL), \
            "fw_gap %.9g vs oracle %.9g" % (float(fw_gap), res.fw_gap)
    return BReport(int(exact.sum()), int((~exact).sum()),
                   float(np.max(dv / np.maximum(np.abs(res.val), 1e-30))), grel)


# --------------------------------------------------------------------------
# the B argmin's partials
# --------------------------------------------------------------------------

NO_VALUE_KEY = (0xff800000 << 32) | 0xffffffff   # (+inf, ~0): a unit that saw no finite value


def check_b_partials(keys, stamps, epoch, n, slice_w):
    """The check the B argmin's reduce makes on its partials, restated on the
    host. keys [n_row_blocks, k] u64 (value key << 32 | row), stamps
    [n_row_blocks, n_slices] u32. Every stamp must be this call's epoch, and
    every key's row must lie in its row range [n rb / NB, n (rb + 1) / NB);
    a key (+inf, ~0) means the unit saw no finite value. Returns the flags
    the device raises for these partials ([] when they are valid)."""
    keys = np.asarray(keys, np.uint64)
    stamps = np.asarray(stamps, np.uint32)
    nb, k = keys.shape
    flags = set()
    cols_slice = np.arange(k) // slice_w
    if np.any(stamps[:, cols_slice] != np.uint32(epoch)):
        flags.add("PARTIALS_INVALID")
    rows = (keys & np.uint64(0xffffffff)).astype(np.int64)
    rb = np.arange(nb, dtype=np.int64)[:, None]
    lo, hi = (n * rb) // nb, (n * (rb + 1)) // nb
    none = keys == np.uint64(NO_VALUE_KEY)
    if np.any(none):
        flags.add("NONFINITE")
    if np.any(~none & ((rows < lo) | (rows >= hi))):
        flags.add("PARTIALS_INVALID")
    return sorted(flags)


# --------------------------------------------------------------------------
# sparse products (device operand construction)
# --------------------------------------------------------------------------

U32 = 2.0 ** -24  # unit roundoff of f32


def check_product(got, want, extra_terms=0, what=""):
    """A device product against oracle.sparse.matmul's: the stored pattern
    bit-exact, and every value within the bound of an f32 sum of t fused
    multiply-adds, 1.01 t 2^-24 sum|a b| (t = the entry's number of products
    plus ``extra_terms`` for the rounding a chained factor carries). Returns
    the largest error relative to sum|a b|."""
    assert got.shape == want.shape, what
    assert np.array_equal(got.indptr, want.indptr), what
    assert np.array_equal(got.indices, want.indices), what
    tol = 1.01 * (want.terms + extra_terms) * U32 * want.abs_value
    err = np.abs(got.data.astype(np.float64) - want.value)
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, "%s: %d entries out of bound, first %s: got %r want %r tol %r" % (
        what, bad.size, bad[:3], got.data[bad[:3]], want.value[bad[:3]], tol[bad[:3]])
    return float((err / np.maximum(want.abs_value, 1e-300)).max()) if err.size else 0.0


def a_change_bound(K, at, used, k2b_used, d_a):
    """Bound on how far G_t[used[t, c], c] moves when every entry of A
    (A^T = ``at``, n x k, non-negative) moves by at most d_a, with K, K2B >= 0:
    d_a (sum_m K2B_t[u, m] (R[m] + R[c]) + (K K 1)[u]), R the row sums of A
    (first order in d_a). ``k2b_used`` [T, k, k] holds the rows K2B_t[u, :]."""
    n = K.shape[0]
    R = np.asarray(at.sum(axis=0), np.float64).ravel()
    Ks = sp.csr_matrix(K, dtype=np.float64)
    k2one = np.asarray(Ks @ (Ks @ np.ones(n)), np.float64).ravel()
    rows = np.abs(k2b_used)
    return d_a * (np.einsum("tcm,m->tc", rows, R) + rows.sum(axis=2) * R[None, :] + k2one[used])


def check_b_loop(K, b0, aat, k2at, T, res_gpu, gammas=None, a_err=None):
    """The device B loop (saa.fw_b_loop's result) against oracle.b_loop
    replaying its picks: every pick the oracle's or within the tie rule, the
    minimum values and gaps under the B argmin's policy, B after the loop
    within 1e-5, K^2 B within 5e-5 relative. Returns (picks that differ,
    worst relative error of K^2 B).

    a_err = (dA, at): the oracle's A A^T and K^2 A^T come from its own f64 A
    (``at``, n x k, the A^T of its replay of the A update) while the
    device's come from its f32 A, which differs from it by at most dA per
    entry. With A >= 0 that moves G[i, c] = sum_m K2B[i, m] AAt[m, c] -
    K2At[i, c] by at most dA (sum_m K2B[i, m] (R[m] + R[c]) + (K^2 1)[i])
    (R: row sums of A, i.e. column sums of ``at``; K2B >= 0; the dA^2 terms
    are below 1e-7 here), which is added to the tolerance of each minimum
    value at its row. The device's products A A^T and K^2 A^T are also
    rounded to f32, relative to the size of their terms, so the minimum
    values then also get the tie rule's window, TIE_REL of G's term scale."""
    from oracle import b_loop as BL
    b_gpu, k2b_gpu, picks, mins, gaps = res_gpu
    picks = picks.cpu().numpy().astype(np.int64)
    mins = mins.cpu().numpy().astype(np.float64)
    gaps = gaps.cpu().numpy().astype(np.float64)
    n = b0.shape[0]
    assert np.all((picks >= 0) & (picks < n))
    orc = BL.fw_b_loop(K, b0, aat, k2at, T, gammas=gammas, force=picks, keep_rows=a_err is not None)
    exact = picks == orc.pick
    second = np.where(np.isfinite(orc.second), orc.second, 0.0)
    over = (orc.g_used - orc.gmin) > TIE_REL * np.maximum.reduce(
        [np.abs(orc.gmin), np.abs(second), orc.scale])
    assert not np.any(over & ~exact), "pick outside the tie rule at %s" % (
        np.argwhere(over & ~exact)[:3].tolist(),)
    tol = VAL_ABS + VAL_REL * np.abs(orc.g_used)
    if a_err is not None:
        d_a, at = a_err
        tol = tol + a_change_bound(K, at, orc.used, orc.k2b_used, d_a) + TIE_REL * orc.scale
    bad = np.abs(mins - orc.g_used) > tol
    if np.any(bad):
        t, c = np.argwhere(bad)[0]
        raise AssertionError("step %d column %d: device min %.9g, oracle %.9g, tol %.3g "
                             "(scale %.3g); %d values out" % (t, c, mins[t, c], orc.g_used[t, c],
                                                               tol[t, c], orc.scale[t, c],
                                                               int(bad.sum())))
    for t in range(T):
        assert abs(gaps[t] - orc.gap[t]) <= GAP_REL * max(abs(orc.gap[t]), 1e-4 / GAP_REL), t
    from tests.gpu_run import host
    bd = host(b_gpu).toarray().astype(np.float64)
    assert np.max(np.abs(bd - orc.b)) <= 1e-5
    kd = host(k2b_gpu).toarray().astype(np.float64)
    err = np.abs(kd - orc.k2b)
    assert np.all(err <= 5e-5 * np.abs(orc.k2b) + 1e-6 * np.max(np.abs(orc.k2b)))
    return int((~exact).sum()), float(np.max(err / np.maximum(np.abs(orc.k2b), 1e-30)))
