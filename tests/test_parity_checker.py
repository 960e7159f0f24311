"""The parity checker against itself (CPU only): oracle results fed in as if
they came from the GPU pass, and each planted fault is flagged."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests import parity


@pytest.fixture(scope="module")
def case():
    w = W.make("c1")
    cells = np.arange(0, 300, 3)
    tr = oracle.fw_a_columns(w.t1, w.k2b, w.a_prev_t, w.n, w.k, w.T, cells=cells)
    cap = w.cap
    idx = np.zeros((cells.shape[0], cap), np.int64)
    val = np.zeros((cells.shape[0], cap), np.float32)
    cnt = np.zeros(cells.shape[0], np.int64)
    for r, j in enumerate(cells):
        s0, s1 = w.a_prev_t.indptr[j], w.a_prev_t.indptr[j + 1]
        atoms = list(w.a_prev_t.indices[s0:s1])
        for p in tr.pick[r]:
            if int(p) not in atoms:
                atoms.append(int(p))
        idx[r, :len(atoms)] = atoms
        val[r, :len(atoms)] = tr.a[r, atoms]
        cnt[r] = len(atoms)
    return w, cells, tr, idx, val, cnt


def test_accepts_the_oracle_itself(case):
    w, cells, tr, idx, val, cnt = case
    rep = parity.check_a(w, tr.pick, idx, val, cnt, cells)
    assert rep.exact == rep.steps and rep.max_abs_err < 1e-6


def test_flags_a_pick_outside_the_tie_window(case):
    w, cells, tr, idx, val, cnt = case
    # a step whose runner-up is clearly worse than the minimum
    r, t = np.argwhere((tr.g_second - tr.g_min) > 1e-2 * np.maximum(1, tr.g_scale))[0]
    bad = tr.pick.astype(np.int64).copy()
    g = bad[r, t]
    bad[r, t] = (g + 1) % w.k
    with pytest.raises(AssertionError):
        parity.check_a(w, bad, idx, val, cnt, cells)


def test_flags_an_a_entry_off_by_2e_5(case):
    w, cells, tr, idx, val, cnt = case
    v2 = val.copy()
    v2[5, 0] += 2e-5
    with pytest.raises(AssertionError):
        parity.check_a(w, tr.pick, idx, v2, cnt, cells)


def test_flags_duplicate_or_reordered_atoms(case):
    w, cells, tr, idx, val, cnt = case
    i2 = idx.copy()
    i2[3, 1] = i2[3, 0]
    with pytest.raises(AssertionError):
        parity.check_a(w, tr.pick, i2, val, cnt, cells)
    i3, v3 = idx.copy(), val.copy()
    c = cnt[7]
    i3[7, [c - 1, c - 2]] = i3[7, [c - 2, c - 1]]
    v3[7, [c - 1, c - 2]] = v3[7, [c - 2, c - 1]]
    with pytest.raises(AssertionError):
        parity.check_a(w, tr.pick, i3, v3, cnt, cells)


def test_flags_a_lowest_index_violation_at_structural_zero_tie():
    # t1 = I (k = 3), t2 = 0 and a_prev = e_2: g = (0, 0, 1) at step 0, two
    # structural zeros; the lowest (0) must win, and picking 1 is flagged
    n, k = 2, 3
    t1 = W.dense_to_csr(np.eye(k))
    k2b = W.dense_to_csr(np.zeros((n, k)))
    ap = W.dense_to_csr(np.array([[0, 0, 1.0], [0, 0, 1.0]]))
    cfg = W.Config("eye3", n, 0, 0, 0, k, 1, 0, T=5)
    w = W.Workload(cfg, 0, t1=t1, k2b=k2b, a_prev_t=ap, aat=t1, k2at=k2b, b=k2b,
                   init_cells=np.zeros(0, np.int64))
    tr = oracle.fw_a_columns(t1, k2b, ap, n, k, 5, cells=[0])
    assert tr.pick[0, 0] == 0 and tr.g_min[0, 0] == 0.0 and tr.g_second[0, 0] == 0.0
    # the wrong pick at step 0, then the oracle's own picks from that state on
    f = np.full((1, 5), -1, np.int64)
    f[0, 0] = 1
    bad = oracle.fw_a_columns(t1, k2b, ap, n, k, 5, cells=[0], force=f).pick.astype(np.int64)
    bad[0, 0] = 1
    rep = oracle.fw_a_columns(t1, k2b, ap, n, k, 5, cells=[0], force=bad)
    atoms = [2] + [int(p) for p in dict.fromkeys(bad[0].tolist()) if p != 2]
    idx = np.array([atoms])
    val = rep.a[:, atoms].astype(np.float32)
    with pytest.raises(AssertionError, match="structural zero tie"):
        parity.check_a(w, bad, idx, val, np.array([len(atoms)]), [0], T=5)


def test_b_checker_flags_wrong_row_and_value():
    w = W.make("c1")
    res = oracle.fw_b_argmin(w.k2b, w.aat, w.k2at, w.b, w.n, w.k)
    parity.check_b(w, res.val.astype(np.float32), res.row, res.gap, res=res)
    clear = np.flatnonzero((res.second - res.val) > 1e-3 * np.maximum(1, np.abs(res.val)))
    bad = res.row.astype(np.int64).copy()
    bad[clear[0]] = (bad[clear[0]] + 1) % w.n
    with pytest.raises(AssertionError):
        parity.check_b(w, res.val, bad, res.gap, res=res)
    v = res.val.copy()
    v[2] += 1e-3 * max(1.0, abs(v[2]))
    with pytest.raises(AssertionError):
        parity.check_b(w, v, res.row, res.gap, res=res)
    with pytest.raises(AssertionError):
        parity.check_b(w, res.val, res.row, res.gap * 1.01 + 1.0, res=res)


# --- the B argmin's partials check, restated on the host -------------------

def _order_key(v):
    """Order-preserving u32 image of f32 values (-0 folded onto +0)."""
    u = (np.asarray(v, np.float32) + np.float32(0.0)).view(np.uint32).astype(np.uint64)
    neg = (u & np.uint64(0x80000000)) != 0
    return np.where(neg, ~u & np.uint64(0xffffffff), u | np.uint64(0x80000000))


@pytest.fixture(scope="module")
def partials():
    """Partials as the reduce receives them, built from the oracle on c1:
    7 row ranges x 3 column slices, one key per (range, column)."""
    w = W.make("c1")
    nb, slice_w = 7, 10
    n_slices = -(-w.k // slice_w)
    keys = np.zeros((nb, w.k), np.uint64)
    for rb in range(nb):
        r0, r1 = w.n * rb // nb, w.n * (rb + 1) // nb
        res = oracle.fw_b_argmin(w.k2b[r0:r1], w.aat, w.k2at[r0:r1], None, r1 - r0, w.k)
        keys[rb] = (_order_key(res.val.astype(np.float32)) << np.uint64(32)) | \
            (res.row.astype(np.uint64) + np.uint64(r0))
    epoch = 0x5EAC1234
    stamps = np.full((nb, n_slices), epoch, np.uint32)
    return w, keys, stamps, epoch, slice_w


def test_partials_rule_accepts_valid_partials_and_their_minimum_is_the_argmin(partials):
    w, keys, stamps, epoch, slice_w = partials
    assert parity.check_b_partials(keys, stamps, epoch, w.n, slice_w) == []
    # the u64 minimum over row ranges is (lowest value, then lowest row)
    best = keys.min(axis=0)
    full = oracle.fw_b_argmin(w.k2b, w.aat, w.k2at, None, w.n, w.k)
    np.testing.assert_array_equal((best & np.uint64(0xffffffff)).astype(np.int64), full.row)


@pytest.mark.parametrize("fault", ["stale_stamp", "row_past_n", "row_of_another_range",
                                   "wrong_epoch", "no_value"])
def test_partials_rule_flags_each_planted_fault(partials, fault):
    w, keys, stamps, epoch, slice_w = partials
    keys, stamps = keys.copy(), stamps.copy()
    want = ["PARTIALS_INVALID"]
    if fault == "stale_stamp":
        stamps[3, 1] = epoch - 1
    elif fault == "row_past_n":
        keys[2, 5] = (keys[2, 5] & ~np.uint64(0xffffffff)) | np.uint64(w.n + 5)
    elif fault == "row_of_another_range":
        r1 = w.n * 3 // 7  # first row of range 3, planted in range 2
        keys[2, 5] = (keys[2, 5] & ~np.uint64(0xffffffff)) | np.uint64(r1)
    elif fault == "wrong_epoch":
        epoch += 1
    else:
        keys[4, 0] = np.uint64(parity.NO_VALUE_KEY)
        want = ["NONFINITE"]
    assert parity.check_b_partials(keys, stamps, epoch, w.n, slice_w) == want
