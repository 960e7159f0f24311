"""Plain f64 CPU oracle for the SEACells Frank-Wolfe hot path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
never calls it, and the two share no code: this package is C compiled with
gcc (``seacells_oracle.c``) plus dense numpy (``dense.py``), scipy sparse
products (``sparse.py``: the operand construction, sparse add, the RSS) and
the B update as a loop of Frank-Wolfe steps (``b_loop.py``), all written
from the method as the source page states it (bixverse-rs 0.6.4,
``seacells_kernels.rs``: the module doc, the ``fw_columns_a_gpu`` and
``fw_argmin_b`` docs and the ``cpu_fw_argmin_b`` test reference).

Every function here takes the same f32 CSR operands the GPU receives (as
numpy arrays or ``scipy.sparse.csr_matrix``) and computes in f64.

Parity pins: every function is pinned in ``tests/test_oracle_pins.py`` (and
``tests/test_oracle_sparse_pins.py`` for ``sparse.py``) against brute-force
objective differences, vertex enumeration, closed forms, a worked example
with K = I, special cases that reduce to library routines, brute-force loops
on tiny inputs, and the independent dense implementation in ``dense.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "seacells_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_seacells.so")

_U32P = ctypes.POINTER(ctypes.c_uint32)
_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)

ERRORS = {-1: "bad argument", -2: "index out of range", -3: "allocation failed",
          -4: "B row capacity exceeded"}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle_seacells.so``."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_fw_a_columns.restype = ctypes.c_int
    lib.oracle_fw_a_columns.argtypes = (
        [ctypes.c_uint32] * 3 + [_U32P, _U32P, _F32P] * 3 + [_F64P, _U32P, ctypes.c_uint32,
                                                              _I64P, _F64P, _U32P, _F64P, _F64P,
                                                              _F64P, _F64P, _F64P, ctypes.c_int])
    lib.oracle_fw_a_columns_pruned.restype = ctypes.c_int
    lib.oracle_fw_a_columns_pruned.argtypes = (
        [ctypes.c_uint32] * 3 + [_U32P, _U32P, _F32P] * 3 + [_F64P, _U32P, ctypes.c_uint32,
                                                              _I64P, ctypes.c_double, _F64P,
                                                              _U32P, _F64P, _F64P, _F64P, _F64P,
                                                              _F64P, _U32P, _F64P, ctypes.c_int])
    lib.oracle_fw_b_argmin.restype = ctypes.c_int
    lib.oracle_fw_b_argmin.argtypes = (
        [ctypes.c_uint32] * 2 + [_U32P, _U32P, _F32P] * 4 + [_F64P, _U32P, _F64P, _F64P, _F64P,
                                                              ctypes.c_int])
    lib.oracle_fw_b_grad_at.restype = ctypes.c_int
    lib.oracle_fw_b_grad_at.argtypes = (
        [ctypes.c_uint32] * 2 + [_U32P, _U32P, _F32P] * 3 + [_U32P, _U32P, ctypes.c_uint32,
                                                              _F64P, _F64P])
    lib.oracle_fw_b_apply.restype = ctypes.c_int
    lib.oracle_fw_b_apply.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _U32P, _F64P, _U32P,
                                      _U32P, ctypes.c_double]
    _lib = lib
    return lib


def _p(a, ptype):
    if a is None:
        return ctypes.cast(None, ptype)
    return a.ctypes.data_as(ptype)


def _csr(m, rows: int, cols: int):
    """(ptr u32, idx u32, val f32) arrays of a CSR given as scipy or a tuple."""
    if isinstance(m, tuple):
        ptr, idx, val = m
    else:
        if m.shape != (rows, cols):
            raise ValueError("operand shape %s, expected %s" % (m.shape, (rows, cols)))
        ptr, idx, val = m.indptr, m.indices, m.data
    ptr = np.ascontiguousarray(ptr, dtype=np.uint32)
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    val = np.ascontiguousarray(val, dtype=np.float32)
    if ptr.shape[0] != rows + 1:
        raise ValueError("row pointer length %d, expected %d" % (ptr.shape[0], rows + 1))
    return ptr, idx, val


def _check(rc):
    if rc != 0:
        raise RuntimeError("oracle call failed: %s (%d)" % (ERRORS.get(rc, "?"), rc))


def _threads(n_threads):
    if n_threads is not None:
        return int(n_threads)
    return len(os.sched_getaffinity(0))


@dataclass
class ATrace:
    """Result of :func:`fw_a_columns` for the listed cells."""
    cells: np.ndarray      # [m] cell indices
    a: np.ndarray          # [m, k] f64 final columns of A
    pick: np.ndarray       # [m, T] oracle argmin per step
    g_min: np.ndarray      # [m, T]
    g_second: np.ndarray   # [m, T]
    g_scale: np.ndarray    # [m, T]
    g_taken: np.ndarray    # [m, T] g at the index used for the update
    g_dot: np.ndarray = None   # [m, T] <g, a> at each step's iterate (before the update)
    drops: np.ndarray = None   # [m, T] weights dropped per step (pruned runs only)
    margin: np.ndarray = None  # [m, T] min | |a| - threshold | before the drop (pruned runs)

    @property
    def fw_gap(self) -> np.ndarray:
        """[m, T] Frank-Wolfe duality gap of each step's iterate a_t:
        <g_t, a_t> - min_c g_t[c] = max over simplex vertices e_v of
        <g_t, a_t - e_v> (g without the factor 2, as on the page)."""
        return self.g_dot - self.g_min


def fw_a_columns(t1, k2b, a_prev_t, n: int, k: int, T: int, cells=None, force=None,
                 gamma=None, n_threads=None, prune=None) -> ATrace:
    """Oracle A update for ``cells`` (default: all n cells).

    ``force`` ([len(cells), T] int, -1 = free) replays another trajectory:
    the update takes the forced index while the oracle's own argmin and the
    tie statistics are still reported for that state. ``prune`` (a
    threshold >= 0) adds the page's drop-and-renormalise step after every
    update and fills ``drops`` and ``margin``.
    """
    lib = _load()
    t1p = _csr(t1, k, k)
    k2p = _csr(k2b, n, k)
    app = _csr(a_prev_t, n, k)
    cells = np.arange(n, dtype=np.uint32) if cells is None else np.ascontiguousarray(cells, np.uint32)
    m = cells.shape[0]
    if force is not None:
        force = np.ascontiguousarray(force, dtype=np.int64)
        if force.shape != (m, T):
            raise ValueError("force must be [cells, T]")
    if gamma is not None:
        gamma = np.ascontiguousarray(gamma, dtype=np.float64)
        if gamma.shape != (T,):
            raise ValueError("gamma must be [T]")
    a = np.empty((m, k), np.float64)
    pick = np.empty((m, T), np.uint32)
    gmin, g2, gs, gt, gd = (np.empty((m, T), np.float64) for _ in range(5))
    ops = (n, k, T, _p(t1p[0], _U32P), _p(t1p[1], _U32P), _p(t1p[2], _F32P),
           _p(k2p[0], _U32P), _p(k2p[1], _U32P), _p(k2p[2], _F32P),
           _p(app[0], _U32P), _p(app[1], _U32P), _p(app[2], _F32P),
           _p(gamma, _F64P), _p(cells, _U32P), m, _p(force, _I64P))
    outs = (_p(pick, _U32P), _p(gmin, _F64P), _p(g2, _F64P), _p(gs, _F64P), _p(gt, _F64P),
            _p(gd, _F64P))
    if prune is None:
        rc = lib.oracle_fw_a_columns(*ops, _p(a, _F64P), *outs, _threads(n_threads))
        _check(rc)
        return ATrace(cells, a, pick, gmin, g2, gs, gt, gd)
    drops = np.empty((m, T), np.uint32)
    margin = np.empty((m, T), np.float64)
    rc = lib.oracle_fw_a_columns_pruned(*ops, float(prune), _p(a, _F64P), *outs,
                                        _p(drops, _U32P), _p(margin, _F64P), _threads(n_threads))
    _check(rc)
    return ATrace(cells, a, pick, gmin, g2, gs, gt, gd, drops, margin)


@dataclass
class BResult:
    val: np.ndarray        # [k] min_i G[i, c]
    row: np.ndarray        # [k] lowest argmin row
    second: np.ndarray     # [k] runner-up value
    gap: float             # sum(B * G)
    row_scale: np.ndarray  # [n]

    @property
    def fw_gap(self) -> float:
        """Full Frank-Wolfe duality gap of the B subproblem: sum(B * G) minus
        sum_c min_i G[i, c] = max over vertex matrices S (one-hot columns)
        of <G, B - S> (G without the factor 2, as on the page)."""
        return self.gap - float(np.sum(self.val))


def fw_b_argmin(k2b, aat, k2at, b, n: int, k: int, n_threads=None) -> BResult:
    """Oracle B-gradient argmin over cells for every column (B may be None)."""
    lib = _load()
    k2p = _csr(k2b, n, k)
    aap = _csr(aat, k, k)
    k2a = _csr(k2at, n, k)
    bp = _csr(b, n, k) if b is not None else (None, None, None)
    val = np.empty(k, np.float64)
    row = np.empty(k, np.uint32)
    second = np.empty(k, np.float64)
    gap = np.zeros(1, np.float64)
    rs = np.empty(n, np.float64)
    rc = lib.oracle_fw_b_argmin(
        n, k, _p(k2p[0], _U32P), _p(k2p[1], _U32P), _p(k2p[2], _F32P),
        _p(aap[0], _U32P), _p(aap[1], _U32P), _p(aap[2], _F32P),
        _p(k2a[0], _U32P), _p(k2a[1], _U32P), _p(k2a[2], _F32P),
        _p(bp[0], _U32P), _p(bp[1], _U32P), _p(bp[2], _F32P),
        _p(val, _F64P), _p(row, _U32P), _p(second, _F64P), _p(gap, _F64P), _p(rs, _F64P),
        _threads(n_threads))
    _check(rc)
    return BResult(val, row, second, float(gap[0]), rs)


def fw_b_grad_at(k2b, aat, k2at, n: int, k: int, rows, cols):
    """G[rows[e], cols[e]] from the definition, and the row term scale."""
    lib = _load()
    k2p = _csr(k2b, n, k)
    aap = _csr(aat, k, k)
    k2a = _csr(k2at, n, k)
    rows = np.ascontiguousarray(rows, np.uint32)
    cols = np.ascontiguousarray(cols, np.uint32)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    out = np.empty(rows.shape[0], np.float64)
    sc = np.empty(rows.shape[0], np.float64)
    rc = lib.oracle_fw_b_grad_at(
        n, k, _p(k2p[0], _U32P), _p(k2p[1], _U32P), _p(k2p[2], _F32P),
        _p(aap[0], _U32P), _p(aap[1], _U32P), _p(aap[2], _F32P),
        _p(k2a[0], _U32P), _p(k2a[1], _U32P), _p(k2a[2], _F32P),
        _p(rows, _U32P), _p(cols, _U32P), rows.shape[0], _p(out, _F64P), _p(sc, _F64P))
    _check(rc)
    return out, sc


def fw_b_apply(bt_idx, bt_val, bt_cnt, arg_idx, gamma: float):
    """B step on padded B^T rows (copies in, f64 values out).

    Returns (idx [k, cap_b] u32, val [k, cap_b] f64, cnt [k] u32).
    Raises on a full row, as the GPU reports it.
    """
    lib = _load()
    idx = np.array(bt_idx, dtype=np.uint32, order="C", copy=True)
    val = np.array(bt_val, dtype=np.float64, order="C", copy=True)
    cnt = np.array(bt_cnt, dtype=np.uint32, copy=True)
    arg = np.ascontiguousarray(arg_idx, np.uint32)
    k, cap_b = idx.shape
    rc = lib.oracle_fw_b_apply(k, cap_b, _p(idx, _U32P), _p(val, _F64P), _p(cnt, _U32P),
                               _p(arg, _U32P), float(gamma))
    _check(rc)
    return idx, val, cnt
