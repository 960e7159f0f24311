"""Seeded synthetic SEACells workloads: points -> kNN kernel -> FW operands.

This module produces inputs only. It holds none of the Frank-Wolfe
arithmetic (no gradient, argmin or step); the f64 oracle and the HIP library
both consume what it writes, and neither imports the other.

The pages fix no dataset. Each workload is a seeded single-cell stand-in:

* points: a C-component Gaussian mixture in d dimensions. Means are
  N(0, 4 I) (sigma 2 per coordinate). The per-component std is 1, or
  U(0.5, 2) for the larger configs. Component weights are equal, or Zipf
  r^-s for the skewed config. Labels are i.i.d. from those weights.
* kernel K: exact Euclidean kNN with the cell itself excluded and ties
  broken by index. Adaptive Gaussian weights W_ij = exp(-d_ij^2 / (s_i s_j))
  with s_i the distance to the kNN-th neighbour, then K = (W + W^T) / 2
  with K_ii = 1. K^2 is never formed: products are K (K X) in f64.
* B (n x k, column-stochastic): k distinct uniformly random init cells give
  the one-hot start. For s_B > 0 the configs name "B after s_B prior FW
  steps": that B is stored input data under ``workloads/prior_b/``, written
  once by ``oracle/prior_b.py`` (s_B Frank-Wolfe B steps of the f64 oracle
  from the one-hot start, with A = A_prev fixed). This module only loads
  it, and checks that it was made from the same K and A_prev (SHA-256 of
  both). The ``*_standin`` variants keep an earlier construction that runs
  no FW step: each column also takes s_B cells drawn uniformly, with
  replacement, from its init cell's mixture component, with Dirichlet(1)
  weights.
* A_prev (k x n, column-stochastic): column j is supported on the s_A
  archetypes whose init cells lie nearest to x_j (ties by index), with
  Dirichlet(1) weights.
* operands, built in f64 with scipy.sparse, symmetrised where the maths says
  symmetric, then cast once to f32 with sorted int32 indices and no stored
  zeros:
    t1 = B^T K^2 B (k x k), K2B = K^2 B (n x k), A_prev^T (n x k) for the A
    update; K2B, AAt = A A^T (k x k), K2At = K^2 A^T (n x k) and B for the
    B argmin.

RNG: numpy PCG64 ``default_rng(1000 * index + seed)``. Draws happen in this
order: means, scales, labels, noise, init cells, (stand-in variants only:
B supports, B weights), A weights.
"""
from __future__ import annotations

import hashlib
import json
import os
import time
from dataclasses import asdict, dataclass, field

import numpy as np
import scipy.sparse as sp

GENERATOR_VERSION = 2
_REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@dataclass(frozen=True)
class Config:
    name: str
    n: int            # cells
    d: int            # point dimension
    comps: int        # mixture components
    knn: int          # neighbours per cell in the kernel graph
    k: int            # archetypes
    s_a: int          # non-zeros per A_prev column
    s_b: int          # prior Frank-Wolfe B steps (stand-in: extra B cells per column)
    scale: tuple | None = None   # per-component std range, None = 1
    zipf: float | None = None    # component-weight exponent, None = equal
    T: int = 50                  # A steps
    index: int = 0               # RNG stream index
    b_init: str = "fw"           # "fw": stored B after s_b FW steps; "standin": random cells


CONFIGS = {
    "c1": Config("c1", 2_000, 10, 5, 15, 25, 5, 0, index=1),
    "c2": Config("c2", 20_000, 20, 10, 15, 250, 8, 3, index=2),
    "c3": Config("c3", 100_000, 30, 20, 20, 1_300, 10, 10, scale=(0.5, 2.0), index=3),
    "c4": Config("c4", 500_000, 30, 50, 20, 6_700, 12, 20, scale=(0.5, 2.0), index=4),
    "c5": Config("c5", 1_000_000, 50, 100, 30, 10_000, 16, 30, scale=(0.5, 2.0), zipf=1.1,
                 index=5),
}
# the earlier B construction (no FW step), same points, kernel and init cells
for _nm in ("c2", "c3", "c4", "c5"):
    _c = CONFIGS[_nm]
    CONFIGS[_nm + "_standin"] = Config(**{**asdict(_c), "name": _nm + "_standin",
                                          "b_init": "standin"})

DESCRIPTIONS = {
    "c1": "n=2000 d=10 C=5 kNN=15 k=25 s_A=5 B one-hot T=50",
    "c2": "n=20000 d=20 C=10 kNN=15 k=250 s_A=8 B after 3 FW steps T=50",
    "c3": "n=100000 d=30 C=20 std~U(0.5,2) kNN=20 k=1300 s_A=10 B after 10 FW steps T=50",
    "c4": "n=500000 d=30 C=50 std~U(0.5,2) kNN=20 k=6700 s_A=12 B after 20 FW steps T=50",
    "c5": "n=1000000 d=50 C=100 Zipf(1.1) std~U(0.5,2) kNN=30 k=10000 s_A=16 "
          "B after 30 FW steps T=50",
}
for _nm in ("c2", "c3", "c4", "c5"):
    DESCRIPTIONS[_nm + "_standin"] = DESCRIPTIONS[_nm].split(" B after")[0] + \
        " B stand-in (%d random same-component cells, Dirichlet(1)) T=50" % CONFIGS[_nm].s_b


@dataclass
class Workload:
    cfg: Config
    seed: int
    t1: sp.csr_matrix          # k x k, f32, symmetric
    k2b: sp.csr_matrix         # n x k, f32
    a_prev_t: sp.csr_matrix    # n x k, f32 (rows are columns of A_prev)
    aat: sp.csr_matrix         # k x k, f32, symmetric
    k2at: sp.csr_matrix        # n x k, f32
    b: sp.csr_matrix           # n x k, f32
    init_cells: np.ndarray     # [k]
    meta: dict = field(default_factory=dict)
    K: sp.csr_matrix | None = None  # n x n, f32, symmetric (None: not kept, see kernel_matrix)

    @property
    def n(self):
        return self.cfg.n

    @property
    def k(self):
        return self.cfg.k

    @property
    def T(self):
        return self.cfg.T

    @property
    def cap(self):
        """Atom capacity: widest A_prev column plus one append per step."""
        widest = int(np.diff(self.a_prev_t.indptr).max()) if self.n else 0
        return widest + self.cfg.T


# --------------------------------------------------------------------------
# points and kernel
# --------------------------------------------------------------------------

def _points(cfg: Config, rng):
    C, d, n = cfg.comps, cfg.d, cfg.n
    means = rng.normal(0.0, 2.0, size=(C, d))
    if cfg.scale is None:
        scales = np.ones(C)
    else:
        scales = rng.uniform(cfg.scale[0], cfg.scale[1], size=C)
    if cfg.zipf is None:
        w = np.full(C, 1.0 / C)
    else:
        w = np.arange(1, C + 1, dtype=np.float64) ** (-cfg.zipf)
        w /= w.sum()
    labels = rng.choice(C, size=n, p=w)
    noise = rng.normal(0.0, 1.0, size=(n, d))
    X = means[labels] + scales[labels, None] * noise
    return X, labels


def _nearest(Q, P, kk, exclude_self=False, margin=8, block=2048):
    """Exact kk nearest rows of P for every row of Q (Euclidean, f64).

    Candidates come from an f32 pass on torch (GPU when present); the top
    kk + margin candidates are re-ranked by exact f64 distance with ties
    broken by index, so the result does not depend on the device.
    """
    import torch

    dev = "cuda" if torch.cuda.is_available() else "cpu"
    nq, npnt = Q.shape[0], P.shape[0]
    m = min(kk + margin, npnt - (1 if exclude_self else 0))
    Pt = torch.from_numpy(P.astype(np.float32)).to(dev)
    psq = (Pt * Pt).sum(1)
    Qt_all = torch.from_numpy(Q.astype(np.float32))
    cand = np.empty((nq, m), np.int64)
    for s in range(0, nq, block):
        e = min(nq, s + block)
        q = Qt_all[s:e].to(dev)
        d2 = (q * q).sum(1)[:, None] + psq[None, :] - 2.0 * (q @ Pt.T)
        if exclude_self:
            r = torch.arange(e - s, device=dev)
            d2[r, r + s] = float("inf")
        _, idx = torch.topk(d2, m, dim=1, largest=False, sorted=False)
        cand[s:e] = idx.cpu().numpy()
    # exact re-rank
    out_i = np.empty((nq, kk), np.int64)
    out_d = np.empty((nq, kk), np.float64)
    for s in range(0, nq, 16384):
        e = min(nq, s + 16384)
        c = cand[s:e]
        diff = Q[s:e, None, :] - P[c]
        dd = np.einsum("ijk,ijk->ij", diff, diff)
        # sort by (distance, index): index first, then a stable sort on distance
        o1 = np.argsort(c, axis=1, kind="stable")
        c1 = np.take_along_axis(c, o1, 1)
        d1 = np.take_along_axis(dd, o1, 1)
        o2 = np.argsort(d1, axis=1, kind="stable")[:, :kk]
        out_i[s:e] = np.take_along_axis(c1, o2, 1)
        out_d[s:e] = np.take_along_axis(d1, o2, 1)
    return out_i, out_d


def _kernel(X, knn):
    n = X.shape[0]
    nb, d2 = _nearest(X, X, knn, exclude_self=True)
    sig = np.sqrt(d2[:, -1])
    sig = np.where(sig > 0, sig, 1.0)
    rows = np.repeat(np.arange(n), knn)
    cols = nb.ravel()
    w = np.exp(-d2.ravel() / (sig[rows] * sig[cols]))
    W = sp.csr_matrix((w, (rows, cols)), shape=(n, n))
    # the cell itself is excluded from its neighbours, so the diagonal of W
    # is structurally empty and adding I sets K_ii = 1
    K = ((W + W.T) * 0.5 + sp.identity(n, format="csr")).tocsr()
    K.sum_duplicates()
    K.sort_indices()
    return K


# --------------------------------------------------------------------------
# B, A_prev and operands
# --------------------------------------------------------------------------

def _b_matrix(cfg: Config, rng, labels, init):
    n, k = cfg.n, cfg.k
    members = [np.flatnonzero(labels == c) for c in range(cfg.comps)]
    supports = []
    for c in range(k):
        cells = [int(init[c])]
        if cfg.s_b > 0:
            pool = members[labels[init[c]]]
            cells.extend(int(x) for x in rng.choice(pool, size=cfg.s_b, replace=True))
        supports.append(np.unique(np.asarray(cells, np.int64)))
    rows, cols, vals = [], [], []
    for c, sup in enumerate(supports):
        wts = rng.dirichlet(np.ones(sup.shape[0])) if sup.shape[0] > 1 else np.ones(1)
        rows.append(sup)
        cols.append(np.full(sup.shape[0], c))
        vals.append(wts)
    return sp.csr_matrix((np.concatenate(vals), (np.concatenate(rows), np.concatenate(cols))),
                         shape=(n, k))


def _a_prev_t(cfg: Config, rng, X, init):
    n, k = cfg.n, cfg.k
    s_a = min(cfg.s_a, k)
    nb, _ = _nearest(X, X[init], s_a, exclude_self=False)
    wts = rng.dirichlet(np.ones(s_a), size=n)
    rows = np.repeat(np.arange(n), s_a)
    return sp.csr_matrix((wts.ravel(), (rows, nb.ravel())), shape=(n, k))


_SPGEMM_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_spgemm.c")
_SPGEMM_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspgemm.so")
_spgemm_lib = None


def build_spgemm(force: bool = True) -> str:
    """Compile the generator's sparse-product helper (gcc, OpenMP)."""
    import subprocess
    if force or not os.path.exists(_SPGEMM_LIB) or \
            os.path.getmtime(_SPGEMM_LIB) < os.path.getmtime(_SPGEMM_SRC):
        tmp = _SPGEMM_LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
                        _SPGEMM_SRC], check=True)
        os.replace(tmp, _SPGEMM_LIB)
    return _SPGEMM_LIB


def _spgemm_load():
    global _spgemm_lib
    if _spgemm_lib is None:
        import ctypes
        build_spgemm(force=False)
        lib = ctypes.CDLL(_SPGEMM_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.spgemm_count.argtypes = [I, I, P, P, P, P, P]
        lib.spgemm_fill.argtypes = [I, I, P, P, P, P, P, P, P, P, P, P]
        _spgemm_lib = lib
    return _spgemm_lib


def _matmul(A: sp.csr_matrix, B: sp.csr_matrix) -> sp.csr_matrix:
    """A @ B in f64 with the values scipy's product gives (same summation
    order), sorted columns and no stored zeros, over all host cores."""
    lib = _spgemm_load()
    A = sp.csr_matrix(A, dtype=np.float64)
    B = sp.csr_matrix(B, dtype=np.float64)
    ap = np.ascontiguousarray(A.indptr, np.int64)
    ai = np.ascontiguousarray(A.indices, np.int32)
    av = np.ascontiguousarray(A.data, np.float64)
    bp = np.ascontiguousarray(B.indptr, np.int64)
    bi = np.ascontiguousarray(B.indices, np.int32)
    bv = np.ascontiguousarray(B.data, np.float64)
    n, m = A.shape[0], B.shape[1]
    cnt = np.empty(n, np.int64)
    P = lambda a: a.ctypes.data
    if lib.spgemm_count(n, m, P(ap), P(ai), P(bp), P(bi), P(cnt)) != 0:
        raise MemoryError("sparse product: out of memory")
    cp = np.zeros(n + 1, np.int64)
    np.cumsum(cnt, out=cp[1:])
    ci = np.empty(int(cp[-1]), np.int32)
    cv = np.empty(int(cp[-1]), np.float64)
    kept = np.empty(n, np.int64)
    if lib.spgemm_fill(n, m, P(ap), P(ai), P(av), P(bp), P(bi), P(bv), P(cp), P(ci), P(cv),
                       P(kept)) != 0:
        raise MemoryError("sparse product: out of memory")
    if not np.array_equal(kept, cnt):  # exact zeros were dropped: close the gaps
        keep = np.arange(ci.shape[0]) - np.repeat(cp[:-1], cnt) < np.repeat(kept, cnt)
        ci, cv = ci[keep], cv[keep]
        cp = np.zeros(n + 1, np.int64)
        np.cumsum(kept, out=cp[1:])
    out = sp.csr_matrix((cv, ci, cp), shape=(n, m))
    out.has_sorted_indices = True
    return out


def _f32(m, symmetric=False):
    m = sp.csr_matrix(m, dtype=np.float64)
    if symmetric:
        m = sp.csr_matrix((m + m.T) * 0.5)
    m.sum_duplicates()
    m.sort_indices()
    out = sp.csr_matrix((m.data.astype(np.float32), m.indices, m.indptr), shape=m.shape)
    out.eliminate_zeros()
    out.sort_indices()
    if out.nnz >= 2 ** 31:
        raise ValueError("operand has 2^31 or more non-zeros")
    out.indices = out.indices.astype(np.int32)
    out.indptr = out.indptr.astype(np.int32)
    return out


def _sha(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def _progress(log, what, t0):
    if log is not None:
        log("[workload] %s done at %.1f s" % (what, time.time() - t0))


PRIOR_B_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "prior_b")


def prior_b_path(cfg: Config, seed: int = 0) -> str:
    """Where the stored B after cfg.s_b prior FW steps lives."""
    return os.path.join(PRIOR_B_DIR, "%s_s%d.npz" % (cfg.name, seed))


@dataclass
class Base:
    """The inputs every operand is built from: K (n x n, f64, symmetric),
    the k init cells, A_prev^T (n x k, f64) and, for the stand-in variants,
    B (n x k, f64). No Frank-Wolfe arithmetic went into any of them."""
    cfg: Config
    seed: int
    K: sp.csr_matrix
    init: np.ndarray
    At: sp.csr_matrix
    B_standin: sp.csr_matrix | None
    seconds: dict

    def sha(self) -> dict:
        """SHA-256 of K and A_prev^T as their f32 CSR operands."""
        k32, a32 = _f32(self.K), _f32(self.At)
        return {"K": _sha(k32.indptr, k32.indices, k32.data),
                "a_prev_t": _sha(a32.indptr, a32.indices, a32.data)}


def base(cfg: Config, seed: int = 0, log=None) -> Base:
    """Points, kernel, init cells and A_prev (and the stand-in B)."""
    t0 = time.time()
    rng = np.random.default_rng(1000 * cfg.index + seed)
    X, labels = _points(cfg, rng)
    t_pts = time.time()
    _progress(log, "points", t0)
    K = _kernel(X, cfg.knn)
    t_knn = time.time()
    _progress(log, "kNN kernel (%d nnz)" % K.nnz, t0)
    init = rng.choice(cfg.n, size=cfg.k, replace=False)
    Bs = _b_matrix(cfg, rng, labels, init) if cfg.b_init == "standin" else None
    At = _a_prev_t(cfg, rng, X, init)
    _progress(log, "init cells and A_prev", t0)
    return Base(cfg, seed, K, np.asarray(init, np.int64), At, Bs,
                {"points": t_pts - t0, "kernel": t_knn - t_pts, "init_a": time.time() - t_knn})


def one_hot_b(n: int, init) -> sp.csr_matrix:
    """The one-hot start of B: column c is e_{init[c]} (n x k, f64)."""
    k = len(init)
    return sp.csr_matrix((np.ones(k), (np.asarray(init, np.int64), np.arange(k))), shape=(n, k))


def k2_times(K: sp.csr_matrix, X: sp.csr_matrix) -> sp.csr_matrix:
    """K (K X) in f64 (the kernel construction's product; K^2 is never formed)."""
    return _matmul(K, _matmul(K, X))


def load_prior_b(bs: Base) -> sp.csr_matrix:
    """The stored B after cfg.s_b prior FW steps (n x k, f64), checked
    against the K and A_prev it was computed from."""
    cfg = bs.cfg
    path = prior_b_path(cfg, bs.seed)
    if not os.path.exists(path):
        raise FileNotFoundError(
            "%s is missing: the B after %d prior FW steps of config %s is written by "
            "`python -m oracle.prior_b %s`" % (path, cfg.s_b, cfg.name, cfg.name))
    z = np.load(path, allow_pickle=False)
    want = bs.sha()
    got = {"K": str(z["k_sha"]), "a_prev_t": str(z["a_prev_t_sha"])}
    if got != want:
        raise ValueError("%s was computed from another K or A_prev (SHA-256 %s, these inputs %s); "
                         "rerun `python -m oracle.prior_b %s`" % (path, got, want, cfg.name))
    if int(z["steps"]) != cfg.s_b:
        raise ValueError("%s holds %d steps, config %s names %d"
                         % (path, int(z["steps"]), cfg.name, cfg.s_b))
    bt = sp.csr_matrix((z["bt_val"], z["bt_idx"], z["bt_ptr"]), shape=(cfg.k, cfg.n))
    return sp.csr_matrix(bt.T)


def operands(K: sp.csr_matrix, B: sp.csr_matrix, At: sp.csr_matrix, log=None, t0=None) -> dict:
    """The f32 operands of both updates from K, B and A_prev^T (products in
    f64, symmetrised where the maths is symmetric, one cast to f32)."""
    t0 = time.time() if t0 is None else t0
    K2B = k2_times(K, B)
    t1 = B.T @ K2B
    _progress(log, "K2B and t1", t0)
    K2At = k2_times(K, At)
    AAt = At.T @ At
    _progress(log, "K2At and AAt", t0)
    return {"t1": _f32(t1, symmetric=True), "k2b": _f32(K2B), "a_prev_t": _f32(At),
            "aat": _f32(AAt, symmetric=True), "k2at": _f32(K2At), "b": _f32(B)}


def generate(cfg: Config, seed: int = 0, log=None) -> Workload:
    """Build one workload. ``log`` (optional) receives one line per stage."""
    t0 = time.time()
    bs = base(cfg, seed, log)
    if cfg.s_b == 0:
        B, b_note = one_hot_b(cfg.n, bs.init), "one-hot at the init cells"
    elif cfg.b_init == "standin":
        B = bs.B_standin
        b_note = "stand-in: init cell plus %d random same-component cells, Dirichlet(1)" % cfg.s_b
    else:
        B = load_prior_b(bs)
        b_note = "after %d FW steps from the one-hot start (stored, %s)" % (
            cfg.s_b, os.path.relpath(prior_b_path(cfg, seed), _REPO))
    t_b = time.time()
    ops = operands(bs.K, B, bs.At, log, t0)
    w = Workload(cfg, seed, init_cells=bs.init, K=_f32(bs.K), **ops)
    t_end = time.time()
    _progress(log, "f32 operands", t0)
    w.meta = {
        "generator_version": GENERATOR_VERSION,
        "config": asdict(cfg),
        "seed": seed,
        "b_init": b_note,
        "seconds": dict(bs.seconds, operands=t_end - t_b),
        "nnz": {nm: int(getattr(w, nm).nnz) for nm in ("t1", "k2b", "a_prev_t", "aat", "k2at", "b")},
        "nnz_K": int(w.K.nnz),
        "sha256": {nm: _sha(getattr(w, nm).indptr, getattr(w, nm).indices, getattr(w, nm).data)
                   for nm in ("t1", "k2b", "a_prev_t", "aat", "k2at", "b")},
    }
    return w


# --------------------------------------------------------------------------
# cache
# --------------------------------------------------------------------------

def cache_dir():
    return os.environ.get("SEACELLS_WORKLOAD_CACHE", os.path.join(_REPO, ".cache", "workloads"))


_NAMES = ("t1", "k2b", "a_prev_t", "aat", "k2at", "b")


def _save(w: Workload, path):
    arrs = {"init_cells": w.init_cells}
    for nm in _NAMES + (("K",) if w.K is not None else ()):
        m = getattr(w, nm)
        arrs[nm + "_ptr"], arrs[nm + "_idx"], arrs[nm + "_val"] = m.indptr, m.indices, m.data
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tmp = path + ".tmp%d.npz" % os.getpid()
    np.savez(tmp, **arrs)
    os.replace(tmp, path)
    with open(path + ".json", "w") as f:
        json.dump(w.meta, f, indent=1)


def _load(cfg: Config, seed: int, path) -> Workload:
    z = np.load(path, allow_pickle=False)
    n, k = cfg.n, cfg.k
    shapes = {"t1": (k, k), "k2b": (n, k), "a_prev_t": (n, k), "aat": (k, k), "k2at": (n, k),
              "b": (n, k)}
    mats = {nm: sp.csr_matrix((z[nm + "_val"], z[nm + "_idx"], z[nm + "_ptr"]), shape=shapes[nm])
            for nm in _NAMES}
    if "K_ptr" in z.files:
        mats["K"] = sp.csr_matrix((z["K_val"], z["K_idx"], z["K_ptr"]), shape=(n, n))
    with open(path + ".json") as f:
        meta = json.load(f)
    return Workload(cfg, seed, init_cells=z["init_cells"], meta=meta, **mats)


def kernel_matrix(w: Workload) -> sp.csr_matrix:
    """K of a workload (f32, symmetric), rebuilt from its points when the
    workload was loaded from a cache written without it."""
    if w.K is None:
        rng = np.random.default_rng(1000 * w.cfg.index + w.seed)
        X, _ = _points(w.cfg, rng)
        w.K = _f32(_kernel(X, w.cfg.knn))
    return w.K


def make(name_or_cfg, seed: int = 0, cache: bool = True, log=None) -> Workload:
    """The workload for a named config ("c1".."c5") or a custom Config.

    ``log`` (optional, e.g. a print to stderr) receives one line per stage
    when the workload has to be generated.
    """
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if not cache:
        return generate(cfg, seed, log)
    key = "%s_n%d_k%d_s%d_v%d.npz" % (cfg.name, cfg.n, cfg.k, seed, GENERATOR_VERSION)
    path = os.path.join(cache_dir(), key)
    prior = _file_sha(prior_b_path(cfg, seed)) if cfg.s_b > 0 and cfg.b_init == "fw" else None
    if os.path.exists(path) and os.path.exists(path + ".json"):
        with open(path + ".json") as f:
            meta = json.load(f)
        if meta.get("config") == json.loads(json.dumps(asdict(cfg))) and \
                meta.get("prior_b_file_sha") == prior:
            return _load(cfg, seed, path)
    w = generate(cfg, seed, log)
    w.meta["prior_b_file_sha"] = prior
    _save(w, path)
    return w


def _file_sha(path):
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    with open(path, "rb") as f:
        h.update(f.read())
    return h.hexdigest()


# --------------------------------------------------------------------------
# layout helpers (no arithmetic)
# --------------------------------------------------------------------------

def bt_padded(b: sp.csr_matrix, cap_b: int):
    """B (n x k CSR) as padded B^T rows: idx [k, cap_b] u32, val [k, cap_b] f32, cnt [k]."""
    bt = sp.csr_matrix(b.T)
    bt.sort_indices()
    k = bt.shape[0]
    cnt = np.diff(bt.indptr).astype(np.uint32)
    if k and int(cnt.max()) > cap_b:
        raise ValueError("cap_b %d below the widest B column %d" % (cap_b, int(cnt.max())))
    idx = np.zeros((k, cap_b), np.uint32)
    val = np.zeros((k, cap_b), np.float32)
    for c in range(k):
        s, e = bt.indptr[c], bt.indptr[c + 1]
        idx[c, : e - s] = bt.indices[s:e]
        val[c, : e - s] = bt.data[s:e]
    return idx, val, cnt


# --------------------------------------------------------------------------
# the source page's deterministic test fixtures
# --------------------------------------------------------------------------

def page_fixture(length: int, seed: int, zero_every: int) -> np.ndarray:
    """The page's dense test fixture (test helper `fixture` of
    bixverse-rs 0.6.4, seacells_kernels.rs): value ((37 i + 17 seed) mod 23
    - 11) * 0.1 computed in f32, zero wherever (i + seed) is a multiple of
    zero_every. Values are signed."""
    i = np.arange(length, dtype=np.int64)
    v = (np.float32(1.0) * ((i * 37 + seed * 17) % 23).astype(np.float32) - np.float32(11.0)) \
        * np.float32(0.1)
    v = v.astype(np.float32)
    v[(i + seed) % zero_every == 0] = np.float32(0.0)
    return v


def dense_to_csr(a: np.ndarray) -> sp.csr_matrix:
    """Row-major dense f32 to CSR keeping only non-zero entries (int32 indices)."""
    m = sp.csr_matrix(np.asarray(a, np.float32))
    m.eliminate_zeros()
    m.sort_indices()
    m.indices = m.indices.astype(np.int32)
    m.indptr = m.indptr.astype(np.int32)
    return m


# --------------------------------------------------------------------------
# random sparse operands for shape and edge cases (no kernel construction)
# --------------------------------------------------------------------------

def _rand_csr(rng, rows, cols, per_row, signed=False, empty_every=0, lo=0.05, hi=1.0):
    per_row = max(0, min(per_row, cols))
    indptr = [0]
    indices, data = [], []
    for r in range(rows):
        if empty_every and r % empty_every == 0:
            indptr.append(len(indices))
            continue
        cnt = int(rng.integers(0, 2 * per_row + 1)) if per_row else 0
        cnt = min(cnt, cols)
        cs = np.sort(rng.choice(cols, size=cnt, replace=False))
        vs = rng.uniform(lo, hi, size=cnt)
        if signed:
            vs *= rng.choice([-1.0, 1.0], size=cnt)
        indices.extend(cs.tolist())
        data.extend(vs.tolist())
        indptr.append(len(indices))
    return sp.csr_matrix((np.asarray(data, np.float64), np.asarray(indices, np.int64),
                          np.asarray(indptr, np.int64)), shape=(rows, cols))


def random_workload(n: int, k: int, t1_per_row: int = 8, k2b_per_row: int = 6, s_a: int = 4,
                    T: int = 50, seed: int = 0, signed: bool = False, empty_k2b_every: int = 0,
                    empty_ap_every: int = 0, aat_per_row: int = 8, k2at_per_row: int = 6,
                    b_per_col: int = 3) -> Workload:
    """Random sparse operands of the right shapes and symmetry, for cases the
    kernel-based workloads do not reach (large k with tiny n, empty rows,
    signed values, ragged sizes). Values are uniform in [0.05, 1) (times a
    random sign when ``signed``); A_prev rows are Dirichlet(1) on random
    supports; B columns are Dirichlet(1) on random cells."""
    rng = np.random.default_rng(seed)
    t1 = _rand_csr(rng, k, k, t1_per_row, signed)
    k2b = _rand_csr(rng, n, k, k2b_per_row, signed, empty_every=empty_k2b_every)
    aat = _rand_csr(rng, k, k, aat_per_row, signed)
    k2at = _rand_csr(rng, n, k, k2at_per_row, signed)
    rows, cols, vals = [], [], []
    for j in range(n):
        if empty_ap_every and j % empty_ap_every == 0:
            continue
        s = min(s_a, k)
        sup = np.sort(rng.choice(k, size=s, replace=False))
        rows.extend([j] * s)
        cols.extend(sup.tolist())
        vals.extend(rng.dirichlet(np.ones(s)).tolist())
    ap = sp.csr_matrix((vals, (rows, cols)), shape=(n, k))
    brow, bcol, bval = [], [], []
    for c in range(k):
        s = min(b_per_col, n)
        sup = rng.choice(n, size=s, replace=False)
        brow.extend(sup.tolist())
        bcol.extend([c] * s)
        bval.extend(rng.dirichlet(np.ones(s)).tolist())
    b = sp.csr_matrix((bval, (brow, bcol)), shape=(n, k))
    cfg = Config("random", n, 0, 0, 0, k, s_a, b_per_col, T=T, index=0)
    return Workload(cfg, seed, t1=_f32(t1, symmetric=True), k2b=_f32(k2b), a_prev_t=_f32(ap),
                    aat=_f32(aat, symmetric=True), k2at=_f32(k2at), b=_f32(b),
                    init_cells=np.zeros(0, np.int64), meta={"random": True})
