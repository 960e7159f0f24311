"""Writes the stored B of the configs that name "B after s_B prior FW steps".

TEST INFRASTRUCTURE (see ``oracle/__init__.py``), run by hand, offline:

    python -m oracle.prior_b c2 c3 c4 c5

For each named config it takes the generator's inputs (K, the k init cells,
A_prev; ``workloads.base``), starts from the one-hot B at the init cells and
runs s_B Frank-Wolfe steps of the B update with A = A_prev fixed, t = 1 ..
s_B:

    K^2 B_t   = K (K B_t)                 (the generator's f64 product, cast
                                           once to f32 like every operand)
    i_c       = the oracle's B argmin of G = K^2 B_t A A^T - K^2 A^T over
                cells, column by column (``oracle.fw_b_argmin``, f64)
    B_{t+1}   = (1 - gamma_t) B_t + gamma_t e_{i_c} per column
                (``oracle.fw_b_apply``, f64), gamma_t = 2 / (t + 2)

Source of the method: bixverse-rs 0.6.4, ``seacells_kernels.rs``, the
``fw_argmin_b`` doc (the B-update gradient and its column argmin with the
lowest row winning a tie). Numbering the prior steps from t = 1 keeps the
one-hot start with weight 2 / ((s+1)(s+2)), so a column holds at most
s_B + 1 cells.

The result goes to ``workloads/prior_b/<config>_s<seed>.npz``: B^T as CSR
with f64 weights, the picks and minimum values of every step, and the
SHA-256 of the f32 K and A_prev^T it was computed from (the generator
refuses the file for other inputs). The generator loads that B and holds no
Frank-Wolfe arithmetic itself.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import scipy.sparse as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def _u32(m: sp.csr_matrix):
    """(ptr, idx, val) as the oracle reads them, converted once."""
    return (np.ascontiguousarray(m.indptr, np.uint32), np.ascontiguousarray(m.indices, np.uint32),
            np.ascontiguousarray(m.data, np.float32))


def b_from_padded(idx, val, cnt, n: int) -> sp.csr_matrix:
    """Padded B^T rows (oracle.fw_b_apply's layout) as B, n x k, f64."""
    k = idx.shape[0]
    rows = np.concatenate([idx[c, :cnt[c]] for c in range(k)]).astype(np.int64)
    cols = np.repeat(np.arange(k), cnt.astype(np.int64))
    vals = np.concatenate([val[c, :cnt[c]] for c in range(k)])
    return sp.csr_matrix((vals, (rows, cols)), shape=(n, k))


def prior_steps(K: sp.csr_matrix, init, At: sp.csr_matrix, steps: int, n_threads=None,
                log=None, checkpoint=None, key=None):
    """s FW steps of the B update from the one-hot start at ``init``.

    ``checkpoint`` (a path): the state after every step is saved there, and a
    run resumes from it when it holds the state of the same inputs (``key``).
    Returns (B n x k f64 CSR, picks [s, k], min values [s, k], gammas [s])."""
    n, k = K.shape[0], len(init)
    aat = _u32(W._f32(At.T @ At, symmetric=True))
    k2at = _u32(W._f32(W.k2_times(K, At)))
    cap = steps + 1
    idx = np.zeros((k, cap), np.uint32)
    val = np.zeros((k, cap), np.float64)
    cnt = np.ones(k, np.uint32)
    idx[:, 0] = np.asarray(init, np.uint32)
    val[:, 0] = 1.0
    picks = np.zeros((steps, k), np.uint32)
    mins = np.zeros((steps, k), np.float64)
    gammas = np.zeros(steps, np.float64)
    done = 0
    if checkpoint is not None and os.path.exists(checkpoint):
        z = np.load(checkpoint, allow_pickle=False)
        if str(z["key"]) == key and z["idx"].shape == idx.shape:
            idx, val, cnt = z["idx"], z["val"], z["cnt"]
            picks, mins, gammas = z["picks"], z["mins"], z["gammas"]
            done = int(z["done"])
            if log is not None:
                log("[prior_b] resuming after step %d from %s" % (done, checkpoint))
    t0 = time.time()
    for t in range(done + 1, steps + 1):
        B = b_from_padded(idx, val, cnt, n)
        k2b = W._f32(W.k2_times(K, B))
        r = oracle.fw_b_argmin(_u32(k2b), aat, k2at, None, n, k, n_threads=n_threads)
        g = 2.0 / (t + 2.0)
        idx, val, cnt = oracle.fw_b_apply(idx, val, cnt, r.row, g)
        picks[t - 1], mins[t - 1], gammas[t - 1] = r.row, r.val, g
        if checkpoint is not None:
            tmp = checkpoint + ".tmp.npz"
            np.savez(tmp, idx=idx, val=val, cnt=cnt, picks=picks, mins=mins, gammas=gammas,
                     done=np.int64(t), key=np.str_(key))
            os.replace(tmp, checkpoint)
        if log is not None:
            log("[prior_b] step %d/%d: K2B %d nnz, B %d nnz, %.1f s"
                % (t, steps, k2b.nnz, int(cnt.sum()), time.time() - t0))
    return b_from_padded(idx, val, cnt, n), picks, mins, gammas


def write(name: str, seed: int = 0, n_threads=None, log=print, out_dir=None,
          checkpoint_dir=None) -> str:
    """Run the prior steps of config ``name`` and store B (under
    ``workloads/prior_b/``, or ``out_dir``)."""
    cfg = W.CONFIGS[name]
    if cfg.s_b == 0 or cfg.b_init != "fw":
        raise ValueError("config %s has no prior FW steps" % name)
    bs = W.base(cfg, seed, log)
    sha = bs.sha()
    ckpt = None
    if checkpoint_dir is not None:
        os.makedirs(checkpoint_dir, exist_ok=True)
        ckpt = os.path.join(checkpoint_dir, "prior_b_%s_s%d.ckpt.npz" % (name, seed))
    B, picks, mins, gammas = prior_steps(bs.K, bs.init, bs.At, cfg.s_b, n_threads, log,
                                         checkpoint=ckpt, key=sha["K"] + sha["a_prev_t"])
    bt = sp.csr_matrix(B.T)
    bt.sort_indices()
    path = W.prior_b_path(cfg, seed)
    if out_dir is not None:
        path = os.path.join(out_dir, os.path.basename(path))
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tmp = path + ".tmp%d.npz" % os.getpid()
    np.savez_compressed(tmp, bt_ptr=bt.indptr.astype(np.int64), bt_idx=bt.indices.astype(np.int32),
                        bt_val=bt.data.astype(np.float64), picks=picks, min_vals=mins,
                        gammas=gammas, init_cells=np.asarray(bs.init, np.int64),
                        steps=np.int64(cfg.s_b), k_sha=np.str_(sha["K"]),
                        a_prev_t_sha=np.str_(sha["a_prev_t"]),
                        config=np.str_(json.dumps({"name": cfg.name, "n": cfg.n, "k": cfg.k,
                                                   "s_b": cfg.s_b, "seed": seed,
                                                   "generator_version": W.GENERATOR_VERSION})))
    os.replace(tmp, path)
    log("[prior_b] %s: B %d nnz (max %d per column) -> %s"
        % (name, bt.nnz, int(np.diff(bt.indptr).max()), path))
    return path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("configs", nargs="*", default=["c2", "c3", "c4", "c5"])
    ap.add_argument("--out-dir", default=None, help="write there instead of workloads/prior_b")
    ap.add_argument("--checkpoint-dir", default=None,
                    help="save the state after every step there, and resume from it")
    a = ap.parse_args()
    for nm in a.configs:
        write(nm, log=lambda m: print(m, flush=True), out_dir=a.out_dir,
              checkpoint_dir=a.checkpoint_dir)
