"""The stored B of the configs named "B after s_B prior FW steps" (CPU).

workloads/prior_b/*.npz hold B after s_B Frank-Wolfe steps of the B update
from the one-hot start (oracle/prior_b.py, the oracle's f64 B argmin and B
step). These tests pin the stored files to what they claim to be: every
column of B on the simplex with at most s_B + 1 cells, the one-hot start
still present with weight 2 / ((s+1)(s+2)) (gamma_t = 2 / (t + 2), t = 1 ..
s), the weights the step closed form gives from the stored picks, and, for
the smallest config, the whole file recomputed from the generator's inputs.
"""
import json
import os

import numpy as np
import pytest
import scipy.sparse as sp

import workloads as W

FILES = sorted(f for f in os.listdir(W.PRIOR_B_DIR) if f.endswith(".npz"))


def _load(name):
    z = np.load(os.path.join(W.PRIOR_B_DIR, name), allow_pickle=False)
    cfg = json.loads(str(z["config"]))
    bt = sp.csr_matrix((z["bt_val"], z["bt_idx"], z["bt_ptr"]), shape=(cfg["k"], cfg["n"]))
    return z, cfg, bt


@pytest.mark.parametrize("name", FILES)
def test_stored_b_is_on_the_simplex_with_the_step_weights(name):
    z, cfg, bt = _load(name)
    s = int(z["steps"])
    assert s == cfg["s_b"] and z["picks"].shape == (s, cfg["k"])
    np.testing.assert_allclose(np.asarray(bt.sum(axis=1)).ravel(), 1.0, rtol=0, atol=1e-12)
    assert np.all(bt.data > 0)
    assert np.diff(bt.indptr).max() <= s + 1
    # closed form: the start keeps prod_t (1 - gamma_t) = 2 / ((s+1)(s+2)); the
    # pick of step t adds gamma_t prod_{u > t} (1 - gamma_u) = 2 (t+1) / ((s+1)(s+2))
    g = z["gammas"]
    np.testing.assert_allclose(g, 2.0 / (np.arange(1, s + 1) + 2.0), rtol=0, atol=0)
    k, n = cfg["k"], cfg["n"]
    rows = np.tile(np.arange(k), s + 1)
    cols = np.concatenate([z["init_cells"]] + [z["picks"][t] for t in range(s)]).astype(np.int64)
    vals = np.concatenate([np.full(k, 2.0 / ((s + 1) * (s + 2)))] +
                          [np.full(k, 2.0 * (t + 1) / ((s + 1) * (s + 2))) for t in range(1, s + 1)])
    want = sp.csr_matrix((vals, (rows, cols)), shape=(k, n))
    want.sum_duplicates()
    want.sort_indices()
    np.testing.assert_array_equal(want.indptr, bt.indptr)
    np.testing.assert_array_equal(want.indices, bt.indices)
    np.testing.assert_allclose(bt.data, want.data, rtol=0, atol=1e-12)


def test_smallest_stored_b_recomputed_by_the_oracle():
    from oracle import prior_b
    cfg = W.CONFIGS["c2"]
    bs = W.base(cfg, 0)
    B, picks, mins, gammas = prior_b.prior_steps(bs.K, bs.init, bs.At, cfg.s_b)
    z, zcfg, bt = _load("c2_s0.npz")
    assert str(z["k_sha"]) == bs.sha()["K"] and str(z["a_prev_t_sha"]) == bs.sha()["a_prev_t"]
    np.testing.assert_array_equal(picks, z["picks"])
    np.testing.assert_array_equal(mins, z["min_vals"])
    mine = sp.csr_matrix(B.T)
    mine.sort_indices()
    np.testing.assert_array_equal(mine.indptr, bt.indptr)
    np.testing.assert_array_equal(mine.indices, bt.indices)
    np.testing.assert_array_equal(mine.data, bt.data)
