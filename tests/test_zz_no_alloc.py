"""The allocation-free A update (seacells_fw_a_columns_noalloc) against the
plain entry point, through the C ABI, on the GPU.

Its workspace is the library's static scratch array, shared by every call
on the GPU and rewritten by each: two calls in a row, the second smaller,
must each give the plain entry point's outputs bit for bit (the same
kernels run). Sizes whose workspace exceeds the array are refused on the
host before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import sparse_archetypal_analysis_amd as saa
import workloads as W
from sparse_archetypal_analysis_amd import native
from tests import parity
from tests.gpu_run import dev

pytestmark = pytest.mark.gpu


def _both(w, T=None):
    T = w.T if T is None else T
    ops = (dev(w.t1), dev(w.k2b), dev(w.a_prev_t))
    need = saa.seacells_fw_a_columns_workspace(w.n, w.k, T, w.cap, w.t1.nnz)
    assert 0 < need <= native.NOALLOC_SCRATCH_BYTES
    g0 = torch.full((w.n,), float("nan"), device="cuda")
    g1 = torch.full((w.n,), float("nan"), device="cuda")
    a = saa.seacells_fw_a_columns(*ops, w.n, w.k, T, w.cap, trace=True, fw_gap=g0)
    # outputs of the allocation-free call start as garbage: nothing may be
    # read from them
    ai = torch.full((w.n, w.cap), -7, dtype=torch.int32, device="cuda")
    av = torch.full((w.n, w.cap), 3.0, dtype=torch.float32, device="cuda")
    ac = torch.full((w.n,), -1, dtype=torch.int32, device="cuda")
    tr = torch.full((w.n, T), -1, dtype=torch.int32, device="cuda")
    b = saa.seacells_fw_a_columns_noalloc(*ops, w.n, w.k, T, w.cap, atom_idx=ai, atom_val=av,
                                          atom_cnt=ac, trace=tr, fw_gap=g1)
    torch.cuda.synchronize()
    assert saa.status_flags(a[4]) == [] and saa.status_flags(b[4]) == []
    cnt = a[2].cpu().numpy()
    assert np.array_equal(cnt, b[2].cpu().numpy())
    slot = np.arange(w.cap)[None, :] < cnt[:, None]
    for x, y in ((a[0], b[0]), (a[1], b[1])):
        xv, yv = x.cpu().numpy(), y.cpu().numpy()
        assert np.array_equal(xv[slot].view(np.uint32), yv[slot].view(np.uint32))
    assert torch.equal(a[3], b[3])
    assert torch.equal(g0.view(torch.int32), g1.view(torch.int32))
    return b


def test_noalloc_equals_plain_on_two_calls_in_a_row():
    # first: large k (the compact support state: queues, counters and the
    # padded t1 copy all in the scratch); second, smaller: one cell per wave
    # with the padded copy only
    big = W.random_workload(3000, 2600, t1_per_row=40, k2b_per_row=30, s_a=6, seed=91)
    small = W.random_workload(700, 1300, t1_per_row=20, k2b_per_row=12, s_a=5, seed=92)
    assert small.n * small.k < big.n * big.k
    ai, av, ac, tr, _ = _both(big)
    rep = parity.check_a(big, tr.cpu().numpy(), ai.cpu().numpy(), av.cpu().numpy(),
                         ac.cpu().numpy(), np.arange(big.n))
    print("\nfirst call: %s" % (rep,))
    ai, av, ac, tr, _ = _both(small)
    rep = parity.check_a(small, tr.cpu().numpy(), ai.cpu().numpy(), av.cpu().numpy(),
                         ac.cpu().numpy(), np.arange(small.n))
    print("second call: %s" % (rep,))


def test_noalloc_refuses_sizes_beyond_the_scratch():
    lib = saa.load()
    n, k, T, cap = 1000, 4000, 50, 60
    nnz = 2 ** 30  # the padded t1 copy alone would need 8 GB
    assert saa.seacells_fw_a_columns_workspace(n, k, T, cap, nnz) > native.NOALLOC_SCRATCH_BYTES
    t1 = native.seacells_csr(0x1000, 0x2000, 0x3000, k, k, nnz)
    k2b = native.seacells_csr(0x1000, 0x2000, 0x3000, n, k, 5)
    ap = native.seacells_csr(0x1000, 0x2000, 0x3000, n, k, 5)
    o = 0x4000
    rc = lib.seacells_fw_a_columns_noalloc(ctypes.byref(t1), ctypes.byref(k2b), ctypes.byref(ap),
                                           n, k, T, cap, None, o, o, o, None, None, 0x9000, None)
    assert rc == -4
