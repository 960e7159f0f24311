"""The B argmin's check of its partials, forced from the host (GPU).

The source page (bixverse-rs 0.6.4, seacells_kernels.rs, the
`B_ARGMIN_WG_TIERS` doc and `reduce_argmin_blocks`) names the hazard: a
reduce that trusts its partials fills the output with whatever the partial
buffers held. Here a normal B argmin leaves its partials in a caller-owned
workspace; the host then corrupts one stamp or one key in that workspace and
runs the reduce stages alone (seacells_debug_b_reduce). Each corruption must
raise PARTIALS_INVALID while every kernel runs to completion, the host
restatement of the rule (parity.check_b_partials) must agree on the same
bytes, and the untouched partials must still give the oracle's answer.
"""
import numpy as np
import pytest
import torch

import sparse_archetypal_analysis_amd as saa
import workloads as W
from tests import parity
from tests.gpu_run import dev

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "c2":   # one column slice (k <= 2048)
        return W.make("c2")
    # several column slices (k > 2048) over ragged row ranges
    return W.random_workload(1537, 5000, aat_per_row=30, k2b_per_row=12, k2at_per_row=10,
                             b_per_col=3, seed=61)


@pytest.mark.parametrize("name", ["c2", "sliced"])
def test_reduce_checks_every_partial(name):
    w = _case(name)
    n, k = w.n, w.k
    k2b, aat, k2at, b = dev(w.k2b), dev(w.aat), dev(w.k2at), dev(w.b)
    ws = torch.empty(saa.seacells_fw_b_argmin_workspace(n, k, w.aat.nnz), dtype=torch.uint8,
                     device="cuda")
    v0, i0, g0, st = saa.seacells_fw_b_argmin(k2b, aat, k2at, b, n, k, workspace=ws)
    epoch = saa.seacells_debug_b_last_epoch()
    torch.cuda.synchronize()
    assert saa.status_flags(st) == []
    rep = parity.check_b(w, v0.cpu().numpy(), i0.cpu().numpy(), float(g0.item()))
    print("\n%s: %s" % (name, rep))

    lay = saa.seacells_debug_b_layout(n, k, w.aat.nnz)
    nb, ns, sw = lay["n_row_blocks"], lay["n_slices"], lay["slice_w"]
    assert (ns > 1) == (name == "sliced")
    ko, so = lay["keys_offset"], lay["stamps_offset"]
    keys = ws[ko:ko + nb * k * 8].view(torch.int64).view(nb, k)
    stamps = ws[so:so + nb * ns * 4].view(torch.int32).view(nb, ns)

    def host_rule(ep=epoch):
        kh = keys.cpu().numpy().view(np.uint64)
        sh = stamps.cpu().numpy().view(np.uint32)
        return parity.check_b_partials(kh, sh, ep, n, sw)

    def reduce(ep=epoch):
        v, i, g, s = saa.seacells_debug_b_reduce(n, k, w.aat.nnz, ep, ws)
        torch.cuda.synchronize()  # every kernel ran to completion
        return v, i, g, saa.status_flags(s)

    # untouched partials: the reduce alone repeats the call's outputs bit for bit
    assert host_rule() == []
    v, i, g, flags = reduce()
    assert flags == []
    assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    assert torch.equal(g.view(torch.int32), g0.view(torch.int32))

    # the partials of another call
    assert host_rule(epoch + 1) == ["PARTIALS_INVALID"]
    assert reduce(epoch + 1)[3] == ["PARTIALS_INVALID"]

    # one stale stamp
    rb, sl = nb // 2, ns - 1
    keep = stamps[rb, sl].item()
    stamps[rb, sl] = (epoch - 1) & 0x7fffffff
    assert host_rule() == ["PARTIALS_INVALID"]
    assert reduce()[3] == ["PARTIALS_INVALID"]
    stamps[rb, sl] = keep

    # one key whose row is past n, and one whose row belongs to another range
    c = k - 1
    kept = keys[rb, c].item()
    hi = kept & ~0xffffffff
    for row in (n + 5, (n * (rb + 1)) // nb):
        keys[rb, c] = hi | row
        assert host_rule() == ["PARTIALS_INVALID"], row
        assert reduce()[3] == ["PARTIALS_INVALID"], row
    keys[rb, c] = kept

    # a unit that saw no finite value for a column
    keys[0, 0] = parity.NO_VALUE_KEY - (1 << 64)
    assert host_rule() == ["NONFINITE"]
    assert "NONFINITE" in reduce()[3]
    keys[0, 0] = 0
    torch.cuda.synchronize()

    # restored: the oracle's answer again, and the next call runs normally
    ws2 = ws.clone()
    saa.seacells_fw_b_argmin(k2b, aat, k2at, b, n, k, workspace=ws2)
    torch.cuda.synchronize()
    keys[:] = ws2[ko:ko + nb * k * 8].view(torch.int64).view(nb, k)
    stamps[:] = ws2[so:so + nb * ns * 4].view(torch.int32).view(nb, ns)
    v, i, g, flags = reduce(saa.seacells_debug_b_last_epoch())
    assert flags == []
    assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
