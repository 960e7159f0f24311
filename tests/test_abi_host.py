"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import sparse_archetypal_analysis_amd as saa
from sparse_archetypal_analysis_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            src = open(os.path.join(inc, fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(seacells_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = saa.load()
    names = header_functions()
    assert set(names) == set(native.EXPORTS)
    for nm in names:
        assert hasattr(lib, nm), nm


def test_package_exports_every_wrapped_entry_point():
    wrapped = [nm for nm in native.EXPORTS if hasattr(native, nm)]
    assert len(wrapped) >= len(native.EXPORTS) - 3  # status/error/version have no wrapper
    for nm in wrapped:
        assert hasattr(saa, nm), nm


def test_version_and_status_strings():
    lib = saa.load()
    assert lib.seacells_version() >> 16 == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.seacells_status_string(code) != b"unknown status"
    assert lib.seacells_status_string(7) == b"unknown status"
    assert lib.seacells_last_error() == b""


def csr(rows, cols, nnz=0, ptr=0x1000):
    return native.seacells_csr(ptr, 0x2000 if nnz else None, 0x3000 if nnz else None, rows, cols,
                               nnz)


def call_a(t1, k2b, ap, n, k, T, cap, ws=None, ws_bytes=0, outs=True, status=0x9000):
    lib = saa.load()
    o = 0x4000 if outs else None
    return lib.seacells_fw_a_columns(ctypes.byref(t1) if t1 else None,
                                     ctypes.byref(k2b) if k2b else None,
                                     ctypes.byref(ap) if ap else None, n, k, T, cap, None, o, o,
                                     o, None, None, ws, ws_bytes, status, None)


def test_a_columns_rejects_bad_arguments_on_host():
    n, k, T, cap = 10, 4, 5, 8
    t1, k2b, ap = csr(k, k, 3), csr(n, k, 5), csr(n, k, 5)
    assert call_a(None, k2b, ap, n, k, T, cap) == -1
    assert call_a(t1, k2b, ap, n, k, T, cap, outs=False) == -1
    assert call_a(t1, k2b, ap, n, k, T, cap, status=None) == -1
    assert call_a(t1, k2b, ap, 0, k, T, cap) == -2
    assert call_a(t1, k2b, ap, n, k, 0, cap) == -2
    assert call_a(t1, k2b, ap, n, k, T, 0) == -2
    assert call_a(csr(k + 1, k, 3), k2b, ap, n, k, T, cap) == -2
    assert call_a(t1, csr(n, k + 1, 5), ap, n, k, T, cap) == -2
    assert call_a(t1, k2b, csr(n - 1, k, 5), n, k, T, cap) == -2
    assert call_a(t1, k2b, csr(n, k, 2 ** 31), n, k, T, cap) == -4
    # non-empty operand without index/value arrays
    bad = native.seacells_csr(0x1000, None, None, n, k, 5)
    assert call_a(t1, bad, ap, n, k, T, cap) == -1


def test_a_columns_workspace_sizes():
    # one cell per wave (always for the pruning variant, which the size also
    # covers): the padded copy of t1, at most 8 (nnz + 64 k) bytes
    for k, nnz in ((1000, 80_000), (1300, 108_000)):
        pad = saa.seacells_fw_a_columns_workspace(1000, k, 50, 60, nnz)
        assert 8 * (nnz + k) <= pad <= 8 * (nnz + 64 * k) + 4 * (k + 1) + 1024
    # support state (large k): counters, the queues of cells, and the copy
    sup = saa.seacells_fw_a_columns_workspace(1000, 10000, 50, 66, 10)
    assert sup >= 256 + 2 * 1000 * 4 + 8 * 10000 and sup % 256 == 0
    # k too large for either state in LDS: dense state slices in the workspace
    big = saa.seacells_fw_a_columns_workspace(1000, 60000, 50, 66, 10)
    assert big >= 1000 * 60000 * 4 and big % 256 == 0
    # a call without the workspace is refused on the host
    n, k, T, cap = 1000, 60000, 50, 66
    assert call_a(csr(k, k, 3), csr(n, k, 5), csr(n, k, 5), n, k, T, cap) == -3
    assert call_a(csr(1300, 1300, 3), csr(n, 1300, 5), csr(n, 1300, 5), n, 1300, T, cap) == -3
    # k from 2^30 on is refused
    k = 2 ** 30
    assert call_a(csr(k, k, 3), csr(n, k, 5), csr(n, k, 5), n, k, T, cap) == -4


def test_b_argmin_rejects_bad_arguments_on_host():
    lib = saa.load()
    n, k = 100, 30
    k2b, aat, k2at, b = csr(n, k, 5), csr(k, k, 5), csr(n, k, 5), csr(n, k, 5)
    ws = saa.seacells_fw_b_argmin_workspace(n, k, 5)
    assert ws > 0 and ws % 256 == 0

    def call(k2b=k2b, aat=aat, k2at=k2at, b=b, n=n, k=k, ws_ptr=0x100000, ws_bytes=ws,
             out=0x4000, status=0x9000, fw_gap=None):
        r = lambda m: ctypes.byref(m) if m is not None else None
        return lib.seacells_fw_b_argmin(r(k2b), r(aat), r(k2at), r(b), n, k, out, out, None,
                                        fw_gap, ws_ptr, ws_bytes, status, None)
    assert call(k2b=None) == -1
    assert call(b=None, fw_gap=0x5000) == -1   # the full gap needs B
    assert call(out=None) == -1
    assert call(status=None) == -1
    assert call(n=0) == -2
    assert call(aat=csr(k, k + 1, 5)) == -2
    assert call(b=csr(n + 1, k, 5)) == -2
    assert call(ws_bytes=ws - 1) == -3
    assert call(ws_ptr=None) == -3
    assert call(ws_ptr=0x100010) == -3        # not 256-byte aligned
    assert call(k2at=csr(n, k, 2 ** 31)) == -4


def test_b_workspace_grows_with_slices():
    one = saa.seacells_fw_b_argmin_workspace(100_000, 1300, 143_000)
    many = saa.seacells_fw_b_argmin_workspace(100_000, 10_000, 6_500_000)
    assert one > 0 and many > one
    # one slice: the padded copy of A A^T, at least 8 bytes per entry
    assert one - saa.seacells_fw_b_argmin_workspace(100_000, 1300, 0) >= 8 * 143_000


def test_b_apply_rejects_bad_arguments_on_host():
    lib = saa.load()
    p = 0x4000
    assert lib.seacells_fw_b_apply(None, p, p, 10, 4, 3, p, 0.5, p, None) == -1
    assert lib.seacells_fw_b_apply(p, p, p, 10, 0, 3, p, 0.5, p, None) == -2
    assert lib.seacells_fw_b_apply(p, p, p, 10, 4, 0, p, 0.5, p, None) == -2
    assert lib.seacells_fw_b_apply(p, p, p, 10, 4, 3, p, 0.0, p, None) == -2
    assert lib.seacells_fw_b_apply(p, p, p, 10, 4, 3, p, 1.5, p, None) == -2


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(saa.SeacellsError):
        saa.DeviceCSR(torch.zeros(3, dtype=torch.int32), torch.zeros(0, dtype=torch.int32),
                      torch.zeros(0), (2, 2))


def test_a_columns_pruned_rejects_bad_threshold_on_host():
    lib = saa.load()
    n, k, T, cap = 10, 4, 5, 8
    t1, k2b, ap = csr(k, k, 3), csr(n, k, 5), csr(n, k, 5)
    o = 0x4000

    def call(thr, t1=t1):
        return lib.seacells_fw_a_columns_pruned(ctypes.byref(t1), ctypes.byref(k2b),
                                                ctypes.byref(ap), n, k, T, cap, None, thr, o, o,
                                                o, None, None, None, 0, 0x9000, None)
    assert call(-0.1) == -2
    assert call(float("nan")) == -2
    assert call(float("inf")) == -2
    assert call(0.5, t1=csr(k + 1, k, 3)) == -2


# --- sparse operations (include/seacells_sparse.h) ---------------------------

def test_sparse_ops_reject_bad_arguments_on_host():
    lib = saa.load()
    P = ctypes.byref
    a, b = csr(5, 7, 3), csr(7, 4, 2)
    st, out = 0x9000, 0x4000
    # product: nulls, inner-dimension mismatch, too many entries
    mneed = lib.seacells_csr_matmul_workspace(5)
    assert mneed > 0 and mneed % 256 == 0
    ws = 0x10000
    assert lib.seacells_csr_matmul_rows(None, P(b), out, ws, mneed, st, None) == -1
    assert lib.seacells_csr_matmul_rows(P(a), P(b), None, ws, mneed, st, None) == -1
    assert lib.seacells_csr_matmul_rows(P(a), P(b), out, ws, mneed, None, None) == -1
    assert lib.seacells_csr_matmul_rows(P(a), P(csr(6, 4, 2)), out, ws, mneed, st, None) == -2
    assert lib.seacells_csr_matmul_rows(P(a), P(b), out, None, mneed, st, None) == -3
    assert lib.seacells_csr_matmul_rows(P(a), P(b), out, ws, mneed - 1, st, None) == -3
    assert lib.seacells_csr_matmul_rows(P(a), P(b), out, ws + 4, mneed, st, None) == -3
    assert lib.seacells_csr_matmul_fill(P(a), P(csr(6, 4, 2)), out, out, out, 8, None, 0, st,
                                        None) == -2
    assert lib.seacells_csr_matmul_fill(P(a), P(b), None, out, out, 8, None, 0, st, None) == -1
    # the kept row bitmaps: m * ceil(q / 32) words after the scan partials, none past 16384 columns
    assert lib.seacells_csr_matmul_pattern_workspace(5, 100) >= mneed + 5 * 4 * 4
    assert lib.seacells_csr_matmul_pattern_workspace(5, 16384) > 0
    assert lib.seacells_csr_matmul_pattern_workspace(5, 16385) == 0
    assert lib.seacells_csr_matmul_rows(P(csr(5, 7, 2 ** 31)), P(b), out, ws, mneed, st,
                                        None) == -4
    assert lib.seacells_csr_matmul_rows(P(csr(5, 7, 3, ptr=None)), P(b), out, ws, mneed, st,
                                        None) == -1
    # transpose: nulls and workspace
    need = lib.seacells_csr_transpose_workspace(5, 7)
    assert need >= 7 * 4 and need % 256 == 0
    assert lib.seacells_csr_transpose(P(a), None, out, out, 0x10000, need, st, None) == -1
    assert lib.seacells_csr_transpose(P(a), out, None, out, 0x10000, need, st, None) == -1
    assert lib.seacells_csr_transpose(P(a), out, out, out, 0x10000, need - 1, st, None) == -3
    assert lib.seacells_csr_transpose(P(a), out, out, out, 0x10004, need, st, None) == -3
    assert lib.seacells_csr_transpose(P(a), out, out, out, None, need, st, None) == -3
    # inner product: shapes, nulls, workspace
    dneed = lib.seacells_csr_dot_workspace()
    assert dneed > 0 and dneed % 256 == 0
    x = csr(5, 7, 3)
    assert lib.seacells_csr_dot(P(x), P(csr(5, 6, 3)), ctypes.c_double(1.0), out, 0x10000, dneed,
                                st, None) == -2
    assert lib.seacells_csr_dot(P(x), P(x), ctypes.c_double(1.0), None, 0x10000, dneed, st,
                                None) == -1
    assert lib.seacells_csr_dot(P(x), P(x), ctypes.c_double(1.0), out, 0x10000, dneed - 8, st,
                                None) == -3


def test_sparse_add_and_vertex_reject_bad_arguments_on_host():
    lib = saa.load()
    P = ctypes.byref
    st, out, ws = 0x9000, 0x4000, 0x10000
    x, y = csr(5, 7, 3), csr(5, 7, 4)
    need = lib.seacells_csr_add_workspace(5)
    assert need > 0 and need % 256 == 0
    assert lib.seacells_csr_add_rows(None, P(y), out, ws, need, st, None) == -1
    assert lib.seacells_csr_add_rows(P(x), P(y), None, ws, need, st, None) == -1
    assert lib.seacells_csr_add_rows(P(x), P(csr(5, 6, 4)), out, ws, need, st, None) == -2
    assert lib.seacells_csr_add_rows(P(x), P(csr(4, 7, 4)), out, ws, need, st, None) == -2
    assert lib.seacells_csr_add_rows(P(x), P(y), out, ws, need - 1, st, None) == -3
    assert lib.seacells_csr_add_rows(P(x), P(y), out, ws + 8, need, st, None) == -3
    assert lib.seacells_csr_add_rows(P(csr(5, 7, 2 ** 30)), P(csr(5, 7, 2 ** 30)), out, ws, need,
                                     st, None) == -4
    f = ctypes.c_float
    assert lib.seacells_csr_add_fill(f(1), P(x), f(1), P(y), None, out, out, 8, st, None) == -1
    assert lib.seacells_csr_add_fill(f(1), P(x), f(1), P(y), out, None, out, 8, st, None) == -1
    assert lib.seacells_csr_add_fill(f(1), P(x), f(1), P(csr(5, 8, 1)), out, out, out, 8, st,
                                     None) == -2
    vneed = lib.seacells_fw_b_vertex_workspace(10, 100)
    assert vneed > 0 and vneed % 256 == 0
    assert lib.seacells_fw_b_vertex(None, 10, 100, f(1), out, out, out, ws, vneed, st, None) == -1
    assert lib.seacells_fw_b_vertex(out, 10, 100, f(1), None, out, out, ws, vneed, st, None) == -1
    assert lib.seacells_fw_b_vertex(out, 10, 0, f(1), out, out, out, ws, vneed, st, None) == -2
    assert lib.seacells_fw_b_vertex(out, 10, 100, f(1), out, out, out, ws, vneed - 1, st,
                                    None) == -3
    assert lib.seacells_fw_b_vertex(out, 2 ** 31, 100, f(1), out, out, out, ws, vneed, st,
                                    None) == -4


def test_atoms_to_csr_rejects_bad_arguments_on_host():
    lib = saa.load()
    st, out, ws = 0x9000, 0x4000, 0x10000
    need = lib.seacells_fw_a_to_csr_workspace(10)
    assert need > 0 and need % 256 == 0
    assert lib.seacells_fw_a_to_csr_rows(None, out, out, 10, 5, 4, out, ws, need, st, None) == -1
    assert lib.seacells_fw_a_to_csr_rows(out, out, out, 10, 0, 4, out, ws, need, st, None) == -2
    assert lib.seacells_fw_a_to_csr_rows(out, out, out, 10, 5, 0, out, ws, need, st, None) == -2
    assert lib.seacells_fw_a_to_csr_rows(out, out, out, 10, 5, 4, None, ws, need, st, None) == -1
    assert lib.seacells_fw_a_to_csr_rows(out, out, out, 10, 5, 4, out, ws, need - 1, st,
                                         None) == -3
    assert lib.seacells_fw_a_to_csr_fill(out, out, out, 10, 5, 4, None, out, out, st, None) == -1
    assert lib.seacells_fw_a_to_csr_fill(out, out, out, 2 ** 31, 5, 4, out, out, out, st,
                                         None) == -4


@pytest.mark.parametrize("k", [2048, 2049, 262_144, 262_145, 300_000, 1 << 24, (1 << 31) - 1])
def test_b_argmin_has_a_plan_for_every_k(k):
    # no ceiling on k: slices of at most 2048 columns cover every column, and
    # the partial keys stay within 2 GiB by taking fewer row ranges (one at least)
    n = 1_000_000
    lay = saa.seacells_debug_b_layout(n, k, 8 * k)
    assert 1 <= lay["slice_w"] <= 2048
    assert lay["n_slices"] * lay["slice_w"] >= k > (lay["n_slices"] - 1) * lay["slice_w"]
    assert lay["n_row_blocks"] >= 1
    assert lay["n_row_blocks"] == 1 or lay["n_row_blocks"] * k * 8 <= 1 << 31
    ws = saa.seacells_fw_b_argmin_workspace(n, k, 8 * k)
    assert ws >= lay["keys_offset"] + lay["n_row_blocks"] * k * 8
    assert ws >= lay["stamps_offset"] + lay["n_row_blocks"] * lay["n_slices"] * 4


def test_debug_hooks_reject_bad_options():
    lib = saa.load()
    bad = native.seacells_a_options(2, 0, 0, 0, -1)
    assert lib.seacells_debug_set_a_options(ctypes.byref(bad)) == -2
    bad = native.seacells_a_options(-1, 3, 0, 0, -1)
    assert lib.seacells_debug_set_a_options(ctypes.byref(bad)) == -2
    bad = native.seacells_a_options(-1, 0, 0, 48, -1)
    assert lib.seacells_debug_set_a_options(ctypes.byref(bad)) == -2
    assert lib.seacells_debug_set_a_options(None) == 0
    # the overrides reach the workspace query (the support state's queues)
    base = saa.seacells_fw_a_columns_workspace(1000, 6700, 50, 62, 10)
    saa.seacells_debug_set_a_options(support=0)
    try:
        assert saa.seacells_fw_a_columns_workspace(1000, 6700, 50, 62, 10) < base
    finally:
        saa.seacells_debug_set_a_options()
    assert saa.seacells_fw_a_columns_workspace(1000, 6700, 50, 62, 10) == base
    assert lib.seacells_debug_b_layout(0, 5, 0, ctypes.byref(native.seacells_b_layout())) == -2
    assert lib.seacells_debug_b_reduce(10, 5, 0, 1, None, None, None, None, 0, None, None) == -1


def test_default_step_size_in_f32():
    import numpy as np
    # gamma_t = 2 / (t + 2) and 1 - gamma_t, each rounded once to f32
    for t in (0, 1, 2, 3, 7, 48, 49, 1000, 2**31):
        g, keep = saa.seacells_fw_step_size(t)
        want = np.float32(2.0) / np.float32(t + 2)
        assert np.float32(g) == want
        assert np.float32(keep) == np.float32(1.0) - want
    assert saa.seacells_fw_step_size(0) == (1.0, 0.0)
