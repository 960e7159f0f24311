"""Thin ctypes binding of ``libseacells_fw.so`` (include/seacells_fw.h,
include/seacells_sparse.h, include/seacells_debug.h).

The functions carry the C names and only marshal arguments: device tensors
become raw pointers, torch's current stream becomes the hipStream_t. Every
step of the computation runs in the library's HIP kernels; there is no CPU
fallback, and a missing library is an error.

PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import _build

SEACELLS_OK = 0
ERRORS = {-1: "E_NULL", -2: "E_SHAPE", -3: "E_WORKSPACE", -4: "E_TOO_LARGE", -5: "E_HIP"}
FLAGS = {0x1: "CAP_OVERFLOW", 0x2: "PARTIALS_INVALID", 0x4: "B_CAP_OVERFLOW", 0x8: "BAD_INDEX",
         0x10: "NONFINITE", 0x20: "BAD_GAMMA", 0x40: "OUTPUT_TOO_LARGE"}

EXPORTS = ("seacells_fw_a_columns_workspace", "seacells_fw_a_columns",
           "seacells_fw_a_columns_pruned", "seacells_fw_a_columns_noalloc",
           "seacells_fw_b_argmin_workspace", "seacells_fw_b_argmin", "seacells_fw_b_apply",
           "seacells_csr_matmul_workspace", "seacells_csr_matmul_pattern_workspace",
           "seacells_csr_matmul_rows", "seacells_csr_matmul_fill",
           "seacells_csr_transpose_workspace", "seacells_csr_transpose",
           "seacells_csr_dot_workspace", "seacells_csr_dot",
           "seacells_csr_add_workspace", "seacells_csr_add_rows", "seacells_csr_add_fill",
           "seacells_fw_b_vertex_workspace", "seacells_fw_b_vertex",
           "seacells_fw_a_to_csr_workspace", "seacells_fw_a_to_csr_rows",
           "seacells_fw_a_to_csr_fill",
           "seacells_debug_set_a_options", "seacells_debug_b_layout",
           "seacells_debug_b_last_epoch", "seacells_debug_b_reduce",
           "seacells_fw_step_size",
           "seacells_status_string", "seacells_last_error", "seacells_version")


class seacells_csr(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("val", ctypes.c_void_p), ("n_rows", ctypes.c_uint32),
                ("n_cols", ctypes.c_uint32), ("nnz", ctypes.c_uint32)]


class seacells_a_options(ctypes.Structure):
    _fields_ = [("support", ctypes.c_int32), ("support_waves", ctypes.c_uint32),
                ("dense_argmin", ctypes.c_int32), ("group", ctypes.c_uint32),
                ("support_wide", ctypes.c_int32)]


class seacells_b_layout(ctypes.Structure):
    _fields_ = [("keys_offset", ctypes.c_uint64), ("stamps_offset", ctypes.c_uint64),
                ("n_row_blocks", ctypes.c_uint32), ("n_slices", ctypes.c_uint32),
                ("slice_w", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_CSR_P = ctypes.POINTER(seacells_csr)
_VP = ctypes.c_void_p
_U32 = ctypes.c_uint32
_lib = None


class SeacellsError(RuntimeError):
    pass


def library_path() -> str:
    return _build.LIB


def load():
    """The loaded library. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path):
        raise SeacellsError("libseacells_fw.so is not built; run __graft_entry__.build() "
                            "(or python -m sparse_archetypal_analysis_amd._build)")
    lib = ctypes.CDLL(path)
    lib.seacells_fw_a_columns_workspace.restype = ctypes.c_size_t
    lib.seacells_fw_a_columns_workspace.argtypes = [_U32, _U32, _U32, _U32, _U32]
    lib.seacells_fw_a_columns.restype = ctypes.c_int
    lib.seacells_fw_a_columns.argtypes = [_CSR_P, _CSR_P, _CSR_P, _U32, _U32, _U32, _U32, _VP, _VP,
                                          _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_fw_a_columns_pruned.restype = ctypes.c_int
    lib.seacells_fw_a_columns_pruned.argtypes = [_CSR_P, _CSR_P, _CSR_P, _U32, _U32, _U32, _U32,
                                                 _VP, ctypes.c_float, _VP, _VP, _VP, _VP, _VP,
                                                 _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_fw_a_columns_noalloc.restype = ctypes.c_int
    lib.seacells_fw_a_columns_noalloc.argtypes = [_CSR_P, _CSR_P, _CSR_P, _U32, _U32, _U32, _U32,
                                                  _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.seacells_fw_b_argmin_workspace.restype = ctypes.c_size_t
    lib.seacells_fw_b_argmin_workspace.argtypes = [_U32, _U32, _U32]
    lib.seacells_fw_b_argmin.restype = ctypes.c_int
    lib.seacells_fw_b_argmin.argtypes = [_CSR_P, _CSR_P, _CSR_P, _CSR_P, _U32, _U32, _VP, _VP, _VP,
                                         _VP, _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_fw_b_apply.restype = ctypes.c_int
    lib.seacells_fw_b_apply.argtypes = [_VP, _VP, _VP, _U32, _U32, _U32, _VP, ctypes.c_float,
                                        _VP, _VP]
    lib.seacells_csr_matmul_workspace.restype = ctypes.c_size_t
    lib.seacells_csr_matmul_workspace.argtypes = [_U32]
    lib.seacells_csr_matmul_rows.restype = ctypes.c_int
    lib.seacells_csr_matmul_rows.argtypes = [_CSR_P, _CSR_P, _VP, _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_csr_matmul_fill.restype = ctypes.c_int
    lib.seacells_csr_matmul_fill.argtypes = [_CSR_P, _CSR_P, _VP, _VP, _VP, ctypes.c_size_t, _VP,
                                             ctypes.c_size_t, _VP, _VP]
    lib.seacells_csr_matmul_pattern_workspace.restype = ctypes.c_size_t
    lib.seacells_csr_matmul_pattern_workspace.argtypes = [_U32, _U32]
    lib.seacells_csr_transpose_workspace.restype = ctypes.c_size_t
    lib.seacells_csr_transpose_workspace.argtypes = [_U32, _U32]
    lib.seacells_csr_transpose.restype = ctypes.c_int
    lib.seacells_csr_transpose.argtypes = [_CSR_P, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_csr_dot_workspace.restype = ctypes.c_size_t
    lib.seacells_csr_dot_workspace.argtypes = []
    lib.seacells_csr_dot.restype = ctypes.c_int
    lib.seacells_csr_dot.argtypes = [_CSR_P, _CSR_P, ctypes.c_double, _VP, _VP, ctypes.c_size_t,
                                     _VP, _VP]
    lib.seacells_csr_add_workspace.restype = ctypes.c_size_t
    lib.seacells_csr_add_workspace.argtypes = [_U32]
    lib.seacells_csr_add_rows.restype = ctypes.c_int
    lib.seacells_csr_add_rows.argtypes = [_CSR_P, _CSR_P, _VP, _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_csr_add_fill.restype = ctypes.c_int
    lib.seacells_csr_add_fill.argtypes = [ctypes.c_float, _CSR_P, ctypes.c_float, _CSR_P, _VP, _VP,
                                          _VP, ctypes.c_size_t, _VP, _VP]
    lib.seacells_fw_b_vertex_workspace.restype = ctypes.c_size_t
    lib.seacells_fw_b_vertex_workspace.argtypes = [_U32, _U32]
    lib.seacells_fw_b_vertex.restype = ctypes.c_int
    lib.seacells_fw_b_vertex.argtypes = [_VP, _U32, _U32, ctypes.c_float, _VP, _VP, _VP, _VP,
                                         ctypes.c_size_t, _VP, _VP]
    lib.seacells_fw_a_to_csr_workspace.restype = ctypes.c_size_t
    lib.seacells_fw_a_to_csr_workspace.argtypes = [_U32]
    lib.seacells_fw_a_to_csr_rows.restype = ctypes.c_int
    lib.seacells_fw_a_to_csr_rows.argtypes = [_VP, _VP, _VP, _U32, _U32, _U32, _VP, _VP,
                                              ctypes.c_size_t, _VP, _VP]
    lib.seacells_fw_a_to_csr_fill.restype = ctypes.c_int
    lib.seacells_fw_a_to_csr_fill.argtypes = [_VP, _VP, _VP, _U32, _U32, _U32, _VP, _VP, _VP,
                                              _VP, _VP]
    lib.seacells_debug_set_a_options.restype = ctypes.c_int
    lib.seacells_debug_set_a_options.argtypes = [ctypes.POINTER(seacells_a_options)]
    lib.seacells_debug_b_layout.restype = ctypes.c_int
    lib.seacells_debug_b_layout.argtypes = [_U32, _U32, _U32, ctypes.POINTER(seacells_b_layout)]
    lib.seacells_debug_b_last_epoch.restype = ctypes.c_uint32
    lib.seacells_debug_b_last_epoch.argtypes = []
    lib.seacells_debug_b_reduce.restype = ctypes.c_int
    lib.seacells_debug_b_reduce.argtypes = [_U32, _U32, _U32, _U32, _VP, _VP, _VP, _VP,
                                            ctypes.c_size_t, _VP, _VP]
    lib.seacells_status_string.restype = ctypes.c_char_p
    lib.seacells_status_string.argtypes = [ctypes.c_int]
    lib.seacells_last_error.restype = ctypes.c_char_p
    lib.seacells_last_error.argtypes = []
    lib.seacells_version.restype = ctypes.c_int
    lib.seacells_version.argtypes = []
    lib.seacells_fw_step_size.restype = ctypes.c_int
    lib.seacells_fw_step_size.argtypes = [ctypes.c_uint32, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_float)]
    _lib = lib
    return lib


def _check_rc(rc: int):
    if rc != SEACELLS_OK:
        lib = load()
        msg = lib.seacells_status_string(rc).decode()
        if rc == -5:
            msg += ": " + lib.seacells_last_error().decode()
        raise SeacellsError("%s (%d): %s" % (ERRORS.get(rc, "?"), rc, msg))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class DeviceCSR:
    """A CSR operand held in device memory as int32 / float32 tensors.

    The C side reads the int32 index tensors as u32; values must stay below
    2^31 (checked when built from the host).
    """

    def __init__(self, row_ptr: torch.Tensor, col_idx: torch.Tensor, val: torch.Tensor, shape):
        for t, dt in ((row_ptr, torch.int32), (col_idx, torch.int32), (val, torch.float32)):
            if t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise SeacellsError("CSR arrays must be contiguous cuda int32/int32/float32")
        if row_ptr.numel() != shape[0] + 1 or col_idx.numel() != val.numel():
            raise SeacellsError("CSR array lengths do not match the shape")
        self.row_ptr, self.col_idx, self.val = row_ptr, col_idx, val
        self.shape = (int(shape[0]), int(shape[1]))
        self.nnz = int(val.numel())

    @classmethod
    def from_scipy(cls, m, device="cuda"):
        ptr = np.asarray(m.indptr)
        if ptr[-1] >= 2 ** 31:
            raise SeacellsError("operand has 2^31 or more non-zeros")
        return cls(torch.from_numpy(ptr.astype(np.int32)).to(device),
                   torch.from_numpy(np.asarray(m.indices).astype(np.int32)).to(device),
                   torch.from_numpy(np.asarray(m.data).astype(np.float32)).to(device),
                   m.shape)

    def struct(self) -> seacells_csr:
        return seacells_csr(self.row_ptr.data_ptr(),
                            self.col_idx.data_ptr() if self.nnz else None,
                            self.val.data_ptr() if self.nnz else None,
                            self.shape[0], self.shape[1], self.nnz)


def new_status(device="cuda") -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


def status_flags(status: torch.Tensor) -> list:
    """Names of the flags set in a status word (synchronises)."""
    v = int(status.item()) & 0xffffffff
    return [nm for bit, nm in FLAGS.items() if v & bit]


def raise_on_status(status: torch.Tensor):
    names = status_flags(status)
    if names:
        raise SeacellsError("device status: " + ", ".join(names))


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def seacells_fw_a_columns_workspace(n, k, T, cap, t1_nnz) -> int:
    return int(load().seacells_fw_a_columns_workspace(n, k, T, cap, t1_nnz))


def seacells_fw_a_columns(t1: DeviceCSR, k2b: DeviceCSR, a_prev_t: DeviceCSR, n: int, k: int,
                          T: int, cap: int, gamma=None, atom_idx=None, atom_val=None,
                          atom_cnt=None, trace=None, workspace=None, status=None, stream=None,
                          fw_gap=None):
    """A update. Returns (atom_idx [n, cap], atom_val [n, cap], atom_cnt [n], trace, status).

    Outputs and workspace are allocated when not given; pass ``trace=True``
    to get the per-step argmin trace [n, T]. ``fw_gap`` (a float32 [n]
    device tensor, filled in place) receives the Frank-Wolfe gap of each
    returned column.
    """
    return _a_columns(None, t1, k2b, a_prev_t, n, k, T, cap, gamma, atom_idx, atom_val,
                      atom_cnt, trace, fw_gap, workspace, status, stream)


def seacells_fw_a_columns_pruned(t1: DeviceCSR, k2b: DeviceCSR, a_prev_t: DeviceCSR, n: int,
                                 k: int, T: int, cap: int, threshold: float, gamma=None,
                                 atom_idx=None, atom_val=None, atom_cnt=None, trace=None,
                                 workspace=None, status=None, stream=None, fw_gap=None):
    """A update with the pruning + renormalisation step; as seacells_fw_a_columns."""
    return _a_columns(float(threshold), t1, k2b, a_prev_t, n, k, T, cap, gamma, atom_idx,
                      atom_val, atom_cnt, trace, fw_gap, workspace, status, stream)


def _a_columns(threshold, t1, k2b, a_prev_t, n, k, T, cap, gamma, atom_idx, atom_val, atom_cnt,
               trace, fw_gap, workspace, status, stream):
    lib = load()
    dev = t1.row_ptr.device
    if atom_idx is None:
        atom_idx = torch.empty((n, cap), dtype=torch.int32, device=dev)
    if atom_val is None:
        atom_val = torch.empty((n, cap), dtype=torch.float32, device=dev)
    if atom_cnt is None:
        atom_cnt = torch.empty(n, dtype=torch.int32, device=dev)
    if trace is True:
        trace = torch.empty((n, T), dtype=torch.int32, device=dev)
    elif trace is False:
        trace = None
    if status is None:
        status = new_status(dev)
    ws_bytes = seacells_fw_a_columns_workspace(n, k, T, cap, t1.nnz)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s1, s2, s3 = t1.struct(), k2b.struct(), a_prev_t.struct()
    if fw_gap is not None and (fw_gap.dtype != torch.float32 or fw_gap.numel() < n):
        raise SeacellsError("fw_gap must be a float32 tensor of at least n entries")
    tail = (_ptr(atom_idx), _ptr(atom_val), _ptr(atom_cnt), _ptr(trace), _ptr(fw_gap),
            _ptr(workspace), 0 if workspace is None else workspace.numel(), _ptr(status),
            _stream(stream))
    if threshold is None:
        rc = lib.seacells_fw_a_columns(ctypes.byref(s1), ctypes.byref(s2), ctypes.byref(s3), n,
                                       k, T, cap, _ptr(gamma), *tail)
    else:
        rc = lib.seacells_fw_a_columns_pruned(ctypes.byref(s1), ctypes.byref(s2),
                                              ctypes.byref(s3), n, k, T, cap, _ptr(gamma),
                                              threshold, *tail)
    _check_rc(rc)
    return atom_idx, atom_val, atom_cnt, trace, status


NOALLOC_SCRATCH_BYTES = 128 << 20  # SEACELLS_NOALLOC_SCRATCH_BYTES


def seacells_fw_a_columns_noalloc(t1: DeviceCSR, k2b: DeviceCSR, a_prev_t: DeviceCSR, n: int,
                                  k: int, T: int, cap: int, gamma=None, atom_idx=None,
                                  atom_val=None, atom_cnt=None, trace=None, status=None,
                                  stream=None, fw_gap=None):
    """The A update with the library's static scratch as its workspace (the C
    entry point allocates nothing; outputs given here are used as they are).
    Returns (atom_idx, atom_val, atom_cnt, trace, status)."""
    lib = load()
    dev = t1.row_ptr.device
    if atom_idx is None:
        atom_idx = torch.empty((n, cap), dtype=torch.int32, device=dev)
    if atom_val is None:
        atom_val = torch.empty((n, cap), dtype=torch.float32, device=dev)
    if atom_cnt is None:
        atom_cnt = torch.empty(n, dtype=torch.int32, device=dev)
    if trace is True:
        trace = torch.empty((n, T), dtype=torch.int32, device=dev)
    elif trace is False:
        trace = None
    if status is None:
        status = new_status(dev)
    s1, s2, s3 = t1.struct(), k2b.struct(), a_prev_t.struct()
    rc = lib.seacells_fw_a_columns_noalloc(ctypes.byref(s1), ctypes.byref(s2), ctypes.byref(s3),
                                           n, k, T, cap, _ptr(gamma), _ptr(atom_idx),
                                           _ptr(atom_val), _ptr(atom_cnt), _ptr(trace),
                                           _ptr(fw_gap), _ptr(status), _stream(stream))
    _check_rc(rc)
    return atom_idx, atom_val, atom_cnt, trace, status


def seacells_fw_b_argmin_workspace(n, k, aat_nnz) -> int:
    return int(load().seacells_fw_b_argmin_workspace(n, k, aat_nnz))


def seacells_fw_b_argmin(k2b: DeviceCSR, aat: DeviceCSR, k2at: DeviceCSR, b, n: int, k: int,
                         out_val=None, out_idx=None, gap=None, workspace=None, status=None,
                         stream=None, fw_gap=None):
    """B-gradient argmin. Returns (out_val [k], out_idx [k], gap [1], status).

    ``fw_gap`` (a float32 [1] device tensor, filled in place) receives the
    full Frank-Wolfe gap sum(B * G) - sum_c min_i G[i, c]; it needs ``b``.
    """
    lib = load()
    dev = k2b.row_ptr.device
    if out_val is None:
        out_val = torch.empty(k, dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int32, device=dev)
    if gap is None:
        gap = torch.empty(1, dtype=torch.float32, device=dev)
    if status is None:
        status = new_status(dev)
    ws_bytes = seacells_fw_b_argmin_workspace(n, k, aat.nnz)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    s1, s2, s3 = k2b.struct(), aat.struct(), k2at.struct()
    sb = b.struct() if b is not None else None
    rc = lib.seacells_fw_b_argmin(ctypes.byref(s1), ctypes.byref(s2), ctypes.byref(s3),
                                  ctypes.byref(sb) if sb is not None else None, n, k,
                                  _ptr(out_val), _ptr(out_idx), _ptr(gap), _ptr(fw_gap),
                                  _ptr(workspace), workspace.numel(), _ptr(status),
                                  _stream(stream))
    _check_rc(rc)
    return out_val, out_idx, gap, status


def seacells_fw_b_apply(bt_idx, bt_val, bt_cnt, n: int, arg_idx, gamma: float, status=None,
                        stream=None):
    """B step in place on padded B^T rows ([k, cap_b] int32 / float32, [k] int32)."""
    lib = load()
    k, cap_b = bt_idx.shape
    if status is None:
        status = new_status(bt_idx.device)
    rc = lib.seacells_fw_b_apply(_ptr(bt_idx), _ptr(bt_val), _ptr(bt_cnt), n, k, cap_b,
                                 _ptr(arg_idx), float(gamma), _ptr(status), _stream(stream))
    _check_rc(rc)
    return bt_idx, bt_val, bt_cnt, status


# --------------------------------------------------------------------------
# test and experiment hooks (include/seacells_debug.h)
# --------------------------------------------------------------------------

def seacells_debug_set_a_options(support=-1, support_waves=0, dense_argmin=False, group=0,
                                 support_wide=-1):
    """Plan overrides of the A update (process-wide); no arguments restore
    the defaults."""
    opt = seacells_a_options(int(support), int(support_waves), 1 if dense_argmin else 0,
                             int(group), int(support_wide))
    _check_rc(load().seacells_debug_set_a_options(ctypes.byref(opt)))


def seacells_debug_b_layout(n: int, k: int, aat_nnz: int) -> dict:
    """Where seacells_fw_b_argmin keeps its partial keys and stamps."""
    out = seacells_b_layout()
    _check_rc(load().seacells_debug_b_layout(n, k, aat_nnz, ctypes.byref(out)))
    return {nm: int(getattr(out, nm)) for nm, _ in seacells_b_layout._fields_ if nm != "reserved"}


def seacells_debug_b_last_epoch() -> int:
    return int(load().seacells_debug_b_last_epoch())


def seacells_debug_b_reduce(n: int, k: int, aat_nnz: int, epoch: int, workspace, out_val=None,
                            out_idx=None, gap=None, status=None, stream=None):
    """The B argmin's reduce stages alone over the partials in ``workspace``.
    Returns (out_val, out_idx, gap, status)."""
    dev = workspace.device
    if out_val is None:
        out_val = torch.empty(k, dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int32, device=dev)
    if gap is None:
        gap = torch.empty(1, dtype=torch.float32, device=dev)
    if status is None:
        status = new_status(dev)
    rc = load().seacells_debug_b_reduce(n, k, aat_nnz, int(epoch) & 0xffffffff, _ptr(out_val),
                                        _ptr(out_idx), _ptr(gap), _ptr(workspace),
                                        workspace.numel(), _ptr(status), _stream(stream))
    _check_rc(rc)
    return out_val, out_idx, gap, status


# --------------------------------------------------------------------------
# sparse operations (include/seacells_sparse.h)
# --------------------------------------------------------------------------

def seacells_csr_matmul_workspace(m: int) -> int:
    return int(load().seacells_csr_matmul_workspace(m))


def seacells_csr_matmul_rows(a: DeviceCSR, b: DeviceCSR, c_row_ptr=None, workspace=None,
                             status=None, stream=None):
    """Row pointer of a @ b ([m + 1] int32, last entry = nnz). Returns (c_row_ptr, status)."""
    lib = load()
    dev = a.row_ptr.device
    if c_row_ptr is None:
        c_row_ptr = torch.empty(a.shape[0] + 1, dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty(seacells_csr_matmul_workspace(a.shape[0]), dtype=torch.uint8,
                                device=dev)
    sa, sb = a.struct(), b.struct()
    rc = lib.seacells_csr_matmul_rows(ctypes.byref(sa), ctypes.byref(sb), _ptr(c_row_ptr),
                                      _ptr(workspace), workspace.numel(), _ptr(status),
                                      _stream(stream))
    _check_rc(rc)
    return c_row_ptr, status


def seacells_csr_matmul_pattern_workspace(m: int, q: int) -> int:
    return int(load().seacells_csr_matmul_pattern_workspace(m, q))


def seacells_csr_matmul_fill(a: DeviceCSR, b: DeviceCSR, c_row_ptr, c_col_idx, c_val,
                             workspace=None, status=None, stream=None):
    """Columns and values of a @ b into buffers sized by c_row_ptr[-1]
    (``workspace``: the rows pass's, to reuse the row bitmaps it kept)."""
    lib = load()
    if status is None:
        status = new_status(a.row_ptr.device)
    sa, sb = a.struct(), b.struct()
    rc = lib.seacells_csr_matmul_fill(ctypes.byref(sa), ctypes.byref(sb), _ptr(c_row_ptr),
                                      _ptr(c_col_idx) if c_col_idx.numel() else None,
                                      _ptr(c_val) if c_val.numel() else None,
                                      min(c_col_idx.numel(), c_val.numel()), _ptr(workspace),
                                      0 if workspace is None else workspace.numel(),
                                      _ptr(status), _stream(stream))
    _check_rc(rc)
    return c_col_idx, c_val, status


PATTERN_WORKSPACE_LIMIT = 4 << 30  # bytes of row bitmaps csr_matmul keeps between its passes


def csr_matmul(a: DeviceCSR, b: DeviceCSR, status=None, stream=None, bound=None,
               out: "OutBuffers" = None) -> DeviceCSR:
    """a @ b as a DeviceCSR; the rows pass keeps its row bitmaps for the fill
    pass when they take at most PATTERN_WORKSPACE_LIMIT bytes.

    Without ``bound``: one synchronisation between the passes reads the
    output size, and a device status flag raises. With ``bound`` (an upper
    bound on the entries, e.g. the number of products): no synchronisation;
    the outputs hold ``bound`` entries, the returned matrix's nnz is that
    bound (its rows end at the true size), and a bound that is too small
    raises OUTPUT_TOO_LARGE in ``status`` with nothing written. ``out``
    (OutBuffers) reuses its arrays; a and b must not live in them."""
    dev = a.row_ptr.device
    if status is None:
        status = new_status(dev)
    m, q = a.shape[0], b.shape[1]
    ws_bytes = seacells_csr_matmul_pattern_workspace(m, q)
    if ws_bytes == 0 or ws_bytes > PATTERN_WORKSPACE_LIMIT:
        ws_bytes = seacells_csr_matmul_workspace(m)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    c_ptr = out.row_ptr(m, dev) if out is not None else None
    c_ptr, _ = seacells_csr_matmul_rows(a, b, c_row_ptr=c_ptr, workspace=ws, status=status,
                                        stream=stream)
    if bound is None:
        raise_on_status(status)  # synchronises; c_ptr[-1] is valid after it
        nnz = int(c_ptr[-1].item()) & 0xffffffff
    else:
        nnz = int(bound)
    if out is not None:
        c_idx, c_val = out.entries(nnz, dev)
    else:
        c_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
        c_val = torch.empty(nnz, dtype=torch.float32, device=dev)
    seacells_csr_matmul_fill(a, b, c_ptr, c_idx, c_val, workspace=ws, status=status,
                             stream=stream)
    return DeviceCSR(c_ptr, c_idx, c_val, (a.shape[0], b.shape[1]))


def seacells_csr_transpose_workspace(m: int, q: int) -> int:
    return int(load().seacells_csr_transpose_workspace(m, q))


def seacells_csr_transpose(a: DeviceCSR, at_row_ptr=None, at_col_idx=None, at_val=None,
                           workspace=None, status=None, stream=None):
    """Transpose of a. Returns (DeviceCSR of a^T, status)."""
    lib = load()
    dev = a.row_ptr.device
    m, q = a.shape
    if at_row_ptr is None:
        at_row_ptr = torch.empty(q + 1, dtype=torch.int32, device=dev)
    if at_col_idx is None:
        at_col_idx = torch.empty(a.nnz, dtype=torch.int32, device=dev)
    if at_val is None:
        at_val = torch.empty(a.nnz, dtype=torch.float32, device=dev)
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty(seacells_csr_transpose_workspace(m, q), dtype=torch.uint8,
                                device=dev)
    sa = a.struct()
    rc = lib.seacells_csr_transpose(ctypes.byref(sa), _ptr(at_row_ptr),
                                    _ptr(at_col_idx) if at_col_idx.numel() else None,
                                    _ptr(at_val) if at_val.numel() else None, _ptr(workspace),
                                    workspace.numel(), _ptr(status), _stream(stream))
    _check_rc(rc)
    return DeviceCSR(at_row_ptr, at_col_idx, at_val, (q, m)), status


def seacells_csr_dot_workspace() -> int:
    return int(load().seacells_csr_dot_workspace())


def seacells_csr_dot(x: DeviceCSR, y: DeviceCSR, alpha: float, acc, workspace=None, status=None,
                     stream=None):
    """acc[0] += alpha * sum(x * y) (acc: float64 [1] device tensor)."""
    lib = load()
    dev = x.row_ptr.device
    if acc.dtype != torch.float64 or acc.numel() < 1:
        raise SeacellsError("acc must be a float64 tensor")
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty(seacells_csr_dot_workspace(), dtype=torch.uint8, device=dev)
    sx, sy = x.struct(), y.struct()
    rc = lib.seacells_csr_dot(ctypes.byref(sx), ctypes.byref(sy), float(alpha), _ptr(acc),
                              _ptr(workspace), workspace.numel(), _ptr(status), _stream(stream))
    _check_rc(rc)
    return acc, status


def rss(K: DeviceCSR, k2b: DeviceCSR, a_t: DeviceCSR, t1: DeviceCSR, aat: DeviceCSR,
        acc=None, status=None, stream=None):
    """||K - K B A||_F^2 = <K, K> - 2 <K^2 B, A^T> + <B^T K^2 B, A A^T>, as a
    float64 [1] device tensor (three inner products on the device)."""
    dev = K.row_ptr.device
    if acc is None:
        acc = torch.zeros(1, dtype=torch.float64, device=dev)
    if status is None:
        status = new_status(dev)
    ws = torch.empty(seacells_csr_dot_workspace(), dtype=torch.uint8, device=dev)
    seacells_csr_dot(K, K, 1.0, acc, ws, status, stream)
    seacells_csr_dot(k2b, a_t, -2.0, acc, ws, status, stream)
    seacells_csr_dot(t1, aat, 1.0, acc, ws, status, stream)
    return acc, status


def device_operands(K: DeviceCSR, B: DeviceCSR, At: DeviceCSR, status=None, stream=None) -> dict:
    """Every Frank-Wolfe operand from K (n x n), B (n x k) and A^T (n x k),
    built by the library's kernels:
      kb = K B, k2b = K kb, bt = B^T, t1 = bt k2b, a = (A^T)^T, aat = a A^T,
      kat = K A^T, k2at = K kat.
    One synchronisation per product sizes its output. Raises on a device
    status flag."""
    if status is None:
        status = new_status(K.row_ptr.device)
    out = {}
    out["kb"] = csr_matmul(K, B, status, stream)
    out["k2b"] = csr_matmul(K, out["kb"], status, stream)
    out["bt"], _ = seacells_csr_transpose(B, status=status, stream=stream)
    out["t1"] = csr_matmul(out["bt"], out["k2b"], status, stream)
    out["a"], _ = seacells_csr_transpose(At, status=status, stream=stream)
    out["aat"] = csr_matmul(out["a"], At, status, stream)
    out["kat"] = csr_matmul(K, At, status, stream)
    out["k2at"] = csr_matmul(K, out["kat"], status, stream)
    raise_on_status(status)
    return out


def seacells_csr_add_workspace(m: int) -> int:
    return int(load().seacells_csr_add_workspace(m))


def seacells_csr_add_rows(x: DeviceCSR, y: DeviceCSR, c_row_ptr=None, workspace=None, status=None,
                          stream=None):
    """Row pointer of x + y (union pattern). Returns (c_row_ptr, status)."""
    lib = load()
    dev = x.row_ptr.device
    if c_row_ptr is None:
        c_row_ptr = torch.empty(x.shape[0] + 1, dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty(seacells_csr_add_workspace(x.shape[0]), dtype=torch.uint8,
                                device=dev)
    sx, sy = x.struct(), y.struct()
    rc = lib.seacells_csr_add_rows(ctypes.byref(sx), ctypes.byref(sy), _ptr(c_row_ptr),
                                   _ptr(workspace), workspace.numel(), _ptr(status),
                                   _stream(stream))
    _check_rc(rc)
    return c_row_ptr, status


def seacells_csr_add_fill(alpha: float, x: DeviceCSR, beta: float, y: DeviceCSR, c_row_ptr,
                          c_col_idx, c_val, status=None, stream=None):
    """Columns and values of alpha x + beta y into buffers sized by c_row_ptr[-1]."""
    lib = load()
    if status is None:
        status = new_status(x.row_ptr.device)
    sx, sy = x.struct(), y.struct()
    rc = lib.seacells_csr_add_fill(float(alpha), ctypes.byref(sx), float(beta), ctypes.byref(sy),
                                   _ptr(c_row_ptr), _ptr(c_col_idx) if c_col_idx.numel() else None,
                                   _ptr(c_val) if c_val.numel() else None,
                                   min(c_col_idx.numel(), c_val.numel()), _ptr(status),
                                   _stream(stream))
    _check_rc(rc)
    return c_col_idx, c_val, status


class OutBuffers:
    """Reusable output arrays for repeated sums or products of growing size:
    a row pointer and index / value arrays kept with headroom, handed out as
    views of the length each call needs (the arrays are reallocated only
    when a call needs more)."""

    def __init__(self, headroom: float = 1.25):
        self.headroom = headroom
        self.ptr = self.idx = self.val = None

    def row_ptr(self, rows: int, dev):
        if self.ptr is None or self.ptr.numel() != rows + 1 or self.ptr.device != dev:
            self.ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
        return self.ptr

    def entries(self, nnz: int, dev):
        if self.idx is None or self.idx.numel() < nnz or self.idx.device != dev:
            cap = max(int(nnz * self.headroom), 1)
            self.idx = self.val = None  # let the old arrays go before the new ones exist
            self.idx = torch.empty(cap, dtype=torch.int32, device=dev)
            self.val = torch.empty(cap, dtype=torch.float32, device=dev)
        return self.idx[:nnz], self.val[:nnz]


def csr_add(alpha: float, x: DeviceCSR, beta: float, y: DeviceCSR, status=None,
            stream=None, out: OutBuffers = None, bound=None) -> DeviceCSR:
    """alpha x + beta y as a DeviceCSR. Without ``bound``: one
    synchronisation sizes the output and a device status flag raises; with
    ``bound`` (at least nnz of the sum, e.g. nnz(x) + nnz(y)): no
    synchronisation, as csr_matmul. ``out`` (OutBuffers) reuses its arrays;
    x and y must not live in them."""
    dev = x.row_ptr.device
    if status is None:
        status = new_status(dev)
    c_ptr = out.row_ptr(x.shape[0], dev) if out is not None else None
    c_ptr, _ = seacells_csr_add_rows(x, y, c_row_ptr=c_ptr, status=status, stream=stream)
    if bound is None:
        raise_on_status(status)
        nnz = int(c_ptr[-1].item()) & 0xffffffff
    else:
        nnz = int(bound)
    if out is not None:
        c_idx, c_val = out.entries(nnz, dev)
    else:
        c_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
        c_val = torch.empty(nnz, dtype=torch.float32, device=dev)
    seacells_csr_add_fill(alpha, x, beta, y, c_ptr, c_idx, c_val, status=status, stream=stream)
    return DeviceCSR(c_ptr, c_idx, c_val, x.shape)


def seacells_fw_b_vertex_workspace(k: int, n: int) -> int:
    return int(load().seacells_fw_b_vertex_workspace(k, n))


def seacells_fw_b_vertex(arg_idx, n: int, value: float = 1.0, workspace=None, status=None,
                         stream=None) -> DeviceCSR:
    """The n x k vertex matrix S (``value`` at (arg_idx[c], c)) as a DeviceCSR."""
    lib = load()
    dev = arg_idx.device
    k = int(arg_idx.numel())
    if arg_idx.dtype != torch.int32 or not arg_idx.is_contiguous():
        raise SeacellsError("arg_idx must be a contiguous int32 tensor")
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty(seacells_fw_b_vertex_workspace(k, n), dtype=torch.uint8,
                                device=dev)
    s_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    s_idx = torch.empty(k, dtype=torch.int32, device=dev)
    s_val = torch.empty(k, dtype=torch.float32, device=dev)
    rc = lib.seacells_fw_b_vertex(_ptr(arg_idx) if k else None, k, n, float(value), _ptr(s_ptr),
                                  _ptr(s_idx) if k else None, _ptr(s_val) if k else None,
                                  _ptr(workspace), workspace.numel(), _ptr(status),
                                  _stream(stream))
    _check_rc(rc)
    return DeviceCSR(s_ptr, s_idx, s_val, (n, k))


def seacells_fw_step_size(t: int):
    """(gamma_t, 1 - gamma_t) of the default schedule, as f32 values."""
    g, keep = ctypes.c_float(), ctypes.c_float()
    _check_rc(load().seacells_fw_step_size(t, ctypes.byref(g), ctypes.byref(keep)))
    return g.value, keep.value


def fw_b_loop(K: DeviceCSR, k2b: DeviceCSR, aat: DeviceCSR, k2at: DeviceCSR, b: DeviceCSR,
              steps: int, gammas=None, status=None, stream=None):
    """``steps`` Frank-Wolfe steps of the B update on the device, A fixed.

    Step t: the B argmin (seacells_fw_b_argmin) gives the row of every
    column; S is their vertex matrix; B <- (1 - g) B + g S and
    K^2 B <- (1 - g) K^2 B + g K (K S), with g = gammas[t] (default
    2 / (t + 2)). Returns (b, k2b, picks [steps, k], mins [steps, k],
    gaps [steps]) with the last three on the device. Every product and sum
    runs in the library; the host only reads output sizes.
    """
    n, k = k2b.shape
    dev = k2b.row_ptr.device
    if status is None:
        status = new_status(dev)
    picks = torch.empty((steps, k), dtype=torch.int32, device=dev)
    mins = torch.empty((steps, k), dtype=torch.float32, device=dev)
    gaps = torch.empty(steps, dtype=torch.float32, device=dev)
    ws_b = torch.empty(seacells_fw_b_argmin_workspace(n, k, aat.nnz), dtype=torch.uint8,
                       device=dev)
    ws_v = torch.empty(seacells_fw_b_vertex_workspace(k, n), dtype=torch.uint8, device=dev)
    # B and K^2 B alternate between two sets of arrays (a sum reads the old
    # matrix while it writes the new one), kept across steps with headroom.
    # Sizes are read back per product and sum: bounds known on the host (K's
    # largest row, K^2's largest row) are loose enough on kNN graphs with hub
    # cells that the outputs they reserve cost more than the reads.
    b_out, k_out = (OutBuffers(), OutBuffers()), (OutBuffers(), OutBuffers())
    kw = dict(status=status, stream=stream)
    for t in range(steps):
        if gammas is None:
            g, keep = seacells_fw_step_size(t)
        else:  # a caller's table: its entries as given
            g = float(gammas[t])
            keep = 1.0 - g
        seacells_fw_b_argmin(k2b, aat, k2at, b, n, k, out_val=mins[t], out_idx=picks[t],
                             gap=gaps[t:t + 1], workspace=ws_b, **kw)
        S = seacells_fw_b_vertex(picks[t], n, 1.0, workspace=ws_v, **kw)
        b = csr_add(keep, b, g, S, out=b_out[t % 2], **kw)
        k2s = csr_matmul(K, csr_matmul(K, S, **kw), **kw)
        k2b = csr_add(keep, k2b, g, k2s, out=k_out[t % 2], **kw)
    raise_on_status(status)
    return b, k2b, picks, mins, gaps


def csr_trim(m: DeviceCSR) -> DeviceCSR:
    """The same matrix with nnz read from its row pointer (one
    synchronisation): the exact size of an output of the bounded mode of
    csr_matmul or csr_add."""
    nnz = int(m.row_ptr[-1].item()) & 0xffffffff
    return DeviceCSR(m.row_ptr, m.col_idx[:nnz], m.val[:nnz], m.shape)


def seacells_fw_a_to_csr_workspace(n: int) -> int:
    return int(load().seacells_fw_a_to_csr_workspace(n))


def seacells_fw_a_to_csr_rows(atom_idx, atom_val, atom_cnt, k: int, at_row_ptr=None,
                              workspace=None, status=None, stream=None):
    """Row pointer of A^T from the A update's atoms. Returns (at_row_ptr, status)."""
    lib = load()
    n, cap = atom_idx.shape
    dev = atom_idx.device
    if at_row_ptr is None:
        at_row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty(seacells_fw_a_to_csr_workspace(n), dtype=torch.uint8, device=dev)
    _check_rc(lib.seacells_fw_a_to_csr_rows(_ptr(atom_idx), _ptr(atom_val), _ptr(atom_cnt), n, k,
                                            cap, _ptr(at_row_ptr), _ptr(workspace),
                                            workspace.numel(), _ptr(status), _stream(stream)))
    return at_row_ptr, status


def seacells_fw_a_to_csr_fill(atom_idx, atom_val, atom_cnt, k: int, at_row_ptr, at_col_idx,
                              at_val, status=None, stream=None):
    """Columns and weights of A^T into buffers sized by at_row_ptr[-1]."""
    lib = load()
    n, cap = atom_idx.shape
    if status is None:
        status = new_status(atom_idx.device)
    _check_rc(lib.seacells_fw_a_to_csr_fill(_ptr(atom_idx), _ptr(atom_val), _ptr(atom_cnt), n, k,
                                            cap, _ptr(at_row_ptr),
                                            _ptr(at_col_idx) if at_col_idx.numel() else None,
                                            _ptr(at_val) if at_val.numel() else None,
                                            _ptr(status), _stream(stream)))
    return at_col_idx, at_val, status


def fw_a_to_csr(atom_idx, atom_val, atom_cnt, k: int, status=None, stream=None) -> DeviceCSR:
    """The A update's atoms ([n, cap] int32 / float32, [n] int32) as the CSR
    A^T (n x k): non-zero weights, columns ascending. One synchronisation
    sizes the output; raises on a device status flag."""
    n = atom_idx.shape[0]
    dev = atom_idx.device
    if status is None:
        status = new_status(dev)
    ptr, _ = seacells_fw_a_to_csr_rows(atom_idx, atom_val, atom_cnt, k, status=status,
                                       stream=stream)
    raise_on_status(status)
    nnz = int(ptr[-1].item()) & 0xffffffff
    idx = torch.empty(nnz, dtype=torch.int32, device=dev)
    val = torch.empty(nnz, dtype=torch.float32, device=dev)
    seacells_fw_a_to_csr_fill(atom_idx, atom_val, atom_cnt, k, ptr, idx, val, status=status,
                              stream=stream)
    return DeviceCSR(ptr, idx, val, (n, k))


def outer_iteration(K: DeviceCSR, b: DeviceCSR, k2b: DeviceCSR, a_t: DeviceCSR, steps_a: int,
                    steps_b: int, cap=None, trace=False, status=None, stream=None) -> dict:
    """One SEACells outer iteration on the device, every step in the library.

    A update with B fixed: P = B^T K^2 B (a transpose and a product) and
    t1 = (P + P^T) / 2 (exactly symmetric), then seacells_fw_a_columns from
    A_prev = a_t for steps_a steps (cap default: widest row of a_t +
    steps_a); its atoms become the new A^T. B update with A fixed:
    A A^T = (A^T)^T A^T and K^2 A^T = K (K A^T), then fw_b_loop for
    steps_b steps. Last, the RSS ||K - K B A||^2 of the new pair (f64).
    Returns a dict: b, k2b, a_t, t1, aat, k2at (DeviceCSR), rss ([1] f64),
    a_trace ([n, steps_a] when trace), b_picks, b_mins, b_gaps.
    """
    n, k = b.shape
    dev = b.row_ptr.device
    if status is None:
        status = new_status(dev)
    kw = dict(status=status, stream=stream)
    bt, _ = seacells_csr_transpose(b, **kw)
    p = csr_matmul(bt, k2b, **kw)
    pt, _ = seacells_csr_transpose(p, **kw)
    t1 = csr_add(0.5, p, 0.5, pt, **kw)
    if cap is None:
        rows = np.diff(a_t.row_ptr.cpu().numpy().astype(np.int64))
        cap = int(rows.max() if rows.size else 0) + steps_a
    ai, av, ac, tr, _ = seacells_fw_a_columns(t1, k2b, a_t, n, k, steps_a, cap, trace=bool(trace),
                                              **kw)
    raise_on_status(status)
    a_t2 = fw_a_to_csr(ai, av, ac, k, **kw)
    a, _ = seacells_csr_transpose(a_t2, **kw)
    aat = csr_matmul(a, a_t2, **kw)
    k2at = csr_matmul(K, csr_matmul(K, a_t2, **kw), **kw)
    b2, k2b2, picks, mins, gaps = fw_b_loop(K, k2b, aat, k2at, b, steps_b, **kw)
    bt2, _ = seacells_csr_transpose(b2, **kw)
    p2 = csr_matmul(bt2, k2b2, **kw)
    acc, _ = rss(K, k2b2, a_t2, p2, aat, **kw)
    raise_on_status(status)
    return {"b": b2, "k2b": k2b2, "a_t": a_t2, "t1": t1, "aat": aat, "k2at": k2at, "rss": acc,
            "a_trace": tr, "b_picks": picks, "b_mins": mins, "b_gaps": gaps}
