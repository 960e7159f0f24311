"""SEACells Frank-Wolfe hot path on MI355X (gfx950): HIP kernels behind a C ABI.

``native`` binds ``libseacells_fw.so`` (include/seacells_fw.h for the A and B
updates, include/seacells_sparse.h for the operand construction,
include/seacells_debug.h for the test hooks); ``csrc/``
holds the HIP sources; ``_build`` compiles them in-tree.
"""
from .native import (DeviceCSR, SeacellsError, load, new_status, raise_on_status,  # noqa: F401
                     seacells_fw_a_columns, seacells_fw_a_columns_pruned, seacells_fw_a_columns_noalloc,
                     seacells_fw_a_columns_workspace,
                     seacells_fw_b_apply, seacells_fw_b_argmin, seacells_fw_b_argmin_workspace,
                     seacells_csr_matmul_workspace, seacells_csr_matmul_pattern_workspace,
                     seacells_csr_matmul_rows,
                     seacells_csr_matmul_fill, csr_matmul,
                     seacells_csr_transpose_workspace, seacells_csr_transpose,
                     seacells_csr_dot_workspace, seacells_csr_dot, rss, device_operands,
                     seacells_csr_add_workspace, seacells_csr_add_rows, seacells_csr_add_fill,
                     csr_add, seacells_fw_b_vertex_workspace, seacells_fw_b_vertex, fw_b_loop,
                     seacells_fw_a_to_csr_workspace, seacells_fw_a_to_csr_rows,
                     seacells_fw_a_to_csr_fill, fw_a_to_csr, outer_iteration, csr_trim,
                     seacells_debug_set_a_options, seacells_debug_b_layout,
                     seacells_debug_b_last_epoch, seacells_debug_b_reduce, status_flags,
                     seacells_fw_step_size)
