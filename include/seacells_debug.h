/*
 * seacells_debug.h - test and experiment hooks of libseacells_fw.so.
 *
 * Nothing here is needed to run the Frank-Wolfe updates. These entry points
 * exist so that tests can (a) pin the A update's plan to one kernel and
 * compare kernels bit for bit, and (b) exercise the check the B argmin's
 * reduce stage makes on its partials: the source page (bixverse-rs 0.6.4,
 * seacells_kernels.rs, the `B_ARGMIN_WG_TIERS` doc and
 * `reduce_argmin_blocks`) warns that a reduce which trusts its partials
 * fills the output with whatever the partial buffers held, and asks callers
 * to check the partials rather than the output.
 *
 * Conventions, errors and ownership are those of seacells_fw.h.
 */
#ifndef SEACELLS_DEBUG_H
#define SEACELLS_DEBUG_H

#include <stddef.h>
#include <stdint.h>

#include "seacells_fw.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Plan overrides of the A update (seacells_fw_a_columns, its pruning
 * variant and seacells_fw_a_columns_workspace). Process-wide and not
 * thread-safe: set them before the workspace query and leave them unchanged
 * until the calls that use that workspace have been enqueued. Every
 * override gives the same outputs bit for bit (they only choose which
 * kernel computes them); tests use that.
 */
typedef struct seacells_a_options {
    int32_t support;        /* -1: by k (default); 0: never the compact support
                               state; 1: the support state for any k */
    uint32_t support_waves; /* 0: default; 4 .. 32: resident waves per CU the
                               first support pass is sized for */
    int32_t dense_argmin;   /* 1: a dense scan decides every step */
    uint32_t group;         /* 0: by k; 16, 32 or 64 lanes per cell in the
                               dense-state kernels */
    int32_t support_wide;   /* -1: by K2B's mean row length (default); 0: the
                               first support pass keeps 256 K2B entries per
                               cell in registers; 1: 512 */
} seacells_a_options;

/* Set the overrides; NULL restores the defaults. SEACELLS_E_SHAPE on a value
 * outside the ranges above (nothing changes then). */
int seacells_debug_set_a_options(const seacells_a_options *opt);

/*
 * Where seacells_fw_b_argmin keeps its partials in the workspace, for sizes
 * (n, k, aat_nnz). The partials are one u64 key per (row range rb, column c)
 * at byte keys_offset + 8 (rb * k + c): the order-preserving u32 image of
 * the f32 minimum over the unit's rows in the high half (-0 folded onto +0;
 * negative x maps to ~bits(x), non-negative x to bits(x) | 2^31) and the
 * row holding it (lowest on a tie) in the low half. Row range rb covers rows
 * [n rb / n_row_blocks, n (rb + 1) / n_row_blocks) (integer division).
 * Column c belongs to slice c / slice_w, and unit (rb, slice s) writes the
 * u32 stamp at byte stamps_offset + 4 (rb * n_slices + s) with the call's
 * epoch after writing its keys.
 */
typedef struct seacells_b_layout {
    uint64_t keys_offset;
    uint64_t stamps_offset;
    uint32_t n_row_blocks;
    uint32_t n_slices;
    uint32_t slice_w;
    uint32_t reserved;
} seacells_b_layout;

int seacells_debug_b_layout(uint32_t n, uint32_t k, uint32_t aat_nnz, seacells_b_layout *out);

/* The epoch the calling thread's last seacells_fw_b_argmin stamped its
 * partials with (0 before the first call). */
uint32_t seacells_debug_b_last_epoch(void);

/*
 * The reduce stages of seacells_fw_b_argmin alone, over the partials in
 * `workspace` (laid out for (n, k, aat_nnz)), expecting `epoch` in every
 * stamp. Outputs as seacells_fw_b_argmin's out_val, out_idx and gap (gap may
 * be NULL). Every partial is checked: a stamp other than `epoch`, or a key
 * whose row lies outside its row range, sets SEACELLS_FLAG_PARTIALS_INVALID
 * (a unit that saw no value below +inf sets SEACELLS_FLAG_NONFINITE); the
 * outputs are then not valid. *status is overwritten. The kernels read only
 * the workspace and always run to completion.
 */
int seacells_debug_b_reduce(uint32_t n, uint32_t k, uint32_t aat_nnz, uint32_t epoch,
                            float *out_val, uint32_t *out_idx, float *gap, void *workspace,
                            size_t workspace_bytes, uint32_t *status, seacells_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEACELLS_DEBUG_H */
