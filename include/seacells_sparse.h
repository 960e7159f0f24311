/*
 * seacells_sparse.h - C ABI of the sparse operations that build the
 * Frank-Wolfe operands of SEACells on MI355X (gfx950), in the same library
 * as seacells_fw.h (libseacells_fw.so).
 *
 * On the docs.rs source page "bixverse-rs 0.6.4 -
 * src/gpu/sc_gpu/kernels/seacells_kernels.rs" the operands come from host
 * routines (the page's module doc: kernel construction and the RSS stay on
 * the host; its `lower_bound` doc names `csr_matmul_csr`, which sorts each
 * output row, and `transpose_sparse`, which writes rows in ascending major
 * order). These entry points do the same work on the device:
 *
 *   K^2 X  = K (K X)           two products        (X = B or A^T)
 *   t1     = B^T (K^2 B)       a transpose, a product
 *   A A^T  = (A^T)^T A^T       a transpose, a product
 *   RSS    = ||K - K B A||_F^2 = <K, K> - 2 <K^2 B, A^T> + <t1, A A^T>
 *            (three inner products, no n x n or dense product formed)
 *
 * Conventions (as in seacells_fw.h): CSR operands are seacells_csr with
 * device pointers, column indices strictly ascending within a row, nnz <
 * 2^31, finite values. The caller allocates every buffer; the library never
 * allocates or synchronises and enqueues all work on `stream`. Return values
 * are SEACELLS_OK or a negative SEACELLS_E_* code found on the host before
 * anything is enqueued; *status (device) receives the OR of SEACELLS_FLAG_*
 * conditions the kernels met. Results are deterministic (fixed summation
 * orders, no floating-point atomics).
 */
#ifndef SEACELLS_SPARSE_H
#define SEACELLS_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#include "seacells_fw.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The product's (or transpose's) output would hold 2^31 or more entries. */
#define SEACELLS_FLAG_OUTPUT_TOO_LARGE 0x40u

/* Workspace bytes seacells_csr_matmul_rows needs for a product with m rows
 * (> 0; about 8 bytes per 4096 rows). */
size_t seacells_csr_matmul_workspace(uint32_t m);

/* Workspace bytes with which the rows pass also keeps every row's output
 * columns (a bitmap, m * ceil(q / 32) words) for the fill pass, which then
 * reads them instead of recomputing them: an m x q product with q <= 16384;
 * 0 when q is larger (the fill pass always recomputes then). */
size_t seacells_csr_matmul_pattern_workspace(uint32_t m, uint32_t q);

/*
 * Product C = A B, step 1 of 2 (`csr_matmul_csr` on the page): the row
 * pointer of C. a is m x p, b is p x q (else SEACELLS_E_SHAPE).
 * workspace: at least seacells_csr_matmul_workspace(m) bytes, 256-byte
 * aligned (else SEACELLS_E_WORKSPACE); with at least
 * seacells_csr_matmul_pattern_workspace(m, q) bytes it also keeps the rows'
 * column bitmaps for step 2.
 * c_row_ptr  device [m + 1] u32 out: c_row_ptr[i] = first entry of row i;
 *            c_row_ptr[m] = nnz(C), for the caller to size c_col_idx and
 *            c_val (read it after the stream synchronises). Row i holds every
 *            column some product a[i, j] b[j, c] reaches, so a sum that cancels
 *            to 0 stays as an explicit 0 (the page does not say whether its
 *            host product keeps such zeros; with non-negative K, B and A no sum
 *            cancels, so the operands are the same either way).
 * SEACELLS_FLAG_OUTPUT_TOO_LARGE when nnz(C) would reach 2^31 (c_row_ptr
 * is then not valid); BAD_INDEX for malformed rows or columns (skipped).
 */
int seacells_csr_matmul_rows(const seacells_csr *a, const seacells_csr *b, uint32_t *c_row_ptr,
                             void *workspace, size_t workspace_bytes, uint32_t *status,
                             seacells_stream_t stream);

/*
 * Product C = A B, step 2 of 2: columns (ascending in every row) and values.
 * c_row_ptr must be the output of seacells_csr_matmul_rows for the same a
 * and b; c_col_idx and c_val hold c_row_ptr[m] entries each (device, out).
 * workspace (may be NULL): the one step 1 used, unchanged since; when it is
 * at least seacells_csr_matmul_pattern_workspace(m, q) bytes, the row
 * bitmaps step 1 kept there are used (the caller guarantees they belong to
 * this a and b), otherwise the columns are recomputed. c_capacity: the
 * entries c_col_idx and c_val hold; when c_row_ptr[m] exceeds it nothing is
 * written and SEACELLS_FLAG_OUTPUT_TOO_LARGE is raised (so a caller that
 * sizes the outputs by a bound, without reading c_row_ptr[m], stays safe).
 * c[i, c] = sum over the entries j of a's row i, in order, and then over
 * b's row j, of a[i, j] * b[j, c], accumulated in f32 with fused
 * multiply-adds in that order. A row of a with 2048 entries or more, when b
 * has at most 16384 columns, is cut into 16 runs of consecutive entries
 * (run w: entries len * w / 16 to len * (w + 1) / 16 of the row, rounded
 * down), each run is summed that way from 0, and the 16 sums are added in
 * run order (with or without the rows pass's bitmaps). c_col_idx / c_val may be NULL only when the
 * product is empty (a non-empty row with no output arrays is skipped and
 * flagged BAD_INDEX).
 */
int seacells_csr_matmul_fill(const seacells_csr *a, const seacells_csr *b,
                             const uint32_t *c_row_ptr, uint32_t *c_col_idx, float *c_val,
                             size_t c_capacity, void *workspace, size_t workspace_bytes,
                             uint32_t *status, seacells_stream_t stream);

/* Workspace bytes seacells_csr_transpose needs for an m x q matrix (> 0). */
size_t seacells_csr_transpose_workspace(uint32_t m, uint32_t q);

/*
 * Transpose (`transpose_sparse` on the page): a is m x q; at (q x m) gets
 * at_row_ptr [q + 1], at_col_idx and at_val [nnz(a)] (device, out), every
 * row listing a's rows in ascending order. workspace: at least
 * seacells_csr_transpose_workspace(m, q) bytes, 256-byte aligned.
 */
int seacells_csr_transpose(const seacells_csr *a, uint32_t *at_row_ptr, uint32_t *at_col_idx,
                           float *at_val, void *workspace, size_t workspace_bytes,
                           uint32_t *status, seacells_stream_t stream);

/* Workspace bytes seacells_csr_dot needs (> 0). */
size_t seacells_csr_dot_workspace(void);

/*
 * Inner product of two matrices of the same shape, accumulated (the operand
 * with fewer entries is walked, the other searched):
 *     *acc += alpha * sum_{i, c} x[i, c] y[i, c]
 * acc  device [1] f64 (in/out). Products and sums in f64; rows are summed
 * in a fixed order. With K, K^2 B, A^T, t1 and A A^T, three calls into one
 * zeroed acc give the RSS (alpha = 1, -2, 1). workspace: at least
 * seacells_csr_dot_workspace() bytes, 256-byte aligned.
 */
int seacells_csr_dot(const seacells_csr *x, const seacells_csr *y, double alpha, double *acc,
                     void *workspace, size_t workspace_bytes, uint32_t *status,
                     seacells_stream_t stream);

/* Workspace bytes seacells_csr_add_rows needs for m rows (> 0). */
size_t seacells_csr_add_workspace(uint32_t m);

/*
 * Sum C = alpha X + beta Y, step 1 of 2 (`sparse_add_csr` on the page, which
 * merges two sorted rows): the row pointer of C. x and y have the same shape
 * m x q (else SEACELLS_E_SHAPE) and nnz(x) + nnz(y) < 2^31. C's pattern is
 * the union of the two stored patterns: a column stored in either row is
 * stored, even where the sum is 0.
 * c_row_ptr  device [m + 1] u32 out; c_row_ptr[m] = nnz(C).
 * workspace: at least seacells_csr_add_workspace(m) bytes, 256-byte aligned.
 * BAD_INDEX for malformed rows, columns >= q or rows not strictly ascending.
 */
int seacells_csr_add_rows(const seacells_csr *x, const seacells_csr *y, uint32_t *c_row_ptr,
                          void *workspace, size_t workspace_bytes, uint32_t *status,
                          seacells_stream_t stream);

/*
 * Sum C = alpha X + beta Y, step 2 of 2: columns (ascending) and values into
 * c_col_idx and c_val (device, c_row_ptr[m] entries each). c_row_ptr must be
 * seacells_csr_add_rows's output for the same x and y (else BAD_INDEX and no
 * write beyond its row sizes). Each value is alpha x and beta y rounded to
 * f32 separately, then their sum rounded (alpha x or beta y alone where only
 * one operand stores the column). c_capacity: the entries c_col_idx and
 * c_val hold; when c_row_ptr[m] exceeds it nothing is written and
 * SEACELLS_FLAG_OUTPUT_TOO_LARGE is raised.
 */
int seacells_csr_add_fill(float alpha, const seacells_csr *x, float beta, const seacells_csr *y,
                          const uint32_t *c_row_ptr, uint32_t *c_col_idx, float *c_val,
                          size_t c_capacity, uint32_t *status, seacells_stream_t stream);

/* Workspace bytes seacells_fw_b_vertex needs for k columns and n rows (> 0). */
size_t seacells_fw_b_vertex_workspace(uint32_t k, uint32_t n);

/*
 * The Frank-Wolfe vertex of the B step: the n x k CSR matrix S holding
 * `value` at (arg_idx[c], c) for every column c, where arg_idx [k] (device)
 * is the B argmin's row per column (seacells_fw_b_argmin's out_idx). With
 * it a B step is B <- (1 - gamma) B + gamma S (seacells_csr_add_* with value
 * 1), and K^2 B follows as (1 - gamma) K^2 B + gamma K (K S) (two products
 * and a sum), so a loop of B steps stays on the device.
 * s_row_ptr [n + 1], s_col_idx [k], s_val [k] (device, out): every row's
 * columns ascending. n >= 1 (else SEACELLS_E_SHAPE). workspace: at least
 * seacells_fw_b_vertex_workspace(k, n) bytes, 256-byte aligned. A pick >= n
 * is dropped and flagged BAD_INDEX.
 */
int seacells_fw_b_vertex(const uint32_t *arg_idx, uint32_t k, uint32_t n, float value,
                         uint32_t *s_row_ptr, uint32_t *s_col_idx, float *s_val, void *workspace,
                         size_t workspace_bytes, uint32_t *status, seacells_stream_t stream);

/* Workspace bytes seacells_fw_a_to_csr_rows needs for n cells (> 0). */
size_t seacells_fw_a_to_csr_workspace(uint32_t n);

/*
 * The A update's returned columns (seacells_fw_a_columns's atom_idx /
 * atom_val [n, cap], atom_cnt [n], device) as the CSR A^T (n x k) that the
 * next B update's operands are built from (A A^T = (A^T)^T A^T and
 * K^2 A^T = K (K A^T), as the page's layout convention passes every n x k
 * matrix), step 1 of 2: the row pointer. Row j holds cell j's atoms among
 * its first min(atom_cnt[j], cap) slots whose weight is not 0, in ascending
 * column order. at_row_ptr [n + 1] (device, out; at_row_ptr[n] = nnz).
 * workspace: at least seacells_fw_a_to_csr_workspace(n) bytes, 256-byte
 * aligned. BAD_INDEX for a count above cap or a column >= k (dropped).
 */
int seacells_fw_a_to_csr_rows(const uint32_t *atom_idx, const float *atom_val,
                              const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                              uint32_t *at_row_ptr, void *workspace, size_t workspace_bytes,
                              uint32_t *status, seacells_stream_t stream);

/*
 * Step 2 of 2: columns and weights into at_col_idx / at_val (device,
 * at_row_ptr[n] entries each). at_row_ptr must be step 1's output for the same
 * atoms (else BAD_INDEX and no write beyond its row sizes); a column held twice
 * by one cell is flagged BAD_INDEX.
 */
int seacells_fw_a_to_csr_fill(const uint32_t *atom_idx, const float *atom_val,
                              const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                              const uint32_t *at_row_ptr, uint32_t *at_col_idx, float *at_val,
                              uint32_t *status, seacells_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEACELLS_SPARSE_H */
