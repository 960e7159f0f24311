/*
 * seacells_fw.h - C ABI of the SEACells Frank-Wolfe hot path on MI355X
 * (gfx950).
 *
 * The library runs the two data-parallel Frank-Wolfe updates of SEACells
 * kernel archetypal analysis, min ||K - K B A||_F^2 over column-stochastic
 * B (n x k) and A (k x n), on one GPU:
 *
 *   - the per-cell A column solve (seacells_fw_a_columns), and its pruning
 *     variant (seacells_fw_a_columns_pruned);
 *   - the per-archetype B-gradient argmin over cells (seacells_fw_b_argmin)
 *     and the B step that consumes it (seacells_fw_b_apply).
 *
 * The method is the one on the docs.rs source page "bixverse-rs 0.6.4 -
 * src/gpu/sc_gpu/kernels/seacells_kernels.rs". Building K, K^2 B, t1,
 * A A^T, K^2 A^T and the RSS stays with the caller on the host, as the
 * page's module doc places it.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Sparse operands are CSR (seacells_csr). row_ptr, col_idx and val are
 *   device pointers. Column indices are strictly ascending within a row and
 *   below n_cols. nnz == row_ptr[n_rows] and nnz < 2^31. Values are finite.
 *   These are preconditions: the library does not read device memory on the
 *   host to check them.
 * - Every n x k matrix is CSR over cells (rows = cells), as on the page's
 *   module doc. k x k matrices (t1 = B^T K^2 B, A A^T) must be symmetric:
 *   the page adds row `amin` of t1 where the maths adds column `amin`.
 * - Ownership: the caller allocates and frees every buffer (inputs,
 *   outputs, workspace, the status word). The library never allocates,
 *   frees or synchronises. All work is enqueued on `stream` (a hipStream_t;
 *   NULL = the default stream). Outputs are ready when the stream is.
 * - Return value: SEACELLS_OK, or a negative SEACELLS_E_* code detected
 *   synchronously on the host before any device work is enqueued
 *   (SEACELLS_E_HIP: a launch failed; the HIP message is available from
 *   seacells_last_error()).
 * - *status (a device uint32) is overwritten by every call with the OR of
 *   the SEACELLS_FLAG_* conditions the kernels detected; read it after the
 *   stream synchronises. A non-zero status means the outputs are not valid.
 * - Results are deterministic: no floating-point atomics, fixed reduction
 *   orders; two calls on the same inputs give bitwise-equal outputs.
 * - Calls that share a workspace or status word must not overlap.
 * - There is no ceiling on k: state that does not fit the compute unit's
 *   local memory moves to the workspace (A) or is split into column slices
 *   of at most 2048 columns (B, as many slices as k needs). What grows with
 *   k is the workspace the *_workspace() queries report; a caller who cannot
 *   provide it gets SEACELLS_E_WORKSPACE, never a silent no-op.
 */
#ifndef SEACELLS_FW_H
#define SEACELLS_FW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-detected errors (return values). */
#define SEACELLS_OK 0
#define SEACELLS_E_NULL (-1)      /* a required pointer is NULL */
#define SEACELLS_E_SHAPE (-2)     /* n, k or T is 0, or operand shapes disagree */
#define SEACELLS_E_WORKSPACE (-3) /* workspace smaller than the *_workspace() size */
#define SEACELLS_E_TOO_LARGE (-4) /* n, k or nnz >= 2^31, n * cap >= 2^40, atom list > LDS */
#define SEACELLS_E_HIP (-5)       /* a HIP launch or query failed */

/* Device-detected conditions (bits of *status). */
#define SEACELLS_FLAG_CAP_OVERFLOW 0x1u     /* an A column needed more than `cap` atoms */
#define SEACELLS_FLAG_PARTIALS_INVALID 0x2u /* a B partial was stale or out of range */
#define SEACELLS_FLAG_B_CAP_OVERFLOW 0x4u   /* a padded B^T row was full */
#define SEACELLS_FLAG_BAD_INDEX 0x8u        /* an index argument was out of range */
#define SEACELLS_FLAG_NONFINITE 0x10u       /* an argmin found no finite minimum */
#define SEACELLS_FLAG_BAD_GAMMA 0x20u       /* a step size outside (0, 1] */

typedef struct ihipStream_t *seacells_stream_t; /* == hipStream_t */

/* A CSR matrix in device memory (the struct itself lives on the host). */
typedef struct seacells_csr {
    const uint32_t *row_ptr; /* [n_rows + 1], row_ptr[0] == 0, non-decreasing */
    const uint32_t *col_idx; /* [nnz], strictly ascending within a row, < n_cols */
    const float *val;        /* [nnz] */
    uint32_t n_rows;
    uint32_t n_cols;
    uint32_t nnz;
} seacells_csr;

/*
 * Workspace bytes seacells_fw_a_columns needs for these sizes (t1_nnz: the
 * non-zeros of t1). It holds a copy of t1 with every row padded to whole
 * chunks of 64 entries (at most 8 * (t1_nnz + 64 k) bytes) when a wave
 * takes one cell (k above 1024, or the pruning variant); for large k (from
 * 2048) two counters and queues of n cell ids (the cells the compact
 * per-cell state hands on); and per-wave state slices when not even one
 * cell's dense state fits in local memory. 0 when none is needed (small
 * k). Depends only on its arguments (and on the plan overrides of
 * seacells_debug.h, which tests set; they must be the same at the call).
 */
size_t seacells_fw_a_columns_workspace(uint32_t n, uint32_t k, uint32_t T, uint32_t cap,
                                       uint32_t t1_nnz);

/*
 * A update: the per-cell column solve of `fw_columns_a_gpu` on the source
 * page (its doc comment and the `a_columns_capacity` doc).
 *
 * For every cell j in [0, n), starting from a_j = row j of A_prev^T, run T
 * Frank-Wolfe steps t = 0 .. T-1 of
 *     g      = t1 . a_j - K2B[j, :]
 *     idx_t  = argmin_c g[c]   (lowest c on a tie; -0 == +0)
 *     a_j    = (1 - gamma_t) a_j + gamma_t e_idx_t
 * with gamma_t = gamma[t], or 2 / (t + 2) when gamma is NULL.
 *
 * t1        k x k CSR, symmetric (B^T K^2 B).
 * k2b       n x k CSR (K^2 B, rows = cells).
 * a_prev_t  n x k CSR (A_prev^T: row j holds column j of A_prev).
 * gamma     device [T] f32 step sizes in (0, 1], or NULL.
 * cap       atom slots per cell: at least max_j nnz(a_prev_t row j) + T,
 *           the page's `a_columns_capacity` rule. Overflow sets
 *           SEACELLS_FLAG_CAP_OVERFLOW.
 * atom_idx  device [n * cap] u32 out: the atoms of cell j at
 *           [j * cap, j * cap + atom_cnt[j]): the seeds first in A_prev
 *           order (a seed may end at weight 0: gamma_0 = 1 zeroes every
 *           seed), then each newly picked index in order of first pick.
 *           Indices are unique per cell. Slots past atom_cnt[j] are left
 *           unchanged.
 * atom_val  device [n * cap] f32 out: the matching weights of a_j.
 * atom_cnt  device [n] u32 out.
 * trace     device [n * T] u32 out, or NULL: trace[j * T + t] = idx_t.
 * fw_gap    device [n] f32 out, or NULL: the Frank-Wolfe duality gap of
 *           the returned column a_j (after the T steps), <g, a_j> -
 *           min_c g[c] with g = t1 . a_j - K2B[j, :] (without the factor 2,
 *           as on the page), i.e. the largest decrease rate of the objective
 *           towards a simplex vertex, an upper bound on a_j's distance to
 *           the optimum of its subproblem. The page's kernel computes only
 *           the B side's sum(B * G) half. Computed in f32 from the state,
 *           after the last step (no cost when NULL).
 * workspace device buffer of at least seacells_fw_a_columns_workspace()
 *           bytes (may be NULL when that is 0), 256-byte aligned.
 * k must be below 2^30 (else SEACELLS_E_TOO_LARGE).
 * SEACELLS_FLAG_NONFINITE: a cell's gradient state held no value below +inf
 * at some step (NaN or +inf everywhere: non-finite inputs); that step took
 * index 0. Entries that are NaN among finite ones never win the argmin.
 */
int seacells_fw_a_columns(const seacells_csr *t1, const seacells_csr *k2b,
                          const seacells_csr *a_prev_t, uint32_t n, uint32_t k,
                          uint32_t T, uint32_t cap, const float *gamma,
                          uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                          uint32_t *trace, float *fw_gap, void *workspace,
                          size_t workspace_bytes, uint32_t *status,
                          seacells_stream_t stream);

/*
 * A update with pruning and renormalisation: `fw_columns_a_gpu` with
 * `pruning` on the source page (its comments on dropping below the threshold
 * and renormalising the survivors, and `A_RENORM_FLOOR`).
 *
 * Every step is the step of seacells_fw_a_columns, then:
 *     every atom weight with a != 0 and -threshold <= a <= threshold becomes
 *     0 (its slot stays, so a later pick of that index lands back in it);
 *     total = sum of the weights; if total > 1e-15 every weight is multiplied
 *     by 1 / total (and the gradient state with it).
 * threshold   f32, finite and >= 0 (else SEACELLS_E_SHAPE); compared in f32.
 * Other arguments, outputs, errors and the workspace
 * (seacells_fw_a_columns_workspace covers both entry points) are those of
 * seacells_fw_a_columns (fw_gap: of the pruned, renormalised column that is
 * returned); atom_val holds 0 for a dropped slot. A cell that
 * drops an atom is finished by the dense-state kernel, so pruning that bites
 * costs more than the plain update.
 */
int seacells_fw_a_columns_pruned(const seacells_csr *t1, const seacells_csr *k2b,
                                 const seacells_csr *a_prev_t, uint32_t n, uint32_t k,
                                 uint32_t T, uint32_t cap, const float *gamma, float threshold,
                                 uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                                 uint32_t *trace, float *fw_gap, void *workspace,
                                 size_t workspace_bytes, uint32_t *status,
                                 seacells_stream_t stream);

/*
 * A update that allocates nothing, for callers that cannot call hipMalloc:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. It is seacells_fw_a_columns (same arguments, kernels, outputs
 * and errors) with the workspace taken from a static device array of
 * SEACELLS_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends. The caller still provides inputs, outputs and
 * the status word.
 *
 * Returns SEACELLS_E_TOO_LARGE, before anything is enqueued, when
 * seacells_fw_a_columns_workspace() for these sizes exceeds
 * SEACELLS_NOALLOC_SCRATCH_BYTES (at n = 1M, k = 10000 it needs about 80
 * MB). Every call on one GPU shares that GPU's array, and the library
 * rewrites whatever it reads from it on each call: calls that overlap on one
 * GPU (other streams, other threads) race and must not be issued. The first
 * call on a device looks the array's device address up once (a HIP symbol
 * query; SEACELLS_E_HIP if that fails).
 */
#define SEACELLS_NOALLOC_SCRATCH_BYTES (128u << 20)

int seacells_fw_a_columns_noalloc(const seacells_csr *t1, const seacells_csr *k2b,
                                  const seacells_csr *a_prev_t, uint32_t n, uint32_t k,
                                  uint32_t T, uint32_t cap, const float *gamma,
                                  uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                                  uint32_t *trace, float *fw_gap, uint32_t *status,
                                  seacells_stream_t stream);

/*
 * Workspace bytes seacells_fw_b_argmin needs for these sizes (always > 0;
 * aat_nnz: the non-zeros of A A^T). It holds the per-row-range partials
 * (8 bytes per column each; 8192 row ranges for k <= 2048, else 16384, fewer
 * when that would pass 2 GiB, at least one), one stamp and one gap partial
 * per (row range, column slice), an f64 gap sum per reduce chunk (at most
 * 64), and a copy of A A^T made per call. When k
 * fits one column slice (k <= 2048) the copy pads every row to whole
 * chunks of 64 entries (at most 8 (aat_nnz + 64 k) bytes). Otherwise the
 * columns are cut into slices of at most 1024 columns (and about 3.75 MB of
 * A A^T each) and the workspace also holds the column-slice tables of A A^T
 * (4 (k + 1) bytes per slice) and of K2At's rows (4 (n + 1) bytes per
 * slice), the run table (4 bytes per run and 8 per 1024 runs) and the
 * chunked copy of A A^T per slice (chunks of
 * 32 entries at 6 bytes each, at most aat_nnz / 32 + k slices + 1 chunks),
 * the in-slice column order (12 k bytes and 2 bytes per slice column) and,
 * with more slices than the GPU's 8 XCDs, the slices each XCD owns (4 k +
 * 12 bytes per slice + 36). Depends only on its arguments.
 */
size_t seacells_fw_b_argmin_workspace(uint32_t n, uint32_t k, uint32_t aat_nnz);

/*
 * B-gradient argmin: `fw_argmin_b` followed by `reduce_argmin_blocks` on
 * the source page (their doc comments, and the tests
 * `test_fw_argmin_b_handles_empty_rows` and
 * `test_fw_argmin_b_tie_breaks_on_lowest_row`).
 *
 *     G[i, c]    = sum_m K2B[i, m] AAt[m, c] - K2At[i, c]   (never stored)
 *     out_idx[c] = lowest i attaining min_i G[i, c]; out_val[c] = that min
 *     gap        = sum_{i, c} B[i, c] G[i, c]  (the page's sum(B * G) half
 *                  of the duality gap)
 *     fw_gap     = gap - sum_c out_val[c], the full Frank-Wolfe duality gap
 *                  of B (max over vertex matrices S of <G, B - S>)
 * Every row takes part, including rows whose K2B row is empty.
 *
 * k2b   n x k CSR (K^2 B).     aat   k x k CSR, symmetric (A A^T).
 * k2at  n x k CSR (K^2 A^T).   b     n x k CSR (B), or NULL: gap = 0.
 * out_val  device [k] f32 out.   out_idx  device [k] u32 out.
 * gap      device [1] f32 out, or NULL.
 * fw_gap   device [1] f32 out, or NULL; needs b (else SEACELLS_E_NULL).
 *          Both sums are taken in f64 in a fixed order, then rounded.
 * The reduce stage checks every partial it consumes: the stamp of its
 * (row range, column slice) unit must be this call's, and its row must lie
 * in the unit's row range (so below n); otherwise it sets
 * SEACELLS_FLAG_PARTIALS_INVALID. SEACELLS_FLAG_NONFINITE: a column minimum
 * is not finite, or some row range saw no value below +inf in a column.
 */
int seacells_fw_b_argmin(const seacells_csr *k2b, const seacells_csr *aat,
                         const seacells_csr *k2at, const seacells_csr *b, uint32_t n,
                         uint32_t k, float *out_val, uint32_t *out_idx, float *gap,
                         float *fw_gap, void *workspace, size_t workspace_bytes, uint32_t *status,
                         seacells_stream_t stream);

/*
 * B step: B_c <- (1 - gamma) B_c + gamma e_{arg_idx[c]} for every column c,
 * the update the B argmin feeds (the page leaves it to its caller).
 *
 * B^T is held as padded rows, one per archetype: row c has bt_cnt[c]
 * entries at bt_idx[c * cap_b + s] (cell indices, ascending) and
 * bt_val[c * cap_b + s]. A cell not yet in the row is inserted at its
 * sorted position. A full row is left unchanged and sets
 * SEACELLS_FLAG_B_CAP_OVERFLOW; arg_idx[c] >= n sets
 * SEACELLS_FLAG_BAD_INDEX (row unchanged).
 *
 * bt_idx, bt_val  device [k * cap_b], updated in place.
 * bt_cnt          device [k], updated in place.
 * arg_idx         device [k] (out_idx of seacells_fw_b_argmin).
 * gamma           host scalar in (0, 1].
 */
int seacells_fw_b_apply(uint32_t *bt_idx, float *bt_val, uint32_t *bt_cnt, uint32_t n,
                        uint32_t k, uint32_t cap_b, const uint32_t *arg_idx, float gamma,
                        uint32_t *status, seacells_stream_t stream);

/*
 * The default Frank-Wolfe step of step t (from 0), on the host: *gamma =
 * 2 / (t + 2) and *keep = 1 - *gamma, both in f32 with IEEE division and
 * subtraction, the values the A update computes on the device when it has no
 * step-size table (the page's `fw_columns_a_gpu` loop; the B loop steps every
 * column with the same schedule). Either pointer may be NULL. Returns
 * SEACELLS_OK.
 */
int seacells_fw_step_size(uint32_t t, float *gamma, float *keep);

/* Static text for a SEACELLS_E_* code. */
const char *seacells_status_string(int code);

/* Detail of the last SEACELLS_E_HIP on the calling thread ("" if none). */
const char *seacells_last_error(void);

/* ABI version, (major << 16) | minor. */
int seacells_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEACELLS_FW_H */
