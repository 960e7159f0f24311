/*
 * Plain f64 CPU oracle for the two Frank-Wolfe updates of SEACells kernel
 * archetypal analysis: min ||K - K B A||_F^2 over column-stochastic B (n x k)
 * and A (k x n).
 *
 * TEST INFRASTRUCTURE. This is the slow, obviously-correct reference that the
 * HIP library is checked against. Only the test-suite, the smoke entry point
 * and the CPU-baseline leg of the benchmark load it. It shares no code,
 * header, table or helper with the HIP library, and the library never calls
 * it.
 *
 * Source of the method (cited by item, not by line): the docs.rs source page
 * "bixverse-rs 0.6.4 - src/gpu/sc_gpu/kernels/seacells_kernels.rs".
 *   - module doc: every n x k operand (K^2 B, K^2 A^T, B) is CSR over cells,
 *     t1 is k x k CSR with ascending columns.
 *   - `fw_columns_a_gpu` doc: per cell, seed from A_prev's column, then
 *     n_iters steps of amin = argmin_c (w[c] - K^2B[cell, c]) with
 *     w = t1 . a, gamma = 2 / (t + 2), a <- (1 - gamma) a + gamma e_amin;
 *     ties go to the lowest column.
 *   - `fw_argmin_b` doc: G[i, c] = sum_m K^2B[i, m] t1[m, c] - K^2A^T[i, c]
 *     (the t1 of the B update is A A^T), argmin over cells per column with
 *     the lowest row winning a tie, plus the sum(B * G) half of the duality
 *     gap.
 *   - test `cpu_fw_argmin_b`: loop order and strict `<` of the CPU scan.
 *
 * Inputs are exactly the f32 CSR operands the GPU receives; every value is
 * promoted to double (exact) and all arithmetic is f64. The A update
 * recomputes w = t1 . a from scratch at every step (no incremental state).
 *
 * Conventions: CSR arrays are (ptr[rows + 1], idx[nnz], val[nnz]) with u32
 * indices. Return value 0 on success, negative on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_E_ARG (-1)
#define ORACLE_E_INDEX (-2)
#define ORACLE_E_ALLOC (-3)
#define ORACLE_E_CAP (-4)

/* Number of contiguous row chunks the B scan is split into. Fixed, so the
 * f64 gap sum is the same whatever the thread count. */
#define ORACLE_B_CHUNKS 64

static int oracle_threads(int requested) {
#ifdef _OPENMP
    if (requested > 0) return requested;
    return omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

/* Weight sum at or below which the renormalisation is skipped (the page's
 * `A_RENORM_FLOOR`, mirroring the CPU side's floor). */
#define ORACLE_RENORM_FLOOR 1e-15

/* Check a CSR: monotone row pointers, column indices below n_cols. */
static int check_csr(uint32_t rows, uint32_t cols, const uint32_t *ptr,
                     const uint32_t *idx) {
    if (!ptr || !idx) return ORACLE_E_ARG;
    if (ptr[0] != 0) return ORACLE_E_INDEX;
    for (uint32_t r = 0; r < rows; ++r) {
        if (ptr[r + 1] < ptr[r]) return ORACLE_E_INDEX;
        for (uint32_t p = ptr[r]; p < ptr[r + 1]; ++p)
            if (idx[p] >= cols) return ORACLE_E_INDEX;
    }
    return 0;
}

/*
 * A update (the per-cell column solve of `fw_columns_a_gpu`).
 *
 * For every listed cell j, with a the dense k-vector of A_prev^T row j and
 * t2 the dense k-vector of K^2B row j, run T steps of
 *     g[c]  = sum_m t1[c, m] a[m] - t2[c]        for every c in [0, k)
 *     idx   = first c (scanning upward) with g[c] < best, best from +inf
 *     a     = (1 - gamma_t) a ;  a[idx] += gamma_t
 * with gamma_t = gamma[t], or 2 / (t + 2) when gamma is NULL.
 *
 * Trace outputs (each [n_cells * T], row-major by cell, all nullable):
 *   pick     - the oracle's own argmin idx at step t
 *   g_min    - g[idx]
 *   g_second - the second-smallest g over c != idx (equal to g_min on an
 *              exact tie), +inf when k == 1
 *   g_scale  - max(max_c |(t1 a)[c]|, max_c |t2[c]|), the size of the terms
 *              g is a difference of
 *   g_taken  - g at the index actually used for the update
 *   g_dot    - <g, a> = sum_c a[c] g[c] at this step's iterate (before the
 *              update); g_dot - g_min is the Frank-Wolfe duality gap there,
 *              max over simplex vertices e_v of <g, a - e_v>
 * force (nullable, [n_cells * T]): an entry >= 0 replaces idx in the update
 * (trace replay); the oracle's own argmin is still reported in pick.
 * a_out: [n_cells * k] dense f64 result.
 */
static int fw_a_columns_impl(uint32_t n, uint32_t k, uint32_t T,
                             const uint32_t *t1_ptr, const uint32_t *t1_idx,
                             const float *t1_val, const uint32_t *k2b_ptr,
                             const uint32_t *k2b_idx, const float *k2b_val,
                             const uint32_t *ap_ptr, const uint32_t *ap_idx,
                             const float *ap_val, const double *gamma,
                             const uint32_t *cells, uint32_t n_cells,
                             const int64_t *force, int prune, double threshold,
                             double *a_out, uint32_t *pick, double *g_min,
                             double *g_second, double *g_scale, double *g_taken,
                             double *g_dot, uint32_t *drops, double *margin,
                             int n_threads) {
    if (k == 0 || !t1_val || !k2b_val || !ap_val || !cells || !a_out)
        return ORACLE_E_ARG;
    int rc;
    if ((rc = check_csr(k, k, t1_ptr, t1_idx))) return rc;
    if ((rc = check_csr(n, k, k2b_ptr, k2b_idx))) return rc;
    if ((rc = check_csr(n, k, ap_ptr, ap_idx))) return rc;
    for (uint32_t ci = 0; ci < n_cells; ++ci)
        if (cells[ci] >= n) return ORACLE_E_INDEX;
    if (force)
        for (uint64_t e = 0; e < (uint64_t)n_cells * T; ++e)
            if (force[e] >= (int64_t)k) return ORACLE_E_INDEX;

    int fail = 0;
    const int nt = oracle_threads(n_threads);
#pragma omp parallel num_threads(nt)
    {
        double *t2 = (double *)malloc(sizeof(double) * k);
        double *w = (double *)malloc(sizeof(double) * k);
        if (!t2 || !w) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ci = 0; ci < (int64_t)n_cells; ++ci) {
            if (!t2 || !w) continue;
            const uint32_t j = cells[ci];
            double *a = a_out + (size_t)ci * k;
            for (uint32_t c = 0; c < k; ++c) a[c] = 0.0, t2[c] = 0.0;
            for (uint32_t p = ap_ptr[j]; p < ap_ptr[j + 1]; ++p)
                a[ap_idx[p]] = (double)ap_val[p];
            for (uint32_t p = k2b_ptr[j]; p < k2b_ptr[j + 1]; ++p)
                t2[k2b_idx[p]] = (double)k2b_val[p];

            for (uint32_t t = 0; t < T; ++t) {
                /* w = t1 . a, one dot product per row of t1 */
                double scale = 0.0;
                for (uint32_t c = 0; c < k; ++c) {
                    double s = 0.0;
                    for (uint32_t p = t1_ptr[c]; p < t1_ptr[c + 1]; ++p)
                        s += (double)t1_val[p] * a[t1_idx[p]];
                    w[c] = s;
                    if (fabs(s) > scale) scale = fabs(s);
                    if (fabs(t2[c]) > scale) scale = fabs(t2[c]);
                }
                /* lowest-index argmin under strict `<`, plus the runner-up */
                double best = INFINITY, second = INFINITY;
                uint32_t bi = 0;
                for (uint32_t c = 0; c < k; ++c) {
                    const double g = w[c] - t2[c];
                    if (g < best) {
                        second = best;
                        best = g;
                        bi = c;
                    } else if (g < second) {
                        second = g;
                    }
                }
                const size_t e = (size_t)ci * T + t;
                uint32_t take = bi;
                if (force && force[e] >= 0) take = (uint32_t)force[e];
                if (pick) pick[e] = bi;
                if (g_min) g_min[e] = best;
                if (g_second) g_second[e] = second;
                if (g_scale) g_scale[e] = scale;
                if (g_taken) g_taken[e] = w[take] - t2[take];
                if (g_dot) {
                    /* <g, a> at this step's iterate: with g_min, the
                       Frank-Wolfe duality gap <g, a> - min_c g[c] */
                    double d = 0.0;
                    for (uint32_t c = 0; c < k; ++c) d += a[c] * (w[c] - t2[c]);
                    g_dot[e] = d;
                }

                const double gam = gamma ? gamma[t] : 2.0 / ((double)t + 2.0);
                for (uint32_t c = 0; c < k; ++c) a[c] *= (1.0 - gam);
                a[take] += gam;

                if (prune) {
                    /* drop every non-zero weight with |a| <= threshold, then
                       scale the rest back to unit sum unless the sum is at or
                       below the floor */
                    uint32_t nd = 0;
                    double near = INFINITY;
                    for (uint32_t c = 0; c < k; ++c) {
                        if (a[c] == 0.0) continue;
                        const double d = fabs(fabs(a[c]) - threshold);
                        if (d < near) near = d;
                        if (!(a[c] > threshold || a[c] < -threshold)) {
                            a[c] = 0.0;
                            ++nd;
                        }
                    }
                    double total = 0.0;
                    for (uint32_t c = 0; c < k; ++c) total += a[c];
                    if (total > ORACLE_RENORM_FLOOR) {
                        const double r = 1.0 / total;
                        for (uint32_t c = 0; c < k; ++c) a[c] *= r;
                    }
                    if (drops) drops[e] = nd;
                    if (margin) margin[e] = near;
                }
            }
        }
        free(t2);
        free(w);
    }
    return fail ? ORACLE_E_ALLOC : 0;
}

int oracle_fw_a_columns(uint32_t n, uint32_t k, uint32_t T,
                        const uint32_t *t1_ptr, const uint32_t *t1_idx,
                        const float *t1_val, const uint32_t *k2b_ptr,
                        const uint32_t *k2b_idx, const float *k2b_val,
                        const uint32_t *ap_ptr, const uint32_t *ap_idx,
                        const float *ap_val, const double *gamma,
                        const uint32_t *cells, uint32_t n_cells,
                        const int64_t *force, double *a_out, uint32_t *pick,
                        double *g_min, double *g_second, double *g_scale,
                        double *g_taken, double *g_dot, int n_threads) {
    return fw_a_columns_impl(n, k, T, t1_ptr, t1_idx, t1_val, k2b_ptr, k2b_idx,
                             k2b_val, ap_ptr, ap_idx, ap_val, gamma, cells,
                             n_cells, force, 0, 0.0, a_out, pick, g_min,
                             g_second, g_scale, g_taken, g_dot, NULL, NULL,
                             n_threads);
}

/*
 * A update with pruning and renormalisation (`fw_columns_a_gpu` with
 * `pruning`, its comments on dropping and renormalising, and
 * `A_RENORM_FLOOR`).
 *
 * Each step is the step above, followed by:
 *     every weight with a[c] != 0 and -threshold <= a[c] <= threshold is set
 *     to 0 (dropped; its slot is kept, so a later pick of c starts from 0);
 *     total = sum_c a[c]; if total > 1e-15, a = a / total (as a * (1/total)).
 * The gradient of the next step is recomputed from the new a, which is what
 * the page's incremental correction of w (subtract each dropped atom's t1 row,
 * scale by the renormalisation factor) maintains.
 * Extra trace outputs ([n_cells * T], nullable):
 *   drops  - number of weights dropped at step t
 *   margin - min over the non-zero weights before the drop of
 *            | |a[c]| - threshold | (+inf when there are none): how close the
 *            step's drop decisions were
 */
int oracle_fw_a_columns_pruned(
    uint32_t n, uint32_t k, uint32_t T, const uint32_t *t1_ptr,
    const uint32_t *t1_idx, const float *t1_val, const uint32_t *k2b_ptr,
    const uint32_t *k2b_idx, const float *k2b_val, const uint32_t *ap_ptr,
    const uint32_t *ap_idx, const float *ap_val, const double *gamma,
    const uint32_t *cells, uint32_t n_cells, const int64_t *force,
    double threshold, double *a_out, uint32_t *pick, double *g_min,
    double *g_second, double *g_scale, double *g_taken, double *g_dot,
    uint32_t *drops, double *margin, int n_threads) {
    if (!(threshold >= 0.0)) return ORACLE_E_ARG;
    return fw_a_columns_impl(n, k, T, t1_ptr, t1_idx, t1_val, k2b_ptr, k2b_idx,
                             k2b_val, ap_ptr, ap_idx, ap_val, gamma, cells,
                             n_cells, force, 1, threshold, a_out, pick, g_min,
                             g_second, g_scale, g_taken, g_dot, drops, margin,
                             n_threads);
}

/*
 * B-gradient argmin (`fw_argmin_b` + `reduce_argmin_blocks`).
 *
 * For every row i (ascending), the dense k-vector
 *     G[i, :] = sum_{m in K^2B row i} K^2B[i, m] AAt[m, :] - K^2A^T[i, :]
 * and per column c the running minimum under strict `<`, so the lowest row
 * wins a tie; rows with an empty K^2B row take part like any other.
 * Outputs:
 *   best_val[k], best_row[k]   - min_i G[i, c] and the lowest i attaining it
 *   second_val[k] (nullable)   - the second-smallest G[., c] (equal to the
 *                                minimum on an exact tie; +inf when n == 1)
 *   gap[1] (nullable)          - sum_{i, c} B[i, c] G[i, c]; B may be NULL
 *                                (then 0)
 *   row_scale[n] (nullable)    - max(max_c |(K^2B AAt)[i, c]|,
 *                                    max_c |K^2A^T[i, c]|)
 */
int oracle_fw_b_argmin(uint32_t n, uint32_t k, const uint32_t *k2b_ptr,
                       const uint32_t *k2b_idx, const float *k2b_val,
                       const uint32_t *aat_ptr, const uint32_t *aat_idx,
                       const float *aat_val, const uint32_t *k2at_ptr,
                       const uint32_t *k2at_idx, const float *k2at_val,
                       const uint32_t *b_ptr, const uint32_t *b_idx,
                       const float *b_val, double *best_val,
                       uint32_t *best_row, double *second_val, double *gap,
                       double *row_scale, int n_threads) {
    if (n == 0 || k == 0 || !k2b_val || !aat_val || !k2at_val || !best_val ||
        !best_row)
        return ORACLE_E_ARG;
    int rc;
    if ((rc = check_csr(n, k, k2b_ptr, k2b_idx))) return rc;
    if ((rc = check_csr(k, k, aat_ptr, aat_idx))) return rc;
    if ((rc = check_csr(n, k, k2at_ptr, k2at_idx))) return rc;
    if (b_ptr && (rc = check_csr(n, k, b_ptr, b_idx))) return rc;

    const uint32_t chunks = n < ORACLE_B_CHUNKS ? n : ORACLE_B_CHUNKS;
    double *cb = (double *)malloc(sizeof(double) * (size_t)chunks * k);
    double *cs = (double *)malloc(sizeof(double) * (size_t)chunks * k);
    uint32_t *cr = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)chunks * k);
    double *cg = (double *)calloc(chunks, sizeof(double));
    if (!cb || !cs || !cr || !cg) {
        free(cb), free(cs), free(cr), free(cg);
        return ORACLE_E_ALLOC;
    }
    int fail = 0;
    const int nt = oracle_threads(n_threads);
#pragma omp parallel num_threads(nt)
    {
        double *acc = (double *)malloc(sizeof(double) * k);
        if (!acc) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ch = 0; ch < (int64_t)chunks; ++ch) {
            if (!acc) continue;
            double *best = cb + (size_t)ch * k, *second = cs + (size_t)ch * k;
            uint32_t *row = cr + (size_t)ch * k;
            for (uint32_t c = 0; c < k; ++c)
                best[c] = INFINITY, second[c] = INFINITY, row[c] = 0;
            const uint32_t lo = (uint32_t)(((uint64_t)n * ch) / chunks);
            const uint32_t hi = (uint32_t)(((uint64_t)n * (ch + 1)) / chunks);
            double g_sum = 0.0;
            for (uint32_t i = lo; i < hi; ++i) {
                for (uint32_t c = 0; c < k; ++c) acc[c] = 0.0;
                for (uint32_t p = k2b_ptr[i]; p < k2b_ptr[i + 1]; ++p) {
                    const uint32_t m = k2b_idx[p];
                    const double x = (double)k2b_val[p];
                    for (uint32_t q = aat_ptr[m]; q < aat_ptr[m + 1]; ++q)
                        acc[aat_idx[q]] += x * (double)aat_val[q];
                }
                double scale = 0.0;
                for (uint32_t c = 0; c < k; ++c)
                    if (fabs(acc[c]) > scale) scale = fabs(acc[c]);
                for (uint32_t p = k2at_ptr[i]; p < k2at_ptr[i + 1]; ++p) {
                    const double v = (double)k2at_val[p];
                    acc[k2at_idx[p]] -= v;
                    if (fabs(v) > scale) scale = fabs(v);
                }
                if (row_scale) row_scale[i] = scale;
                if (b_ptr)
                    for (uint32_t p = b_ptr[i]; p < b_ptr[i + 1]; ++p)
                        g_sum += (double)b_val[p] * acc[b_idx[p]];
                for (uint32_t c = 0; c < k; ++c) {
                    if (acc[c] < best[c]) {
                        second[c] = best[c];
                        best[c] = acc[c];
                        row[c] = i;
                    } else if (acc[c] < second[c]) {
                        second[c] = acc[c];
                    }
                }
            }
            cg[ch] = g_sum;
        }
        free(acc);
    }
    if (!fail) {
        /* Merge the chunks in row order: a later chunk only wins on a
         * strictly smaller value, which keeps the lowest row on a tie. */
        for (uint32_t c = 0; c < k; ++c) {
            double best = INFINITY, second = INFINITY;
            uint32_t row = 0;
            for (uint32_t ch = 0; ch < chunks; ++ch) {
                const double b = cb[(size_t)ch * k + c];
                const double s = cs[(size_t)ch * k + c];
                if (b < best) {
                    second = best < s ? best : s;
                    best = b;
                    row = cr[(size_t)ch * k + c];
                } else {
                    if (b < second) second = b;
                }
            }
            best_val[c] = best;
            best_row[c] = row;
            if (second_val) second_val[c] = second;
        }
        if (gap) {
            double g = 0.0;
            for (uint32_t ch = 0; ch < chunks; ++ch) g += cg[ch];
            *gap = b_ptr ? g : 0.0;
        }
    }
    free(cb), free(cs), free(cr), free(cg);
    return fail ? ORACLE_E_ALLOC : 0;
}

/*
 * Single entries of the B gradient, G[rows[e], cols[e]] for e < m, each
 * evaluated from its definition (used to judge an argmin that differs from
 * the oracle's). out_scale (nullable) receives the same term scale as
 * row_scale above, for the row of each entry.
 */
int oracle_fw_b_grad_at(uint32_t n, uint32_t k, const uint32_t *k2b_ptr,
                        const uint32_t *k2b_idx, const float *k2b_val,
                        const uint32_t *aat_ptr, const uint32_t *aat_idx,
                        const float *aat_val, const uint32_t *k2at_ptr,
                        const uint32_t *k2at_idx, const float *k2at_val,
                        const uint32_t *rows, const uint32_t *cols, uint32_t m,
                        double *out, double *out_scale) {
    if (!rows || !cols || !out) return ORACLE_E_ARG;
    double *acc = (double *)malloc(sizeof(double) * k);
    if (!acc) return ORACLE_E_ALLOC;
    for (uint32_t e = 0; e < m; ++e) {
        const uint32_t i = rows[e], c = cols[e];
        if (i >= n || c >= k) {
            free(acc);
            return ORACLE_E_INDEX;
        }
        for (uint32_t cc = 0; cc < k; ++cc) acc[cc] = 0.0;
        for (uint32_t p = k2b_ptr[i]; p < k2b_ptr[i + 1]; ++p) {
            const uint32_t mm = k2b_idx[p];
            const double x = (double)k2b_val[p];
            for (uint32_t q = aat_ptr[mm]; q < aat_ptr[mm + 1]; ++q)
                acc[aat_idx[q]] += x * (double)aat_val[q];
        }
        double scale = 0.0;
        for (uint32_t cc = 0; cc < k; ++cc)
            if (fabs(acc[cc]) > scale) scale = fabs(acc[cc]);
        double t2 = 0.0;
        for (uint32_t p = k2at_ptr[i]; p < k2at_ptr[i + 1]; ++p) {
            if (fabs((double)k2at_val[p]) > scale)
                scale = fabs((double)k2at_val[p]);
            if (k2at_idx[p] == c) t2 = (double)k2at_val[p];
        }
        out[e] = acc[c] - t2;
        if (out_scale) out_scale[e] = scale;
    }
    free(acc);
    return 0;
}

/*
 * B step: B_c <- (1 - gamma) B_c + gamma e_{arg_idx[c]} for every column c.
 * B^T is held as padded rows: row c has bt_cnt[c] entries at
 * bt_idx[c * cap_b + s], bt_val[c * cap_b + s], cell indices ascending.
 * A cell not yet in the row is inserted at its sorted position; a full row
 * makes the call fail with ORACLE_E_CAP (nothing of that row is changed).
 */
int oracle_fw_b_apply(uint32_t k, uint32_t cap_b, uint32_t *bt_idx,
                      double *bt_val, uint32_t *bt_cnt,
                      const uint32_t *arg_idx, double gamma) {
    if (!bt_idx || !bt_val || !bt_cnt || !arg_idx || cap_b == 0)
        return ORACLE_E_ARG;
    int rc = 0;
    for (uint32_t c = 0; c < k; ++c) {
        uint32_t *idx = bt_idx + (size_t)c * cap_b;
        double *val = bt_val + (size_t)c * cap_b;
        const uint32_t cnt = bt_cnt[c], i = arg_idx[c];
        if (cnt > cap_b) return ORACLE_E_ARG;
        uint32_t pos = 0;
        while (pos < cnt && idx[pos] < i) ++pos;
        const int present = pos < cnt && idx[pos] == i;
        if (!present && cnt == cap_b) {
            rc = ORACLE_E_CAP;
            continue;
        }
        for (uint32_t s = 0; s < cnt; ++s) val[s] *= (1.0 - gamma);
        if (present) {
            val[pos] += gamma;
        } else {
            for (uint32_t s = cnt; s > pos; --s) {
                idx[s] = idx[s - 1];
                val[s] = val[s - 1];
            }
            idx[pos] = i;
            val[pos] = gamma;
            bt_cnt[c] = cnt + 1;
        }
    }
    return rc;
}
