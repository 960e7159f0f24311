/*
 * Sparse product C = A * B of two CSR matrices in f64, for building the
 * kernel-matrix operands of the synthetic workloads (K (K X)). Input
 * generation only: nothing here is part of the Frank-Wolfe path.
 *
 * Each output row is accumulated in a dense f64 row: for every entry (j, v)
 * of A's row, in stored order, and every entry (c, w) of B's row j, in
 * stored order, sum[c] += v * w (a multiply, then an add). That is the
 * order scipy's CSR product sums in, so the values are the same bit for
 * bit; like it, exact zeros are dropped. Output columns are ascending.
 * Rows are independent and split over OpenMP threads.
 *
 * Built with plain -O2 (no -ffast-math, no FMA contraction).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int cmp_i32(const void *a, const void *b) {
  const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* Pass 1: the number of stored entries of each output row (before zeros
 * are dropped) into cnt[0 .. n_rows). Returns 0, or -1 on allocation
 * failure. */
int spgemm_count(int64_t n_rows, int64_t n_cols, const int64_t *a_ptr, const int32_t *a_idx,
                 const int64_t *b_ptr, const int32_t *b_idx, int64_t *cnt) {
  int fail = 0;
#pragma omp parallel
  {
    int64_t *mark = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_cols > 0 ? n_cols : 1));
    if (mark == NULL) {
#pragma omp atomic write
      fail = 1;
    } else {
      for (int64_t c = 0; c < n_cols; ++c) mark[c] = -1;
#pragma omp for schedule(dynamic, 256)
      for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = 0;
        for (int64_t p = a_ptr[i]; p < a_ptr[i + 1]; ++p) {
          const int32_t j = a_idx[p];
          for (int64_t q = b_ptr[j]; q < b_ptr[j + 1]; ++q) {
            const int32_t c = b_idx[q];
            if (mark[c] != i) {
              mark[c] = i;
              ++m;
            }
          }
        }
        cnt[i] = m;
      }
      free(mark);
    }
  }
  return fail ? -1 : 0;
}

/* Pass 2: row i of C goes to [c_ptr[i], c_ptr[i] + cnt_out[i]) of c_idx /
 * c_val, where c_ptr[i] is the prefix sum of pass 1's counts; cnt_out[i]
 * receives the number of non-zero entries written (<= pass 1's count). */
int spgemm_fill(int64_t n_rows, int64_t n_cols, const int64_t *a_ptr, const int32_t *a_idx,
                const double *a_val, const int64_t *b_ptr, const int32_t *b_idx,
                const double *b_val, const int64_t *c_ptr, int32_t *c_idx, double *c_val,
                int64_t *cnt_out) {
  int fail = 0;
#pragma omp parallel
  {
    double *sum = (double *)malloc(sizeof(double) * (size_t)(n_cols > 0 ? n_cols : 1));
    int64_t *mark = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_cols > 0 ? n_cols : 1));
    if (sum == NULL || mark == NULL) {
#pragma omp atomic write
      fail = 1;
    } else {
      for (int64_t c = 0; c < n_cols; ++c) sum[c] = 0.0, mark[c] = -1;
#pragma omp for schedule(dynamic, 256)
      for (int64_t i = 0; i < n_rows; ++i) {
        int32_t *cols = c_idx + c_ptr[i];
        int64_t m = 0;
        for (int64_t p = a_ptr[i]; p < a_ptr[i + 1]; ++p) {
          const int32_t j = a_idx[p];
          const double v = a_val[p];
          for (int64_t q = b_ptr[j]; q < b_ptr[j + 1]; ++q) {
            const int32_t c = b_idx[q];
            const double prod = v * b_val[q];
            sum[c] = sum[c] + prod;
            if (mark[c] != i) {
              mark[c] = i;
              cols[m++] = c;
            }
          }
        }
        qsort(cols, (size_t)m, sizeof(int32_t), cmp_i32);
        int64_t w = 0;
        for (int64_t e = 0; e < m; ++e) {
          const int32_t c = cols[e];
          const double s = sum[c];
          sum[c] = 0.0;
          if (s != 0.0) {
            cols[w] = c;
            c_val[c_ptr[i] + w] = s;
            ++w;
          }
        }
        cnt_out[i] = w;
      }
    }
    free(sum);
    free(mark);
  }
  return fail ? -1 : 0;
}
