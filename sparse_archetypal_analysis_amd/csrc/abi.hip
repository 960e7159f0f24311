// Exported C ABI (include/seacells_fw.h, include/seacells_sparse.h,
// include/seacells_debug.h): host-side validation, workspace
// sizing and dispatch onto the caller's stream. Argument checks run before
// any HIP call, so they also work on a machine without a GPU.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "seacells_debug.h"
#include "seacells_fw.h"
#include "seacells_sparse.h"
#include "common.hpp"

namespace seacells {

static thread_local char g_last_error[256] = "";

static int hip_fail(hipError_t e, const char *what) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", what, hipGetErrorString(e));
  return SEACELLS_E_HIP;
}

hipError_t device_info(DeviceInfo *out) {
  static DeviceInfo cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!cache[dev].ok) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cache[dev].cus = cus > 0 ? cus : 1;
    cache[dev].ok = 1;
  }
  *out = cache[dev];
  return hipSuccess;
}

// Per-call stamp for the B partials. Starts away from 0 so zero-filled or
// leftover workspace never matches, and never takes the value 0.
static thread_local uint32_t g_last_epoch = 0;

static uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0x5EAC0001u};
  uint32_t e;
  do {
    e = counter.fetch_add(1u, std::memory_order_relaxed);
  } while (e == 0u);
  g_last_epoch = e;
  return e;
}

static int check_csr(const seacells_csr *m, uint32_t rows, uint32_t cols) {
  if (m == nullptr || m->row_ptr == nullptr) return SEACELLS_E_NULL;
  if (m->nnz > 0 && (m->col_idx == nullptr || m->val == nullptr)) return SEACELLS_E_NULL;
  if (m->n_rows != rows || m->n_cols != cols) return SEACELLS_E_SHAPE;
  if (m->nnz >= 0x80000000u) return SEACELLS_E_TOO_LARGE;
  return SEACELLS_OK;
}

static Csr as_csr(const seacells_csr *m) {
  Csr c;
  c.ptr = m->row_ptr;
  c.idx = m->col_idx;
  c.val = m->val;
  c.nnz = m->nnz;
  return c;
}

}  // namespace seacells

using namespace seacells;

extern "C" {

size_t seacells_fw_a_columns_workspace(uint32_t n, uint32_t k, uint32_t T, uint32_t cap,
                                       uint32_t t1_nnz) {
  if (n == 0 || k == 0 || cap == 0) return 0;
  // one size covers the plain and the pruning entry point
  const size_t plain = plan_a(n, k, T, cap, false, t1_nnz).ws_bytes;
  const size_t pruned = plan_a(n, k, T, cap, true, t1_nnz).ws_bytes;
  return plain > pruned ? plain : pruned;
}

static int a_columns(const seacells_csr *t1, const seacells_csr *k2b,
                     const seacells_csr *a_prev_t, uint32_t n, uint32_t k, uint32_t T,
                     uint32_t cap, const float *gamma, bool prune, float threshold,
                     uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt, uint32_t *trace,
                     float *fw_gap, void *workspace, size_t workspace_bytes, uint32_t *status,
                     seacells_stream_t stream) {
  if (t1 == nullptr || k2b == nullptr || a_prev_t == nullptr || atom_idx == nullptr ||
      atom_val == nullptr || atom_cnt == nullptr || status == nullptr)
    return SEACELLS_E_NULL;
  if (n == 0 || k == 0 || T == 0 || cap == 0) return SEACELLS_E_SHAPE;
  if (prune && !(threshold >= 0.0f && threshold <= 3.4e38f)) return SEACELLS_E_SHAPE;
  if (n >= 0x80000000u || k >= 0x40000000u) return SEACELLS_E_TOO_LARGE;
  int rc;
  if ((rc = check_csr(t1, k, k)) != SEACELLS_OK) return rc;
  if ((rc = check_csr(k2b, n, k)) != SEACELLS_OK) return rc;
  if ((rc = check_csr(a_prev_t, n, k)) != SEACELLS_OK) return rc;
  if ((uint64_t)n * cap >= (1ull << 40) || (uint64_t)n * T >= (1ull << 40))
    return SEACELLS_E_TOO_LARGE;
  if (cap >= 0x10000000u) return SEACELLS_E_TOO_LARGE;
  const APlan plan = plan_a(n, k, T, cap, prune, t1->nnz);
  // per-wave LDS must at least hold the atom list
  if (plan.waves_per_block == 0) return SEACELLS_E_TOO_LARGE;
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes))
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_fw_a(plan, as_csr(t1), as_csr(k2b), as_csr(a_prev_t), n, k, T, cap, gamma,
                  threshold, atom_idx, atom_val, atom_cnt, trace, fw_gap, workspace, status, s);
  if (e != hipSuccess) return hip_fail(e, "fw_a_columns launch");
  return SEACELLS_OK;
}

int seacells_fw_a_columns(const seacells_csr *t1, const seacells_csr *k2b,
                          const seacells_csr *a_prev_t, uint32_t n, uint32_t k, uint32_t T,
                          uint32_t cap, const float *gamma, uint32_t *atom_idx, float *atom_val,
                          uint32_t *atom_cnt, uint32_t *trace, float *fw_gap, void *workspace,
                          size_t workspace_bytes, uint32_t *status, seacells_stream_t stream) {
  return a_columns(t1, k2b, a_prev_t, n, k, T, cap, gamma, false, 0.0f, atom_idx, atom_val,
                   atom_cnt, trace, fw_gap, workspace, workspace_bytes, status, stream);
}

int seacells_fw_a_columns_pruned(const seacells_csr *t1, const seacells_csr *k2b,
                                 const seacells_csr *a_prev_t, uint32_t n, uint32_t k,
                                 uint32_t T, uint32_t cap, const float *gamma, float threshold,
                                 uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                                 uint32_t *trace, float *fw_gap, void *workspace,
                                 size_t workspace_bytes, uint32_t *status,
                                 seacells_stream_t stream) {
  return a_columns(t1, k2b, a_prev_t, n, k, T, cap, gamma, true, threshold, atom_idx, atom_val,
                   atom_cnt, trace, fw_gap, workspace, workspace_bytes, status, stream);
}

// --- the A update without allocation ---------------------------------------

}  // extern "C"

namespace seacells {

// The workspace of seacells_fw_a_columns_noalloc: one array per device (the
// code object is loaded on each device the library runs on). In host code
// `scratch` is a host-side stand-in, not a device address; the address comes
// from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[SEACELLS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static void *g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mutex;

static hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace seacells

extern "C" {

int seacells_fw_a_columns_noalloc(const seacells_csr *t1, const seacells_csr *k2b,
                                  const seacells_csr *a_prev_t, uint32_t n, uint32_t k,
                                  uint32_t T, uint32_t cap, const float *gamma,
                                  uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                                  uint32_t *trace, float *fw_gap, uint32_t *status,
                                  seacells_stream_t stream) {
  // the sizes are checked on the host before anything else (the argument
  // checks of a_columns repeat them, and run before any device work)
  if (t1 == nullptr || k2b == nullptr || a_prev_t == nullptr || atom_idx == nullptr ||
      atom_val == nullptr || atom_cnt == nullptr || status == nullptr)
    return SEACELLS_E_NULL;
  if (n == 0 || k == 0 || T == 0 || cap == 0) return SEACELLS_E_SHAPE;
  if (n >= 0x80000000u || k >= 0x40000000u || cap >= 0x10000000u) return SEACELLS_E_TOO_LARGE;
  const size_t need = seacells_fw_a_columns_workspace(n, k, T, cap, t1->nnz);
  if (need > SEACELLS_NOALLOC_SCRATCH_BYTES) return SEACELLS_E_TOO_LARGE;
  void *ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
  }
  return a_columns(t1, k2b, a_prev_t, n, k, T, cap, gamma, false, 0.0f, atom_idx, atom_val,
                   atom_cnt, trace, fw_gap, ws, need > 0 ? (size_t)SEACELLS_NOALLOC_SCRATCH_BYTES : 0,
                   status, stream);
}

size_t seacells_fw_b_argmin_workspace(uint32_t n, uint32_t k, uint32_t aat_nnz) {
  if (n == 0 || k == 0) return 0;
  return plan_b(n, k, aat_nnz).ws_bytes;
}

int seacells_fw_b_argmin(const seacells_csr *k2b, const seacells_csr *aat,
                         const seacells_csr *k2at, const seacells_csr *b, uint32_t n, uint32_t k,
                         float *out_val, uint32_t *out_idx, float *gap, float *fw_gap,
                         void *workspace, size_t workspace_bytes, uint32_t *status,
                         seacells_stream_t stream) {
  if (k2b == nullptr || aat == nullptr || k2at == nullptr || out_val == nullptr ||
      out_idx == nullptr || status == nullptr)
    return SEACELLS_E_NULL;
  if (fw_gap != nullptr && b == nullptr) return SEACELLS_E_NULL;  // the gap needs B
  if (n == 0 || k == 0) return SEACELLS_E_SHAPE;
  if (n >= 0x80000000u || k >= 0x80000000u) return SEACELLS_E_TOO_LARGE;
  int rc;
  if ((rc = check_csr(k2b, n, k)) != SEACELLS_OK) return rc;
  if ((rc = check_csr(aat, k, k)) != SEACELLS_OK) return rc;
  if ((rc = check_csr(k2at, n, k)) != SEACELLS_OK) return rc;
  if (b != nullptr && (rc = check_csr(b, n, k)) != SEACELLS_OK) return rc;
  const BPlan plan = plan_b(n, k, aat->nnz);
  if (plan.pa_chunks >= (1ull << 32)) return SEACELLS_E_TOO_LARGE;
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return SEACELLS_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SEACELLS_E_WORKSPACE;
  Csr bc{};
  if (b != nullptr) bc = as_csr(b);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_fw_b(plan, as_csr(k2b), as_csr(aat), as_csr(k2at), bc, n, k, out_val, out_idx, gap,
                  fw_gap, workspace, status, next_epoch(), s);
  if (e != hipSuccess) return hip_fail(e, "fw_b_argmin launch");
  return SEACELLS_OK;
}

int seacells_fw_b_apply(uint32_t *bt_idx, float *bt_val, uint32_t *bt_cnt, uint32_t n,
                        uint32_t k, uint32_t cap_b, const uint32_t *arg_idx, float gamma,
                        uint32_t *status, seacells_stream_t stream) {
  if (bt_idx == nullptr || bt_val == nullptr || bt_cnt == nullptr || arg_idx == nullptr ||
      status == nullptr)
    return SEACELLS_E_NULL;
  if (n == 0 || k == 0 || cap_b == 0) return SEACELLS_E_SHAPE;
  if (!(gamma > 0.0f && gamma <= 1.0f)) return SEACELLS_E_SHAPE;
  if ((uint64_t)k * cap_b >= (1ull << 40)) return SEACELLS_E_TOO_LARGE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_fw_b_apply(bt_idx, bt_val, bt_cnt, n, k, cap_b, arg_idx, gamma, status, s);
  if (e != hipSuccess) return hip_fail(e, "fw_b_apply launch");
  return SEACELLS_OK;
}

// --- sparse operations (seacells_sparse.h) ---------------------------------

static int check_any_csr(const seacells_csr *m) {
  if (m == nullptr || m->row_ptr == nullptr) return SEACELLS_E_NULL;
  if (m->nnz > 0 && (m->col_idx == nullptr || m->val == nullptr)) return SEACELLS_E_NULL;
  if (m->nnz >= 0x80000000u || m->n_rows >= 0x80000000u || m->n_cols >= 0x80000000u)
    return SEACELLS_E_TOO_LARGE;
  return SEACELLS_OK;
}

size_t seacells_csr_matmul_workspace(uint32_t m) { return matmul_workspace(m); }

size_t seacells_csr_matmul_pattern_workspace(uint32_t m, uint32_t q) {
  const size_t p = matmul_pattern_bytes(m, q);
  return p == 0 ? 0 : matmul_workspace(m) + p;
}

// The rows pass's bitmaps, when the workspace holds them.
static uint32_t *matmul_pattern(void *ws, size_t bytes, uint32_t m, uint32_t q) {
  const size_t p = matmul_pattern_bytes(m, q);
  if (ws == nullptr || p == 0 || bytes < matmul_workspace(m) + p) return nullptr;
  return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + matmul_workspace(m));
}

int seacells_csr_matmul_rows(const seacells_csr *a, const seacells_csr *b, uint32_t *c_row_ptr,
                             void *workspace, size_t workspace_bytes, uint32_t *status,
                             seacells_stream_t stream) {
  int rc;
  if ((rc = check_any_csr(a)) != SEACELLS_OK || (rc = check_any_csr(b)) != SEACELLS_OK) return rc;
  if (c_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (a->n_cols != b->n_rows) return SEACELLS_E_SHAPE;
  if (workspace == nullptr || workspace_bytes < matmul_workspace(a->n_rows) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_spgemm_count(as_csr(a), as_csr(b), a->n_rows, a->n_cols, b->n_cols, c_row_ptr,
                          workspace,
                          matmul_pattern(workspace, workspace_bytes, a->n_rows, b->n_cols), status,
                          s);
  if (e != hipSuccess) return hip_fail(e, "csr_matmul_rows launch");
  return SEACELLS_OK;
}

int seacells_csr_matmul_fill(const seacells_csr *a, const seacells_csr *b,
                             const uint32_t *c_row_ptr, uint32_t *c_col_idx, float *c_val,
                             size_t c_capacity, void *workspace, size_t workspace_bytes,
                             uint32_t *status, seacells_stream_t stream) {
  int rc;
  if ((rc = check_any_csr(a)) != SEACELLS_OK || (rc = check_any_csr(b)) != SEACELLS_OK) return rc;
  if (c_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (a->n_cols != b->n_rows) return SEACELLS_E_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  // (empty outputs may pass NULL arrays: nothing is written then)
  e = launch_spgemm_fill(as_csr(a), as_csr(b), a->n_rows, a->n_cols, b->n_cols, c_row_ptr,
                         c_col_idx, c_val, (uint64_t)c_capacity,
                         matmul_pattern(workspace, workspace_bytes, a->n_rows, b->n_cols), status,
                         s);
  if (e != hipSuccess) return hip_fail(e, "csr_matmul_fill launch");
  return SEACELLS_OK;
}

size_t seacells_csr_transpose_workspace(uint32_t m, uint32_t q) {
  const size_t b = transpose_workspace(m, q);
  return b > 0 ? b : 256;
}

int seacells_csr_transpose(const seacells_csr *a, uint32_t *at_row_ptr, uint32_t *at_col_idx,
                           float *at_val, void *workspace, size_t workspace_bytes,
                           uint32_t *status, seacells_stream_t stream) {
  int rc;
  if ((rc = check_any_csr(a)) != SEACELLS_OK) return rc;
  if (at_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (a->nnz > 0 && (at_col_idx == nullptr || at_val == nullptr)) return SEACELLS_E_NULL;
  if (workspace == nullptr ||
      workspace_bytes < seacells_csr_transpose_workspace(a->n_rows, a->n_cols) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_transpose(as_csr(a), a->n_rows, a->n_cols, at_row_ptr, at_col_idx, at_val,
                       workspace, status, s);
  if (e != hipSuccess) return hip_fail(e, "csr_transpose launch");
  return SEACELLS_OK;
}

size_t seacells_csr_dot_workspace(void) { return align_up(dot_workspace(), 256); }

int seacells_csr_dot(const seacells_csr *x, const seacells_csr *y, double alpha, double *acc,
                     void *workspace, size_t workspace_bytes, uint32_t *status,
                     seacells_stream_t stream) {
  int rc;
  if ((rc = check_any_csr(x)) != SEACELLS_OK || (rc = check_any_csr(y)) != SEACELLS_OK) return rc;
  if (acc == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (x->n_rows != y->n_rows || x->n_cols != y->n_cols) return SEACELLS_E_SHAPE;
  if (workspace == nullptr || workspace_bytes < seacells_csr_dot_workspace() ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_dot(as_csr(x), as_csr(y), x->n_rows, alpha, acc, workspace, status, s);
  if (e != hipSuccess) return hip_fail(e, "csr_dot launch");
  return SEACELLS_OK;
}

size_t seacells_csr_add_workspace(uint32_t m) { return add_workspace(m); }

int seacells_csr_add_rows(const seacells_csr *x, const seacells_csr *y, uint32_t *c_row_ptr,
                          void *workspace, size_t workspace_bytes, uint32_t *status,
                          seacells_stream_t stream) {
  int rc;
  if ((rc = check_any_csr(x)) != SEACELLS_OK || (rc = check_any_csr(y)) != SEACELLS_OK) return rc;
  if (c_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (x->n_rows != y->n_rows || x->n_cols != y->n_cols) return SEACELLS_E_SHAPE;
  if ((uint64_t)x->nnz + y->nnz >= 0x80000000ull) return SEACELLS_E_TOO_LARGE;
  if (workspace == nullptr || workspace_bytes < add_workspace(x->n_rows) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_add_count(as_csr(x), as_csr(y), x->n_rows, x->n_cols, c_row_ptr, workspace, status, s);
  if (e != hipSuccess) return hip_fail(e, "csr_add_rows launch");
  return SEACELLS_OK;
}

int seacells_csr_add_fill(float alpha, const seacells_csr *x, float beta, const seacells_csr *y,
                          const uint32_t *c_row_ptr, uint32_t *c_col_idx, float *c_val,
                          size_t c_capacity, uint32_t *status, seacells_stream_t stream) {
  int rc;
  if ((rc = check_any_csr(x)) != SEACELLS_OK || (rc = check_any_csr(y)) != SEACELLS_OK) return rc;
  if (c_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if ((x->nnz > 0 || y->nnz > 0) && (c_col_idx == nullptr || c_val == nullptr))
    return SEACELLS_E_NULL;
  if (x->n_rows != y->n_rows || x->n_cols != y->n_cols) return SEACELLS_E_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_add_fill(alpha, as_csr(x), beta, as_csr(y), x->n_rows, c_row_ptr, c_col_idx, c_val,
                      (uint64_t)c_capacity, status, s);
  if (e != hipSuccess) return hip_fail(e, "csr_add_fill launch");
  return SEACELLS_OK;
}

size_t seacells_fw_b_vertex_workspace(uint32_t k, uint32_t n) { return vertex_workspace(k, n); }

int seacells_fw_b_vertex(const uint32_t *arg_idx, uint32_t k, uint32_t n, float value,
                         uint32_t *s_row_ptr, uint32_t *s_col_idx, float *s_val, void *workspace,
                         size_t workspace_bytes, uint32_t *status, seacells_stream_t stream) {
  if (s_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (k > 0 && (arg_idx == nullptr || s_col_idx == nullptr || s_val == nullptr))
    return SEACELLS_E_NULL;
  if (n == 0) return SEACELLS_E_SHAPE;
  if (k >= 0x80000000u || n >= 0x80000000u) return SEACELLS_E_TOO_LARGE;
  if (workspace == nullptr || workspace_bytes < vertex_workspace(k, n) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_vertex(arg_idx, k, n, value, s_row_ptr, s_col_idx, s_val, workspace, status, s);
  if (e != hipSuccess) return hip_fail(e, "fw_b_vertex launch");
  return SEACELLS_OK;
}

size_t seacells_fw_a_to_csr_workspace(uint32_t n) { return add_workspace(n); }

static int check_atoms(const uint32_t *atom_idx, const float *atom_val, const uint32_t *atom_cnt,
                       uint32_t n, uint32_t k, uint32_t cap) {
  if (n > 0 && (atom_idx == nullptr || atom_val == nullptr || atom_cnt == nullptr))
    return SEACELLS_E_NULL;
  if (k == 0 || cap == 0) return SEACELLS_E_SHAPE;
  if (n >= 0x80000000u || k >= 0x80000000u) return SEACELLS_E_TOO_LARGE;
  return SEACELLS_OK;
}

int seacells_fw_a_to_csr_rows(const uint32_t *atom_idx, const float *atom_val,
                              const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                              uint32_t *at_row_ptr, void *workspace, size_t workspace_bytes,
                              uint32_t *status, seacells_stream_t stream) {
  int rc;
  if ((rc = check_atoms(atom_idx, atom_val, atom_cnt, n, k, cap)) != SEACELLS_OK) return rc;
  if (at_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (workspace == nullptr || workspace_bytes < add_workspace(n) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_atoms_count(atom_idx, atom_val, atom_cnt, n, k, cap, at_row_ptr, workspace, status, s);
  if (e != hipSuccess) return hip_fail(e, "fw_a_to_csr_rows launch");
  return SEACELLS_OK;
}

int seacells_fw_a_to_csr_fill(const uint32_t *atom_idx, const float *atom_val,
                              const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                              const uint32_t *at_row_ptr, uint32_t *at_col_idx, float *at_val,
                              uint32_t *status, seacells_stream_t stream) {
  int rc;
  if ((rc = check_atoms(atom_idx, atom_val, atom_cnt, n, k, cap)) != SEACELLS_OK) return rc;
  if (at_row_ptr == nullptr || status == nullptr) return SEACELLS_E_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_atoms_fill(atom_idx, atom_val, atom_cnt, n, k, cap, at_row_ptr, at_col_idx, at_val,
                        status, s);
  if (e != hipSuccess) return hip_fail(e, "fw_a_to_csr_fill launch");
  return SEACELLS_OK;
}

// --- test and experiment hooks (seacells_debug.h) -------------------------

int seacells_debug_set_a_options(const seacells_a_options *opt) {
  AOptions o;
  if (opt != nullptr) {
    if (opt->support < -1 || opt->support > 1) return SEACELLS_E_SHAPE;
    if (opt->support_waves != 0 && (opt->support_waves < 4 || opt->support_waves > 32))
      return SEACELLS_E_SHAPE;
    if (opt->dense_argmin < 0 || opt->dense_argmin > 1) return SEACELLS_E_SHAPE;
    if (opt->group != 0 && opt->group != 16 && opt->group != 32 && opt->group != 64)
      return SEACELLS_E_SHAPE;
    if (opt->support_wide < -1 || opt->support_wide > 1) return SEACELLS_E_SHAPE;
    o.support = opt->support;
    o.support_waves = opt->support_waves;
    o.dense_argmin = opt->dense_argmin == 1;
    o.group = opt->group;
    o.support_wide = opt->support_wide;
  }
  a_options() = o;
  return SEACELLS_OK;
}

int seacells_debug_b_layout(uint32_t n, uint32_t k, uint32_t aat_nnz, seacells_b_layout *out) {
  if (out == nullptr) return SEACELLS_E_NULL;
  if (n == 0 || k == 0) return SEACELLS_E_SHAPE;
  if (n >= 0x80000000u || k >= 0x80000000u) return SEACELLS_E_TOO_LARGE;
  const BPlan p = plan_b(n, k, aat_nnz);
  out->keys_offset = p.off_keys;
  out->stamps_offset = p.off_stamp;
  out->n_row_blocks = p.n_row_blocks;
  out->n_slices = p.n_slices;
  out->slice_w = p.slice_w;
  out->reserved = 0;
  return SEACELLS_OK;
}

uint32_t seacells_debug_b_last_epoch(void) { return g_last_epoch; }

int seacells_debug_b_reduce(uint32_t n, uint32_t k, uint32_t aat_nnz, uint32_t epoch,
                            float *out_val, uint32_t *out_idx, float *gap, void *workspace,
                            size_t workspace_bytes, uint32_t *status, seacells_stream_t stream) {
  if (out_val == nullptr || out_idx == nullptr || status == nullptr) return SEACELLS_E_NULL;
  if (n == 0 || k == 0) return SEACELLS_E_SHAPE;
  if (n >= 0x80000000u || k >= 0x80000000u) return SEACELLS_E_TOO_LARGE;
  const BPlan plan = plan_b(n, k, aat_nnz);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return SEACELLS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_status_clear(status, s);
  if (e != hipSuccess) return hip_fail(e, "status clear");
  e = launch_fw_b_reduce(plan, n, k, out_val, out_idx, gap, nullptr, workspace, status, epoch, s);
  if (e != hipSuccess) return hip_fail(e, "fw_b reduce launch");
  return SEACELLS_OK;
}

const char *seacells_status_string(int code) {
  switch (code) {
    case SEACELLS_OK:
      return "ok";
    case SEACELLS_E_NULL:
      return "a required pointer is NULL";
    case SEACELLS_E_SHAPE:
      return "a size is 0, an argument is out of range, or operand shapes disagree";
    case SEACELLS_E_WORKSPACE:
      return "workspace missing, misaligned or smaller than required";
    case SEACELLS_E_TOO_LARGE:
      return "an operand exceeds the 32-bit index range";
    case SEACELLS_E_HIP:
      return "a HIP launch or query failed";
    default:
      return "unknown status";
  }
}

const char *seacells_last_error(void) { return g_last_error; }

int seacells_fw_step_size(uint32_t t, float *gamma, float *keep) {
  const float g = 2.0f / (float)(t + 2u);
  if (gamma != nullptr) *gamma = g;
  if (keep != nullptr) *keep = 1.0f - g;
  return SEACELLS_OK;
}

int seacells_version(void) { return (1 << 16) | 0; }

}  // extern "C"
