// Shared device helpers and internal host interface of the SEACells FW
// library (gfx950, wave64). Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace seacells {

constexpr uint32_t kWave = 64;
constexpr uint32_t kLdsBytesPerCU = 160u * 1024u;  // gfx950 local data share

// Device-side flags, same values as SEACELLS_FLAG_* in the public header.
constexpr uint32_t kFlagCapOverflow = 0x1u;
constexpr uint32_t kFlagPartialsInvalid = 0x2u;
constexpr uint32_t kFlagBCapOverflow = 0x4u;
constexpr uint32_t kFlagBadIndex = 0x8u;
constexpr uint32_t kFlagNonfinite = 0x10u;
constexpr uint32_t kFlagBadGamma = 0x20u;
constexpr uint32_t kFlagOutputTooLarge = 0x40u;

// A CSR as the kernels see it (device pointers).
struct Csr {
  const uint32_t *__restrict__ ptr;
  const uint32_t *__restrict__ idx;
  const float *__restrict__ val;
  uint32_t nnz;  // entries stored; row ranges past it are treated as malformed
};

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// Monotone map of an f32 onto u32 (total order of the finite values and
// +-inf). -0 is folded onto +0 first, so IEEE-equal values get equal keys
// and a (key, index) minimum breaks a tie on the index alone.
__device__ __forceinline__ uint32_t f32_order(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float f32_unorder(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// Minimum of a u32 over the 64 lanes of the wave, returned in an SGPR.
// Called with every lane active. Within each row of 16 lanes: quad_perm
// swaps (xor 1, xor 2), then the half-row and row mirrors; every lane of a
// row then holds the row's minimum. Across rows: row_bcast:15 folds the last
// lane of rows 0 and 2 into rows 1 and 3, row_bcast:31 folds lane 31 into
// rows 2 and 3, so lane 63 ends with the minimum of all four rows. DPP
// sources take 0xffffffff (the identity of min) where a lane has no partner
// or its row is masked off, so each step is one v_min_u32_dpp.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0xB1, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x4E, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x141, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x140, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x142, 0xA, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// (lowest value, then lowest index) over the wave. Lanes with nothing to
// offer pass (+inf key, 0xffffffff).
__device__ __forceinline__ uint32_t wave_argmin(float v, uint32_t i) {
  const uint32_t key = f32_order(v);
  const uint32_t best = wave_min_u32(key);
  return wave_min_u32(key == best ? i : 0xffffffffu);
}

// Sum of an f32 over the wave in a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum_f32(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Ordering point between LDS accesses of different lanes of one wave. The
// LDS executes one wavefront's operations in issue order, so only the
// compiler has to be kept from moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float readlane_f32(float x, uint32_t lane) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), lane));
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t x, uint32_t lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// ---------------------------------------------------------------------------
// internal host interface (implemented in fw_a.hip / fw_b.hip)
// ---------------------------------------------------------------------------

struct DeviceInfo {
  int cus = 0;
  int ok = 0;
};
hipError_t device_info(DeviceInfo *out);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// --- A update -------------------------------------------------------------
// Plan overrides for tests and experiments (set through the debug ABI; the
// defaults choose by k). Process-wide: the workspace query and the calls
// read the same values.
struct AOptions {
  int support = -1;            // -1: by k; 0: never the support state; 1: for any k
  uint32_t support_waves = 0;  // resident waves per CU the first support pass is sized for (0: default)
  bool dense_argmin = false;   // a dense scan decides every step
  uint32_t group = 0;          // lanes per cell of the dense kernels (0: by k; 16, 32, 64)
  int support_wide = -1;       // first support pass: -1 by K2B row length, 0: 256, 1: 512 in registers
};
AOptions &a_options();

struct APlan {
  bool prune;                  // the pruning + renormalisation variant
  uint32_t group;              // lanes per cell (16, 32 or 64)
  uint32_t kpad;               // scan length: k + 1 rounded up to 4 * group (padding holds +inf)
  uint32_t waves_per_block;    // 0: the atom list alone does not fit in LDS
  uint32_t lds_per_wave;       // bytes
  uint32_t sched_words;        // LDS words of the per-block step schedule (0: computed per step)
  bool h_in_lds;
  bool reg_atoms;              // atoms in registers (cap <= 128), else in LDS
  uint32_t global_waves;       // waves that own a workspace slice (state in workspace)
  uint32_t ws_words_per_wave;  // state words per wave in the workspace
  // support state (large k): a first pass settles most cells, the dense
  // kernel above takes the cells it queues
  bool support;
  uint32_t nwords;             // 32-column words of the bitmaps
  size_t ws_list_off;          // cells for the long-row pass (counters sit at offset 0)
  size_t ws_list2_off;         // cells for the dense kernel
  size_t ws_keys_off, ws_hist_off, ws_order_off;  // the cells' locality order (support only)
  size_t ws_dense_off;         // dense state slices
  // one cell per wave: t1 copied with every row padded to whole chunks of 64
  // (column byte offset, value) pairs, so a step reads rows without checks
  bool padded;
  uint32_t pad_chunks;         // bound on the chunks of all rows
  size_t ws_pt_ptr_off;        // [k + 1] u32: 2 * first chunk of row r, | 1 if r has a value < 0
  size_t ws_pt_ent_off;        // [pad_chunks * 64] uint2
  size_t ws_bytes;
};
APlan plan_a(uint32_t n, uint32_t k, uint32_t T, uint32_t cap, bool prune, uint32_t t1_nnz);
hipError_t launch_fw_a(const APlan &plan, Csr t1, Csr k2b, Csr ap, uint32_t n, uint32_t k,
                       uint32_t T, uint32_t cap, const float *gamma, float prune_thr,
                       uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt, uint32_t *trace,
                       float *fw_gap, void *ws, uint32_t *status, hipStream_t stream);

// --- B argmin -------------------------------------------------------------
struct BPlan {
  uint32_t s4;            // float4 column chunks per lane of the accumulator
  uint32_t slice_w;       // columns per slice (<= 256 * s4)
  uint32_t n_slices;
  uint32_t n_row_blocks;  // row ranges; one work unit = (row range, slice)
  uint32_t n_chunks;      // row-range groups of the first reduce stage
  // narrow slices: the two half-waves gather different K2B entries (runs
  // of AAt from the segment table); otherwise one wave per entry reads AAt
  // copied per slice, the run of row m inside slice s padded to whole
  // chunks of pa_ch (accumulator byte offset, value) pairs (chunk 0 is all
  // padding): pa_seg[s * k + m] = first chunk of that run (slice-major).
  bool dual;
  uint32_t pa_ch;         // entries per chunk (64), 0 without the copy
  uint64_t pa_chunks;     // bound on the chunks of all runs, chunk 0 included
  // narrow slices also place each slice's columns in the accumulator in an
  // order of their own (two walk vectors of k floats, then the column ->
  // position and position -> column tables, 16-bit, slice-local)
  size_t off_keys, off_part2, off_gap, off_gap2, off_stamp, off_work, off_seg, off_rs, off_pa_seg,
      off_pa_bsum, off_pa_ent, off_pc_col, off_pc_val, off_walk, off_cpos, off_pcol;
  // narrow slices, more than one per XCD: the slices each XCD owns, chosen
  // per call to even out the XCDs' gather work (a K2B column histogram, the
  // work of every slice, then the slices of XCD x at
  // xcd_list[xcd_off[x] .. xcd_off[x + 1]))
  bool balance;
  size_t off_hist, off_swork, off_xcd_off, off_xcd_list;
  size_t ws_bytes;
};
BPlan plan_b(uint32_t n, uint32_t k, uint64_t aat_nnz);
hipError_t launch_fw_b(const BPlan &plan, Csr k2b, Csr aat, Csr k2at, Csr b, uint32_t n,
                       uint32_t k, float *out_val, uint32_t *out_idx, float *gap,
                       float *fw_gap, void *ws, uint32_t *status, uint32_t epoch,
                       hipStream_t stream);
// the two reduce stages alone, on the partials a launch_fw_b with the same
// plan left in ws (stamped with `epoch`)
hipError_t launch_fw_b_reduce(const BPlan &plan, uint32_t n, uint32_t k, float *out_val,
                              uint32_t *out_idx, float *gap, float *fw_gap, void *ws,
                              uint32_t *status, uint32_t epoch, hipStream_t stream);
hipError_t launch_fw_b_apply(uint32_t *bt_idx, float *bt_val, uint32_t *bt_cnt, uint32_t n,
                             uint32_t k, uint32_t cap_b, const uint32_t *arg_idx, float gamma,
                             uint32_t *status, hipStream_t stream);
hipError_t launch_status_clear(uint32_t *status, hipStream_t stream);

// --- sparse operations that build the operands -----------------------------
uint32_t tr_blocks(uint32_t m, uint32_t q);
size_t transpose_workspace(uint32_t m, uint32_t q);
size_t matmul_workspace(uint32_t m);
size_t matmul_pattern_bytes(uint32_t m, uint32_t q);
size_t add_workspace(uint32_t m);
hipError_t launch_atoms_count(const uint32_t *atom_idx, const float *atom_val,
                              const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                              uint32_t *at_ptr, void *ws, uint32_t *status, hipStream_t stream);
hipError_t launch_atoms_fill(const uint32_t *atom_idx, const float *atom_val,
                             const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                             const uint32_t *at_ptr, uint32_t *at_idx, float *at_val,
                             uint32_t *status, hipStream_t stream);
size_t vertex_workspace(uint32_t k, uint32_t n);
hipError_t launch_add_count(Csr x, Csr y, uint32_t m, uint32_t q, uint32_t *c_ptr, void *ws,
                            uint32_t *status, hipStream_t stream);
hipError_t launch_add_fill(float alpha, Csr x, float beta, Csr y, uint32_t m, const uint32_t *c_ptr,
                           uint32_t *c_idx, float *c_val, uint64_t c_cap, uint32_t *status,
                           hipStream_t stream);
hipError_t launch_vertex(const uint32_t *pick, uint32_t k, uint32_t n, float value, uint32_t *s_ptr,
                         uint32_t *s_idx, float *s_val, void *ws, uint32_t *status,
                         hipStream_t stream);
size_t dot_workspace();
hipError_t launch_spgemm_count(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                               uint32_t *c_ptr, void *ws, uint32_t *pattern, uint32_t *status,
                               hipStream_t stream);
hipError_t launch_spgemm_fill(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                              const uint32_t *c_ptr, uint32_t *c_idx, float *c_val, uint64_t c_cap,
                              const uint32_t *pattern, uint32_t *status, hipStream_t stream);
hipError_t launch_transpose(Csr a, uint32_t m, uint32_t q, uint32_t *at_ptr, uint32_t *at_idx,
                            float *at_val, void *ws, uint32_t *status, hipStream_t stream);
hipError_t launch_dot(Csr x, Csr y, uint32_t m, double alpha, double *acc, void *ws,
                      uint32_t *status, hipStream_t stream);

}  // namespace seacells
