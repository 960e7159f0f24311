// Sparse operations that build the Frank-Wolfe operands on the device: the
// page's host routines `csr_matmul_csr` (product of two CSR matrices, each
// output row sorted), `transpose_sparse` (rows of the transpose in ascending
// order of the original rows), and the sums the RSS identity needs
// (||K - K B A||^2 = <K, K> - 2 <K^2 B, A^T> + <B^T K^2 B, A A^T>).
//
// Product C = A B in two passes, one wave per row of A. The rows pass builds
//   a bitmap of the row's output columns in LDS (a window of 16384 columns at
//   a time) and counts them; a three-pass scan makes the counts the row
//   pointer. With one column window it can keep every row's bitmap and a
//   list of the rows longer than one value window for the fill pass. The
//   fill pass takes the bitmap (kept, or built again), a popcount prefix over
//   it gives every column its rank, and the products are added into an LDS
//   slot per rank (a window of 1024 ranks at a time), then written out in
//   column order (an LDS map from slot to column lets consecutive lanes store
//   consecutive entries); with kept bitmaps the value windows of the listed
//   rows run as units of their own on other waves. The
//   products of the row are flattened over the lanes: 64 entries of A at a
//   time, one per lane, load their B row bounds together; a scan of the B row
//   lengths numbers the products (A entry, then B entry) and each window of
//   64 consecutive products goes one per lane. Adds into the slots run entry
//   by entry within a window (the columns of one B row are unique, so lanes
//   of one entry never collide), so every output sums its products in
//   A-entry order, then B-entry order, in f32 with fma. The output keeps
//   every column that some product reaches (a sum that cancels to 0 stays as
//   an explicit 0). A row of A with kHeavyEntries entries or more (when B has
//   one column window) is taken by a block of kHvWaves waves instead, in both
//   passes: wave w takes run w of the row's entries, marks its columns in the
//   block's bitmap, and sums its products in slots of its own; the runs' sums
//   are then added in run order. (An archetype that many cells keep as an
//   atom makes such a row of A A^T, with ~10^5 to 10^6 products.)
// Transpose: rows are cut into R blocks; one wave per block counts its
//   entries per column, the counts become per-(block, column) write
//   positions, and each wave writes its rows in order, so a transposed row
//   lists the original rows in ascending order (no atomics on positions).
// Sum C = alpha X + beta Y over the union of the two patterns (the page's
//   `sparse_add_csr` merges two sorted rows): one wave per row; each entry's
//   place in the merged row is its rank in its own row plus the number of
//   smaller columns in the other row (a binary search) less the common
//   columns below it (a scan of the matches), so the lanes write
//   independently. A column stored in both is written once, from X's side.
// The Frank-Wolfe vertex of the B step (1 at (pick of column c, c)) is the
//   transpose of the k x n matrix with one entry per row.
// Inner product <X, Y> over two matrices of the same shape: one wave per row
//   looks each entry of the operand with fewer entries up in the other's row
//   (binary search), products in f64; the rows' partial sums are added in a
//   fixed order.
// The A update's atoms as A^T: a thread per cell counts the atoms of non-zero
//   weight, then a wave per cell places each at its rank by column.
#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kSpWaves = 4;        // waves per block
constexpr uint32_t kSpWinWords = 512;   // bitmap words per column window (16384 columns)
constexpr uint32_t kSpSlots = 1024;     // value slots per rank window
constexpr uint32_t kSpGroup = 4;        // product windows loaded together
// Rows of A with many entries (hub rows, e.g. an archetype many cells keep
// as an atom in A A^T) go to a block of kHvWaves waves instead of one wave,
// each wave taking one run of the row's entries, when b has at most one
// column window of columns.
constexpr uint32_t kHeavyEntries = 2048;
constexpr uint32_t kHvWaves = 16;
constexpr uint32_t kHvThreads = kHvWaves * kWave;
constexpr uint32_t kHvSlots = 2048;     // value slots per wave and rank window (heavy rows)
constexpr uint32_t kHvPartBytes = kHvWaves * kHvSlots * sizeof(float);  // 128 KB, dynamic LDS
constexpr uint32_t kTrMaxBlocks = 1024;
constexpr size_t kTrTableBytes = 64u << 20;  // per-(block, column) table of the transpose
constexpr uint32_t kDotBlocks = 1024;

__device__ __forceinline__ bool sp_row(const Csr &m, uint32_t r, uint32_t &lo, uint32_t &hi) {
  lo = m.ptr[r];
  hi = m.ptr[r + 1];
  if (hi > m.nnz || lo > hi) {
    lo = hi = 0;
    return false;
  }
  return true;
}

__device__ __forceinline__ uint64_t u64min(uint64_t x, uint64_t y) { return x < y ? x : y; }

// Ordering point between global accesses of different lanes of one wave:
// every earlier store has completed before a later load is issued (a
// workgroup-scope fence; also a compiler barrier).
__device__ __forceinline__ void wave_mem_wait() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
  for (int off = 32; off >= 1; off >>= 1)
    x += (uint64_t)__shfl_xor((unsigned long long)x, off, kWave);
  return x;
}

// Exclusive prefix sum over the wave (lane order).
__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t x, uint32_t lane) {
  uint32_t incl = x;
  for (uint32_t off = 1; off < kWave; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  return incl - x;
}

// Walk the products of A's row [a0, a1) in order, 64 at a time. For each
// window f(valid, c, bv, a_own, own, owners) is called by the whole wave:
// the lane holds product number base + lane if valid, with B column c and
// value bv (0 unless kVal), the value a_own of its A entry, and own, that
// entry's lane within the current chunk of 64 A entries; owners (uniform) is
// the mask of chunk lanes with products in the window. Returns flags.
template <bool kVal, class F>
__device__ __forceinline__ uint32_t for_products(const Csr &a, const Csr &b, uint32_t p,
                                                 uint32_t a0, uint32_t a1, uint32_t lane,
                                                 F &&f) {
  uint32_t flags = 0;
  for (uint32_t ch = a0; ch < a1; ch += kWave) {
    const uint32_t e = ch + lane;
    uint32_t len = 0, b0 = 0;
    float av = 0.0f;
    if (e < a1) {
      const uint32_t j = a.idx[e];
      if (kVal) av = a.val[e];
      uint32_t lo, hi;
      if (j < p && sp_row(b, j, lo, hi)) {
        b0 = lo;
        len = hi - lo;
      } else {
        flags |= kFlagBadIndex;
      }
    }
    // rows of a well-formed B are disjoint, so the 64 lengths sum below
    // 2^31; overlapping rows (a malformed row pointer) could wrap the scan
    if (wave_sum_u64(len) >= 0x80000000ull) {
      flags |= kFlagBadIndex;
      len = 0;
    }
    // off: number of the entry's first product; nondecreasing over the lanes
    const uint32_t off = wave_excl_scan_u32(len, lane);
    const uint32_t total = readlane_u32(off + len, kWave - 1);
    if (total == 0) continue;
    const uint64_t nonempty = __ballot(len > 0);
    // State of the window starting at product `base` (< total): the lane's
    // owner, its B entry t (for a lane past the end, the window's first
    // product, so every lane loads from inside B), the owner's value and the
    // owners of the window.
    auto window = [&](uint32_t base, uint32_t &own, uint32_t &t, float &a_own, uint64_t &owners) {
      const uint32_t pi = base + lane;
      // the first owner is the last entry starting at or before base (it is
      // never empty); the others start inside the window
      const uint32_t l_lo = (uint32_t)__popcll(__ballot(off <= base)) - 1u;
      const uint64_t upto = __ballot(off < base + kWave);  // lanes 0 .. l_hi
      owners = nonempty & upto & ~((1ull << l_lo) - 1ull);
      const uint32_t o_lo = readlane_u32(off, l_lo), b_lo = readlane_u32(b0, l_lo);
      own = l_lo;
      t = b_lo + (pi - o_lo);
      a_own = kVal ? readlane_f32(av, l_lo) : 0.0f;
      for (uint64_t mm = owners & (owners - 1ull); mm != 0; mm &= mm - 1ull) {
        const uint32_t l = (uint32_t)__builtin_ctzll(mm);
        const uint32_t ol = readlane_u32(off, l);
        const uint32_t bl = readlane_u32(b0, l);
        const float al = kVal ? readlane_f32(av, l) : 0.0f;
        if (ol <= pi) {
          own = l;
          t = bl + (pi - ol);
          a_own = al;
        }
      }
      if (pi >= total) t = b_lo + (base - o_lo);
    };
    if (total <= kWave) {  // one window: no pipeline
      uint32_t own, t;
      float a_own;
      uint64_t owners;
      window(0, own, t, a_own, owners);
      const uint32_t c = b.idx[t];
      const float bv = kVal ? b.val[t] : 0.0f;
      f(lane < total, c, bv, a_own, own, owners);
      continue;
    }
    // Software pipeline over groups of kSpGroup windows: the loads of the
    // next group are in flight while the current group is processed. A
    // window past the end repeats the previous window's loads and is not
    // processed, so the number of loads in flight never depends on the data.
    const uint32_t last = (total - 1u) & ~(kWave - 1u);  // first product of the last window
    uint32_t own[kSpGroup], c[kSpGroup];
    uint64_t om[kSpGroup];
    float ao[kSpGroup], bv[kSpGroup];
    auto issue = [&](uint32_t g0) {  // g0 <= last
      uint32_t t = 0;
#pragma unroll
      for (uint32_t u = 0; u < kSpGroup; ++u) {
        const uint32_t wb = g0 + u * kWave;
        if (u == 0 || wb <= last) {
          window(wb, own[u], t, ao[u], om[u]);
        } else {
          own[u] = own[u - 1];
          ao[u] = ao[u - 1];
          om[u] = om[u - 1];
        }
        c[u] = b.idx[t];
        bv[u] = kVal ? b.val[t] : 0.0f;
      }
    };
    issue(0);
    for (uint32_t g0 = 0; g0 < total; g0 += kSpGroup * kWave) {
      uint32_t own_c[kSpGroup], c_c[kSpGroup];
      uint64_t om_c[kSpGroup];
      float ao_c[kSpGroup], bv_c[kSpGroup];
#pragma unroll
      for (uint32_t u = 0; u < kSpGroup; ++u) {
        own_c[u] = own[u];
        om_c[u] = om[u];
        c_c[u] = c[u];
        ao_c[u] = ao[u];
        bv_c[u] = bv[u];
      }
      const uint32_t g1 = g0 + kSpGroup * kWave;
      issue(g1 <= last ? g1 : last);
#pragma unroll
      for (uint32_t u = 0; u < kSpGroup; ++u) {
        const uint32_t wb = g0 + u * kWave;
        if (wb < total) f(wb + lane < total, c_c[u], bv_c[u], ao_c[u], own_c[u], om_c[u]);
      }
    }
  }
  return flags;
}

__device__ __forceinline__ bool heavy_row(uint32_t a0, uint32_t a1, uint32_t q) {
  return q <= kSpWinWords * 32u && a1 - a0 >= kHeavyEntries;
}

// Run w of kHvWaves consecutive runs of the entries [a0, a1).
__device__ __forceinline__ void heavy_run(uint32_t a0, uint32_t a1, uint32_t w, uint32_t &s0,
                                          uint32_t &s1) {
  const uint64_t len = a1 - a0;
  s0 = a0 + (uint32_t)(len * w / kHvWaves);
  s1 = a0 + (uint32_t)(len * (w + 1u) / kHvWaves);
}

// The heavy rows among r = blockIdx.x + gridDim.x * j, kHvThreads values of
// j at a time, into list[0 .. *nlist) (any order: each row is a unit of its
// own). Returns false when the block has no rows left at j0.
__device__ __forceinline__ bool heavy_batch(const Csr &a, uint32_t m, uint32_t q, uint64_t j0,
                                            uint32_t *list, uint32_t *nlist) {
  if ((uint64_t)blockIdx.x + (uint64_t)gridDim.x * j0 >= m) return false;
  __syncthreads();  // every thread has read the last batch's count
  if (threadIdx.x == 0) *nlist = 0u;
  __syncthreads();
  const uint64_t r = (uint64_t)blockIdx.x + (uint64_t)gridDim.x * (j0 + threadIdx.x);
  if (r < m) {
    uint32_t a0, a1;
    if (sp_row(a, (uint32_t)r, a0, a1) && heavy_row(a0, a1, q))
      list[atomicAdd(nlist, 1u)] = (uint32_t)r;
  }
  __syncthreads();
  return true;
}

// Mark in bits[] (window starting at column w0, nw words) every column some
// product of A's row [a0, a1) reaches. Returns the flags seen.
__device__ __forceinline__ uint32_t mark_columns(const Csr &a, const Csr &b, uint32_t p,
                                                 uint32_t q, uint32_t a0, uint32_t a1,
                                                 uint32_t w0, uint32_t nw, uint32_t *bits,
                                                 uint32_t lane) {
  uint32_t flags = 0;
  flags |= for_products<false>(a, b, p, a0, a1, lane,
                               [&](bool valid, uint32_t c, float, float, uint32_t, uint64_t) {
                                 if (!valid) return;
                                 if (c >= q) {
                                   flags |= kFlagBadIndex;
                                   return;
                                 }
                                 const uint32_t rel = c - w0;
                                 if (rel < nw * 32u) atomicOr(&bits[rel >> 5], 1u << (rel & 31u));
                               });
  return flags;
}

// Output columns per row of A B into cnt[r] (the caller's row pointer + 1).
__global__ void __launch_bounds__(kSpWaves * kWave)
    spgemm_count_kernel(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                        uint32_t *__restrict__ cnt, uint32_t *__restrict__ pattern,
                        uint32_t *__restrict__ long_rows, uint32_t *__restrict__ status) {
  __shared__ uint32_t bits_all[kSpWaves][kSpWinWords];
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t *bits = bits_all[wib];
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * kSpWaves + wib; r < m; r += gridDim.x * kSpWaves) {
    uint32_t a0, a1;
    if (!sp_row(a, r, a0, a1)) flags |= kFlagBadIndex;
    if (heavy_row(a0, a1, q)) continue;  // (spgemm_count_heavy_kernel)
    uint64_t total = 0;
    for (uint64_t w0 = 0; w0 < q; w0 += (uint64_t)kSpWinWords * 32u) {
      const uint32_t nw = (uint32_t)u64min(kSpWinWords, (q - w0 + 31u) / 32u);
      for (uint32_t w = lane; w < nw; w += kWave) bits[w] = 0u;
      wave_lds_sync();
      flags |= mark_columns(a, b, p, q, a0, a1, (uint32_t)w0, nw, bits, lane);
      wave_lds_sync();
      uint32_t part = 0;
      for (uint32_t w = lane; w < nw; w += kWave) {
        const uint32_t x = bits[w];
        part += __popc(x);
        if (pattern != nullptr) pattern[(size_t)r * nw + w] = x;  // (one window only)
      }
      total += wave_sum_u32(part);
      wave_lds_sync();
    }
    if (lane == 0) {
      cnt[r] = total > 0xffffffffull ? 0xffffffffu : (uint32_t)total;
      // rows of more than one value window: listed for the fill pass (any order)
      if (long_rows != nullptr && total > kSpSlots) long_rows[1u + atomicAdd(long_rows, 1u)] = r;
    }
  }
  if (flags != 0) atomicOr(status, flags);
}

// Counts of the heavy rows: one block per row, wave w marks the columns of
// run w of the row's entries in the block's bitmap (integer ORs: the result
// does not depend on their order).
__global__ void __launch_bounds__(kHvThreads)
    spgemm_count_heavy_kernel(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                              uint32_t *__restrict__ cnt, uint32_t *__restrict__ pattern,
                              uint32_t *__restrict__ status) {
  __shared__ uint32_t bits[kSpWinWords];
  __shared__ uint32_t list[kHvThreads];
  __shared__ uint32_t nlist;
  __shared__ uint32_t wsum[kHvWaves];
  const uint32_t lane = lane_id(), w = threadIdx.x / kWave;
  const uint32_t nw = (q + 31u) / 32u;  // <= kSpWinWords for heavy rows
  uint32_t flags = 0;
  for (uint64_t j0 = 0; heavy_batch(a, m, q, j0, list, &nlist); j0 += kHvThreads) {
    const uint32_t nl = nlist;
    for (uint32_t i = 0; i < nl; ++i) {
      const uint32_t r = list[i];
      uint32_t a0, a1, s0, s1;
      sp_row(a, r, a0, a1);
      heavy_run(a0, a1, w, s0, s1);
      for (uint32_t x = threadIdx.x; x < nw; x += kHvThreads) bits[x] = 0u;
      __syncthreads();
      flags |= mark_columns(a, b, p, q, s0, s1, 0u, nw, bits, lane);
      __syncthreads();
      uint32_t part = 0;
      for (uint32_t x = threadIdx.x; x < nw; x += kHvThreads) {
        part += __popc(bits[x]);
        if (pattern != nullptr) pattern[(size_t)r * nw + x] = bits[x];
      }
      part = wave_sum_u32(part);
      if (lane == 0) wsum[w] = part;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t total = 0;
        for (uint32_t x = 0; x < kHvWaves; ++x) total += wsum[x];
        cnt[r] = total;
      }
      __syncthreads();
    }
  }
  if (flags != 0) atomicOr(status, flags);
}

__global__ void __launch_bounds__(64) zero_word_kernel(uint32_t *__restrict__ p) {
  if (threadIdx.x == 0) p[0] = 0u;
}

// Row pointers from counts, in place: ptr[0] = 0 and ptr[1 .. count]
// becomes the inclusive prefix sum of itself. Three passes over tiles of
// kScanTile values (256 threads x 16 consecutive values): tile sums, one
// block scanning the tile sums in 64 bits (part[G] = 1 when the total reaches
// 2^31: the flag is set and every pointer becomes 0, so a later pass over
// them writes nothing), then each tile scanned from its offset.
constexpr uint32_t kScanThreads = 256, kScanItems = 16, kScanTile = kScanThreads * kScanItems;

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x, uint32_t lane) {
  for (uint32_t off = 1; off < kWave; off <<= 1) {
    const uint64_t v = (uint64_t)__shfl_up((unsigned long long)x, off, kWave);
    if (lane >= off) x += v;
  }
  return x;
}

// Exclusive scan over the 256 threads of a block; *total gets the sum.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t x, uint64_t *sh, uint64_t *total) {
  const uint32_t lane = lane_id(), wid = threadIdx.x / kWave;
  const uint64_t incl = wave_incl_scan_u64(x, lane);
  if (lane == kWave - 1) sh[wid] = incl;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (uint32_t w = 0; w < kScanThreads / kWave; ++w) {
    if (w < wid) before += sh[w];
    all += sh[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

__global__ void __launch_bounds__(kScanThreads)
    scan_tile_sums_kernel(const uint32_t *__restrict__ x, uint32_t count,
                          uint64_t *__restrict__ part) {
  __shared__ uint64_t sh[kScanThreads / kWave];
  const size_t i0 = (size_t)blockIdx.x * kScanTile + (size_t)threadIdx.x * kScanItems;
  uint64_t sum = 0;
  for (uint32_t k = 0; k < kScanItems; ++k)
    if (i0 + k < count) sum += x[i0 + k];
  uint64_t total;
  block_excl_scan_u64(sum, sh, &total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

__global__ void __launch_bounds__(kScanThreads)
    scan_partials_kernel(uint64_t *__restrict__ part, uint32_t tiles, uint32_t *__restrict__ ptr,
                         uint32_t too_large_flag, uint32_t *__restrict__ status) {
  __shared__ uint64_t sh[kScanThreads / kWave];
  uint64_t carry = 0;
  for (uint32_t t0 = 0; t0 < tiles; t0 += kScanThreads) {
    const uint32_t i = t0 + threadIdx.x;
    const uint64_t v = i < tiles ? part[i] : 0u;
    uint64_t total;
    const uint64_t ex = block_excl_scan_u64(v, sh, &total);
    if (i < tiles) part[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) {
    const bool too_large = carry >= 0x80000000ull;
    part[tiles] = too_large ? 1u : 0u;
    ptr[0] = 0u;
    if (too_large) atomicOr(status, too_large_flag);
  }
}

__global__ void __launch_bounds__(kScanThreads)
    scan_apply_kernel(uint32_t *__restrict__ x, uint32_t count, const uint64_t *__restrict__ part,
                      uint32_t tiles) {
  __shared__ uint64_t sh[kScanThreads / kWave];
  const size_t i0 = (size_t)blockIdx.x * kScanTile + (size_t)threadIdx.x * kScanItems;
  uint32_t v[kScanItems];
  uint64_t sum = 0;
  for (uint32_t k = 0; k < kScanItems; ++k) {
    v[k] = i0 + k < count ? x[i0 + k] : 0u;
    sum += v[k];
  }
  uint64_t total;
  uint64_t at = part[blockIdx.x] + block_excl_scan_u64(sum, sh, &total);
  const bool too_large = part[tiles] != 0u;
  for (uint32_t k = 0; k < kScanItems; ++k) {
    at += v[k];
    if (i0 + k < count) x[i0 + k] = too_large ? 0u : (uint32_t)at;
  }
}

uint32_t scan_tiles(uint32_t count) { return (uint32_t)(((uint64_t)count + kScanTile - 1) / kScanTile); }

// ptr[0 .. count]: see above. part: scan_tiles(count) + 1 u64 of workspace.
hipError_t launch_scan(uint32_t *ptr, uint32_t count, uint64_t *part, uint32_t *status,
                       hipStream_t stream) {
  const uint32_t tiles = scan_tiles(count);
  hipError_t e;
  if (tiles > 0) {
    hipLaunchKernelGGL(scan_tile_sums_kernel, dim3(tiles), dim3(kScanThreads), 0, stream, ptr + 1,
                       count, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(kScanThreads), 0, stream, part, tiles, ptr,
                     kFlagOutputTooLarge, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tiles > 0) {
    hipLaunchKernelGGL(scan_apply_kernel, dim3(tiles), dim3(kScanThreads), 0, stream, ptr + 1, count,
                       part, tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Columns and values of A B into the rows the count pass sized.
__global__ void __launch_bounds__(kSpWaves * kWave)
    spgemm_fill_kernel(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                       const uint32_t *__restrict__ c_ptr, uint32_t *__restrict__ c_idx,
                       float *__restrict__ c_val, uint64_t c_cap,
                       const uint32_t *__restrict__ pattern,
                       const uint32_t *__restrict__ long_rows, uint32_t *__restrict__ status) {
  // more entries than the output arrays hold: nothing is written
  if (c_ptr[m] > c_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, kFlagOutputTooLarge);
    return;
  }
  __shared__ uint32_t bits_all[kSpWaves][kSpWinWords];
  __shared__ uint16_t rank_all[kSpWaves][kSpWinWords];
  __shared__ float acc_all[kSpWaves][kSpSlots];
  __shared__ uint16_t colof_all[kSpWaves][kSpSlots];
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t *bits = bits_all[wib];
  uint16_t *rank = rank_all[wib];
  float *acc = acc_all[wib];
  uint16_t *colof = colof_all[wib];
  uint32_t flags = 0;

  // ranks of the bitmap words in bits[0, nw): each lane takes a contiguous run
  // of words; returns the columns in the window, sets the lane's run and first
  // rank
  auto ranks = [&](uint32_t nw, uint32_t &v0w, uint32_t &v1w, uint32_t &first) -> uint32_t {
    const uint32_t per = (nw + kWave - 1) / kWave;
    v0w = min(lane * per, nw), v1w = min(v0w + per, nw);
    uint32_t part = 0;
    for (uint32_t w = v0w; w < v1w; ++w) part += __popc(bits[w]);
    uint32_t run = wave_excl_scan_u32(part, lane);
    const uint32_t nwin = wave_sum_u32(part);
    first = run;
    for (uint32_t w = v0w; w < v1w; ++w) {
      rank[w] = (uint16_t)run;  // < 16384: ranks within one column window
      run += __popc(bits[w]);
    }
    wave_lds_sync();
    return nwin;
  };
  // ranks s0 .. s0 + ns of row r's column window w0 (the window's first
  // output at base + done): accumulate them and write them out
  auto value_window = [&](uint32_t base, uint32_t cnt, uint32_t a0, uint32_t a1, uint32_t w0,
                          uint32_t nw, uint32_t done, uint32_t s0, uint32_t ns, uint32_t v0w,
                          uint32_t v1w, uint32_t first) {
    for (uint32_t s = lane; s < ns; s += kWave) acc[s] = 0.0f;
    // slot -> column within the window, from each lane's run of words
    {
      uint32_t pos = first;
      for (uint32_t w = v0w; w < v1w && pos < s0 + ns; ++w) {
        uint32_t x = bits[w];
        while (x != 0u) {
          const uint32_t bpos = (uint32_t)__builtin_ctz(x);
          x &= x - 1u;
          if (pos >= s0 && pos < s0 + ns) colof[pos - s0] = (uint16_t)(w * 32u + bpos);
          ++pos;
        }
      }
    }
    wave_lds_sync();
    // (bad indices were flagged by the marking pass)
    for_products<true>(a, b, p, a0, a1, lane,
                       [&](bool valid, uint32_t c, float bv, float a_own, uint32_t own,
                           uint64_t owners) {
                         const uint32_t rel = c - w0;
                         uint32_t pos = 0xffffffffu;
                         if (valid && c < q && rel < nw * 32u) {
                           const uint32_t w = rel >> 5, bit = 1u << (rel & 31u);
                           pos = rank[w] + __popc(bits[w] & (bit - 1u)) - s0;
                         }
                         const bool mine = pos < ns;
                         // entry by entry: the adds into one slot keep A-entry order
                         for (uint64_t mm = owners; mm != 0; mm &= mm - 1ull) {
                           const uint32_t l = (uint32_t)__builtin_ctzll(mm);
                           if (mine && own == l) acc[pos] = __builtin_fmaf(a_own, bv, acc[pos]);
                           wave_lds_sync();
                         }
                       });
    // out in column order, consecutive lanes on consecutive entries
    for (uint32_t s = lane; s < ns; s += kWave) {
      const uint32_t o = done + s0 + s;
      if (o < cnt) {
        c_idx[(size_t)base + o] = w0 + colof[s];
        c_val[(size_t)base + o] = acc[s];
      }
    }
    wave_lds_sync();
  };

  const uint32_t gw = blockIdx.x * kSpWaves + wib, nwaves = gridDim.x * kSpWaves;
  if (pattern != nullptr) {
    // one column window with the rows pass's bitmaps: the units are (row,
    // value window), window 0 of every row, then the further windows of the
    // long rows the rows pass listed, so a long row's windows run on
    // different waves (each output still sums its products in order)
    const uint32_t nw = (q + 31u) / 32u;
    const uint32_t nvw = (q + kSpSlots - 1u) / kSpSlots;  // value windows a row can need
    const uint32_t nlong = long_rows != nullptr ? min(long_rows[0], m) : 0u;
    const uint64_t units = (uint64_t)m + (uint64_t)nlong * (nvw > 1u ? nvw - 1u : 0u);
    for (uint64_t u = gw; u < units; u += nwaves) {
      uint32_t r, vw;
      if (u < m) {
        r = (uint32_t)u, vw = 0;
      } else {
        const uint64_t v = u - m;
        r = long_rows[1u + (uint32_t)(v % nlong)];
        vw = 1u + (uint32_t)(v / nlong);
        if (r >= m) {  // (the list holds rows below m)
          flags |= kFlagBadIndex;
          continue;
        }
      }
      uint32_t a0, a1;
      if (!sp_row(a, r, a0, a1)) flags |= kFlagBadIndex;
      if (heavy_row(a0, a1, q)) continue;  // (spgemm_fill_heavy_kernel)
      const uint32_t base = c_ptr[r], end = c_ptr[r + 1];
      const uint32_t cnt = end >= base ? end - base : 0u;
      const uint32_t s0 = vw * kSpSlots;
      if (vw > 0 && s0 >= cnt) continue;
      if (cnt > 0 && (c_idx == nullptr || c_val == nullptr)) {  // no output arrays given
        flags |= kFlagBadIndex;
        continue;
      }
      for (uint32_t w = lane; w < nw; w += kWave) bits[w] = pattern[(size_t)r * nw + w];
      wave_lds_sync();
      uint32_t v0w, v1w, first;
      const uint32_t nwin = ranks(nw, v0w, v1w, first);
      if (vw == 0 && nwin != cnt) flags |= kFlagBadIndex;  // not the rows pass's pointers
      if (s0 < nwin)
        value_window(base, cnt, a0, a1, 0u, nw, 0u, s0, min(kSpSlots, nwin - s0), v0w, v1w,
                     first);
      if (vw == 0 && nwin > kSpSlots && long_rows == nullptr) {  // (no list: finish the row here)
        for (uint32_t s1 = kSpSlots; s1 < nwin; s1 += kSpSlots)
          value_window(base, cnt, a0, a1, 0u, nw, 0u, s1, min(kSpSlots, nwin - s1), v0w, v1w,
                       first);
      }
    }
  } else {
    for (uint32_t r = gw; r < m; r += nwaves) {
      uint32_t a0, a1;
      if (!sp_row(a, r, a0, a1)) flags |= kFlagBadIndex;
      if (heavy_row(a0, a1, q)) continue;  // (spgemm_fill_heavy_kernel)
      const uint32_t base = c_ptr[r], end = c_ptr[r + 1];
      const uint32_t cnt = end >= base ? end - base : 0u;
      if (cnt > 0 && (c_idx == nullptr || c_val == nullptr)) {  // no output arrays given
        flags |= kFlagBadIndex;
        continue;
      }
      uint32_t done = 0;
      for (uint64_t w0l = 0; w0l < q; w0l += (uint64_t)kSpWinWords * 32u) {
        const uint32_t w0 = (uint32_t)w0l;
        const uint32_t nw = (uint32_t)u64min(kSpWinWords, (q - w0l + 31u) / 32u);
        for (uint32_t w = lane; w < nw; w += kWave) bits[w] = 0u;
        wave_lds_sync();
        flags |= mark_columns(a, b, p, q, a0, a1, w0, nw, bits, lane);
        wave_lds_sync();
        uint32_t v0w, v1w, first;
        const uint32_t nwin = ranks(nw, v0w, v1w, first);
        for (uint32_t s0 = 0; s0 < nwin; s0 += kSpSlots)
          value_window(base, cnt, a0, a1, w0, nw, done, s0, min(kSpSlots, nwin - s0), v0w, v1w,
                       first);
        done += nwin;
      }
      if (done != cnt) flags |= kFlagBadIndex;  // row pointers not those of the count pass
    }
  }
  if (flags != 0) atomicOr(status, flags);
}

// Values of the heavy rows: one block per row. The row's columns come from
// the rows pass's bitmap (kept) or are marked again (wave w: run w of the
// entries); wave 0 ranks them. Per window of kHvSlots ranks, wave w sums
// the products of run w in its own slots (entry by entry, in order, as a
// light row's wave does), then slot s of the window gets the kHvWaves sums
// added in run order.
__global__ void __launch_bounds__(kHvThreads)
    spgemm_fill_heavy_kernel(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                             const uint32_t *__restrict__ c_ptr, uint32_t *__restrict__ c_idx,
                             float *__restrict__ c_val, uint64_t c_cap,
                             const uint32_t *__restrict__ pattern,
                             uint32_t *__restrict__ status) {
  if (c_ptr[m] > c_cap) return;  // (spgemm_fill_kernel raises the flag)
  __shared__ uint32_t bits[kSpWinWords];
  __shared__ uint16_t rank[kSpWinWords];
  __shared__ uint16_t colof[kHvSlots];
  extern __shared__ float part[];  // kHvWaves x kHvSlots
  __shared__ uint32_t list[kHvThreads];
  __shared__ uint32_t nlist, nwin_s;
  const uint32_t lane = lane_id(), w = threadIdx.x / kWave;
  const uint32_t nw = (q + 31u) / 32u;  // <= kSpWinWords for heavy rows
  float *acc = part + (size_t)w * kHvSlots;
  uint32_t flags = 0;
  for (uint64_t j0 = 0; heavy_batch(a, m, q, j0, list, &nlist); j0 += kHvThreads) {
    const uint32_t nl = nlist;
    for (uint32_t i = 0; i < nl; ++i) {
      const uint32_t r = list[i];
      uint32_t a0, a1, e0, e1;
      sp_row(a, r, a0, a1);
      heavy_run(a0, a1, w, e0, e1);
      const uint32_t base = c_ptr[r], end = c_ptr[r + 1];
      const uint32_t cnt = end >= base ? end - base : 0u;
      if (cnt > 0 && (c_idx == nullptr || c_val == nullptr)) {  // (uniform over the block)
        flags |= kFlagBadIndex;
        continue;
      }
      if (pattern != nullptr) {
        for (uint32_t x = threadIdx.x; x < nw; x += kHvThreads) bits[x] = pattern[(size_t)r * nw + x];
      } else {
        for (uint32_t x = threadIdx.x; x < nw; x += kHvThreads) bits[x] = 0u;
        __syncthreads();
        flags |= mark_columns(a, b, p, q, e0, e1, 0u, nw, bits, lane);
      }
      __syncthreads();
      // wave 0: ranks of the words (each lane a contiguous run of words)
      uint32_t v0w = 0, v1w = 0, first = 0;
      if (w == 0) {
        const uint32_t per = (nw + kWave - 1) / kWave;
        v0w = min(lane * per, nw), v1w = min(v0w + per, nw);
        uint32_t cnt_l = 0;
        for (uint32_t x = v0w; x < v1w; ++x) cnt_l += __popc(bits[x]);
        uint32_t run = wave_excl_scan_u32(cnt_l, lane);
        first = run;
        for (uint32_t x = v0w; x < v1w; ++x) {
          rank[x] = (uint16_t)run;
          run += __popc(bits[x]);
        }
        const uint32_t nwin = wave_sum_u32(cnt_l);
        if (lane == 0) nwin_s = nwin;
      }
      __syncthreads();
      const uint32_t nwin = nwin_s;
      if (nwin != cnt) flags |= kFlagBadIndex;  // not the rows pass's pointers
      for (uint32_t s0 = 0; s0 < nwin; s0 += kHvSlots) {
        const uint32_t ns = min(kHvSlots, nwin - s0);
        if (w == 0) {  // slot -> column
          uint32_t pos = first;
          for (uint32_t x = v0w; x < v1w && pos < s0 + ns; ++x) {
            uint32_t bx = bits[x];
            while (bx != 0u) {
              const uint32_t bpos = (uint32_t)__builtin_ctz(bx);
              bx &= bx - 1u;
              if (pos >= s0 && pos < s0 + ns) colof[pos - s0] = (uint16_t)(x * 32u + bpos);
              ++pos;
            }
          }
        }
        for (uint32_t x = lane; x < ns; x += kWave) acc[x] = 0.0f;
        wave_lds_sync();
        for_products<true>(a, b, p, e0, e1, lane,
                           [&](bool valid, uint32_t c, float bv, float a_own, uint32_t own,
                               uint64_t owners) {
                             uint32_t pos = 0xffffffffu;
                             if (valid && c < q) {
                               const uint32_t x = c >> 5, bit = 1u << (c & 31u);
                               pos = rank[x] + __popc(bits[x] & (bit - 1u)) - s0;
                             }
                             const bool mine = pos < ns;
                             for (uint64_t mm = owners; mm != 0; mm &= mm - 1ull) {
                               const uint32_t l = (uint32_t)__builtin_ctzll(mm);
                               if (mine && own == l) acc[pos] = __builtin_fmaf(a_own, bv, acc[pos]);
                               wave_lds_sync();
                             }
                           });
        __syncthreads();
        for (uint32_t x = threadIdx.x; x < ns; x += kHvThreads) {
          float v = part[x];
          for (uint32_t u = 1; u < kHvWaves; ++u) v += part[(size_t)u * kHvSlots + x];
          const uint32_t o = s0 + x;
          if (o < cnt) {
            c_idx[(size_t)base + o] = colof[x];
            c_val[(size_t)base + o] = v;
          }
        }
        __syncthreads();
      }
    }
  }
  if (flags != 0) atomicOr(status, flags);
}

// Transpose, pass 1: entries per (row block, column). One wave per block,
// rows in order; the columns of a row are unique, so the lanes never add to
// the same counter.
__global__ void __launch_bounds__(kWave)
    tr_count_kernel(Csr a, uint32_t m, uint32_t q, uint32_t nb, uint32_t *__restrict__ table,
                    uint32_t *__restrict__ status) {
  const uint32_t bk = blockIdx.x, lane = threadIdx.x;
  uint32_t *row = table + (size_t)bk * q;
  for (uint32_t c = lane; c < q; c += kWave) row[c] = 0u;
  wave_mem_wait();
  const uint32_t r0 = (uint32_t)(((uint64_t)m * bk) / nb);
  const uint32_t r1 = (uint32_t)(((uint64_t)m * (bk + 1)) / nb);
  uint32_t flags = 0;
  for (uint32_t r = r0; r < r1; ++r) {
    uint32_t lo, hi;
    if (!sp_row(a, r, lo, hi)) flags |= kFlagBadIndex;
    for (uint32_t t = lo + lane; t < hi; t += kWave) {
      const uint32_t c = a.idx[t];
      if (c < q)
        row[c] += 1u;
      else
        flags |= kFlagBadIndex;
    }
    wave_mem_wait();  // the next row's counters see this row's stores
  }
  if (flags != 0) atomicOr(status, flags);
}

// Pass 2: per column, counts over blocks become exclusive offsets within the
// column, and the column's total goes to at_ptr[c + 1].
__global__ void __launch_bounds__(256)
    tr_colsum_kernel(uint32_t q, uint32_t nb, uint32_t *__restrict__ table,
                     uint32_t *__restrict__ at_ptr) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= q) return;
  uint32_t run = 0;
  for (uint32_t bk = 0; bk < nb; ++bk) {
    const size_t i = (size_t)bk * q + c;
    const uint32_t v = table[i];
    table[i] = run;
    run += v;
  }
  at_ptr[c + 1] = run;
}

// Pass 3 (after the scan of at_ptr): offsets become absolute positions.
__global__ void __launch_bounds__(256)
    tr_base_kernel(uint32_t q, uint32_t nb, uint32_t *__restrict__ table,
                   const uint32_t *__restrict__ at_ptr) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= q) return;
  const uint32_t b0 = at_ptr[c];
  for (uint32_t bk = 0; bk < nb; ++bk) table[(size_t)bk * q + c] += b0;
}

// Pass 4: each block writes its rows in order at its own positions. Rows
// that overlap (a row pointer that falls and rises again) can count more
// entries than nnz; positions past nnz are dropped (the count pass flagged
// the falling row).
__global__ void __launch_bounds__(kWave)
    tr_fill_kernel(Csr a, uint32_t m, uint32_t q, uint32_t nb, uint32_t *__restrict__ table,
                   uint32_t *__restrict__ at_idx, float *__restrict__ at_val) {
  const uint32_t bk = blockIdx.x, lane = threadIdx.x;
  uint32_t *row = table + (size_t)bk * q;
  const uint32_t r0 = (uint32_t)(((uint64_t)m * bk) / nb);
  const uint32_t r1 = (uint32_t)(((uint64_t)m * (bk + 1)) / nb);
  for (uint32_t r = r0; r < r1; ++r) {
    uint32_t lo, hi;
    sp_row(a, r, lo, hi);
    for (uint32_t t = lo + lane; t < hi; t += kWave) {
      const uint32_t c = a.idx[t];
      if (c < q) {
        const uint32_t pos = row[c];
        row[c] = pos + 1u;
        if (pos < a.nnz) {
          at_idx[pos] = r;
          at_val[pos] = a.val[t];
        }
      }
    }
    wave_mem_wait();  // the next row's counters see this row's stores
  }
}

// First position in idx[lo, hi) whose column is at least c.
__device__ __forceinline__ uint32_t lower_bound_u32(const uint32_t *__restrict__ idx, uint32_t lo,
                                                    uint32_t hi, uint32_t c) {
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (idx[mid] < c)
      lo = mid + 1u;
    else
      hi = mid;
  }
  return lo;
}

// A row's columns are below q and strictly ascending (flags otherwise).
__device__ __forceinline__ uint32_t check_row(const Csr &a, uint32_t lo, uint32_t hi, uint32_t q,
                                              uint32_t lane) {
  uint32_t flags = 0;
  for (uint32_t t = lo + lane; t < hi; t += kWave) {
    const uint32_t c = a.idx[t];
    if (c >= q || (t + 1u < hi && a.idx[t + 1u] <= c)) flags |= kFlagBadIndex;
  }
  return flags;
}

// Entries per row of X + Y into cnt[r] (the caller's row pointer + 1).
__global__ void __launch_bounds__(kSpWaves * kWave)
    csr_add_count_kernel(Csr x, Csr y, uint32_t m, uint32_t q, uint32_t *__restrict__ cnt,
                         uint32_t *__restrict__ status) {
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * kSpWaves + wib; r < m; r += gridDim.x * kSpWaves) {
    uint32_t x0, x1, y0, y1;
    // both ranges are always read: a malformed row of one operand leaves the
    // other's range intact (and its own empty)
    const bool x_ok = sp_row(x, r, x0, x1), y_ok = sp_row(y, r, y0, y1);
    if (!x_ok || !y_ok) flags |= kFlagBadIndex;
    flags |= check_row(x, x0, x1, q, lane) | check_row(y, y0, y1, q, lane);
    // common columns: the shorter row's entries searched in the longer row
    const bool xs = x1 - x0 <= y1 - y0;
    const Csr &sm = xs ? x : y;
    const Csr &lg = xs ? y : x;
    const uint32_t s0 = xs ? x0 : y0, s1 = xs ? x1 : y1, l0 = xs ? y0 : x0, l1 = xs ? y1 : x1;
    uint32_t common = 0;
    for (uint32_t t = s0 + lane; t < s1; t += kWave) {
      const uint32_t c = sm.idx[t];
      const uint32_t pos = lower_bound_u32(lg.idx, l0, l1, c);
      if (pos < l1 && lg.idx[pos] == c) ++common;
    }
    common = wave_sum_u32(common);
    if (lane == 0) cnt[r] = (x1 - x0) + (y1 - y0) - common;
  }
  if (flags != 0) atomicOr(status, flags);
}

// Columns and values of alpha X + beta Y into the rows the count pass sized:
// alpha x and beta y are each rounded to f32, then their sum (no fused form).
__global__ void __launch_bounds__(kSpWaves * kWave)
    csr_add_fill_kernel(float alpha, Csr x, float beta, Csr y, uint32_t m,
                        const uint32_t *__restrict__ c_ptr, uint32_t *__restrict__ c_idx,
                        float *__restrict__ c_val, uint64_t c_cap, uint32_t *__restrict__ status) {
  // more entries than the output arrays hold: nothing is written
  if (c_ptr[m] > c_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, kFlagOutputTooLarge);
    return;
  }
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * kSpWaves + wib; r < m; r += gridDim.x * kSpWaves) {
    const uint32_t base = c_ptr[r], end = c_ptr[r + 1];
    const uint32_t cnt = end >= base ? end - base : 0u;
    if (cnt > 0 && (c_idx == nullptr || c_val == nullptr)) {  // no output arrays given
      flags |= kFlagBadIndex;
      continue;
    }
    uint32_t x0, x1, y0, y1;
    // both ranges are always read: a malformed row of one operand leaves the
    // other's range intact (and its own empty)
    const bool x_ok = sp_row(x, r, x0, x1), y_ok = sp_row(y, r, y0, y1);
    if (!x_ok || !y_ok) flags |= kFlagBadIndex;
    // place of an entry in the merged row: its rank in its own row, plus the
    // columns below it in the other row, less the common columns below it
    // (both rows ascending: the matched entries before it in its own row)
    uint32_t common = 0;
    for (uint32_t b = x0; b < x1; b += kWave) {
      const uint32_t t = b + lane;
      uint32_t p = y0;
      bool both = false;
      if (t < x1) {
        p = lower_bound_u32(y.idx, y0, y1, x.idx[t]);
        both = p < y1 && y.idx[p] == x.idx[t];
      }
      const uint32_t before = common + wave_excl_scan_u32(both ? 1u : 0u, lane);
      common += wave_sum_u32(both ? 1u : 0u);
      if (t < x1) {
        const float ax = __fmul_rn(alpha, x.val[t]);
        const float v = both ? __fadd_rn(ax, __fmul_rn(beta, y.val[p])) : ax;
        const uint32_t pos = (t - x0) + (p - y0) - before;
        if (pos < cnt) {
          c_idx[(size_t)base + pos] = x.idx[t];
          c_val[(size_t)base + pos] = v;
        }
      }
    }
    uint32_t common_y = 0;
    for (uint32_t b = y0; b < y1; b += kWave) {
      const uint32_t t = b + lane;
      uint32_t p = x0;
      bool both = false;
      if (t < y1) {
        p = lower_bound_u32(x.idx, x0, x1, y.idx[t]);
        both = p < x1 && x.idx[p] == y.idx[t];
      }
      const uint32_t before = common_y + wave_excl_scan_u32(both ? 1u : 0u, lane);
      common_y += wave_sum_u32(both ? 1u : 0u);
      if (t < y1 && !both) {  // a column stored in both was written from X's side
        const uint32_t pos = (t - y0) + (p - x0) - before;
        if (pos < cnt) {
          c_idx[(size_t)base + pos] = y.idx[t];
          c_val[(size_t)base + pos] = __fmul_rn(beta, y.val[t]);
        }
      }
    }
    if ((x1 - x0) + (y1 - y0) - common != cnt || common_y != common)
      flags |= kFlagBadIndex;  // not the count pass's pointers, or rows not ascending
  }
  if (flags != 0) atomicOr(status, flags);
}

// The k x n matrix with one entry per row (row c: column pick[c], value v):
// its row pointer is 0 .. k and every value is v.
__global__ void __launch_bounds__(256)
    vertex_rows_kernel(uint32_t k, float v, uint32_t *__restrict__ ptr, float *__restrict__ val) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c <= k) ptr[c] = c;
  if (c < k) val[c] = v;
}

// The A update's returned columns as A^T (n x k CSR), pass 1: atoms with a
// non-zero weight per cell into cnt[j] (the caller's row pointer + 1).
__global__ void __launch_bounds__(256)
    atoms_count_kernel(const uint32_t *__restrict__ atom_idx, const float *__restrict__ atom_val,
                       const uint32_t *__restrict__ atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                       uint32_t *__restrict__ cnt, uint32_t *__restrict__ status) {
  const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  uint32_t flags = 0;
  uint32_t c = atom_cnt[j];
  if (c > cap) {
    flags |= kFlagBadIndex;
    c = cap;
  }
  const size_t row = (size_t)j * cap;
  uint32_t m = 0;
  for (uint32_t s = 0; s < c; ++s) {
    if (atom_val[row + s] == 0.0f) continue;
    if (atom_idx[row + s] >= k)
      flags |= kFlagBadIndex;
    else
      ++m;
  }
  cnt[j] = m;
  if (flags != 0) atomicOr(status, flags);
}

// Pass 2: one wave per cell; each kept atom goes to its rank among the
// cell's kept atoms by column (the columns of one cell's atoms are unique).
__global__ void __launch_bounds__(kSpWaves * kWave)
    atoms_fill_kernel(const uint32_t *__restrict__ atom_idx, const float *__restrict__ atom_val,
                      const uint32_t *__restrict__ atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                      const uint32_t *__restrict__ c_ptr, uint32_t *__restrict__ at_idx,
                      float *__restrict__ at_val, uint32_t *__restrict__ status) {
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * kSpWaves + wib; r < n; r += gridDim.x * kSpWaves) {
    const uint32_t base = c_ptr[r], end = c_ptr[r + 1];
    const uint32_t cnt = end >= base ? end - base : 0u;
    if (cnt > 0 && (at_idx == nullptr || at_val == nullptr)) {  // no output arrays given
      flags |= kFlagBadIndex;
      continue;
    }
    const uint32_t c = min(atom_cnt[r], cap);
    const uint32_t *__restrict__ ri = atom_idx + (size_t)r * cap;
    const float *__restrict__ rv = atom_val + (size_t)r * cap;
    uint32_t kept = 0;
    for (uint32_t s0 = 0; s0 < c; s0 += kWave) {
      const uint32_t s = s0 + lane;
      const uint32_t mi = s < c ? ri[s] : 0xffffffffu;
      const float mv = s < c ? rv[s] : 0.0f;
      const bool mine = s < c && mv != 0.0f && mi < k;
      uint32_t rank = 0, same = 0;
      for (uint32_t t = 0; t < c; ++t) {  // every lane reads the same atom
        const uint32_t it = ri[t];
        if (rv[t] != 0.0f && it < k) {
          rank += it < mi ? 1u : 0u;
          same += it == mi ? 1u : 0u;
        }
      }
      if (mine && same != 1u) flags |= kFlagBadIndex;  // a column twice in one cell
      if (mine && rank < cnt) {
        at_idx[(size_t)base + rank] = mi;
        at_val[(size_t)base + rank] = mv;
      }
      kept += wave_sum_u32(mine ? 1u : 0u);
    }
    if (kept != cnt) flags |= kFlagBadIndex;  // not the count pass's row pointer
  }
  if (flags != 0) atomicOr(status, flags);
}

// <X, Y> row by row: each X entry is looked up in Y's (ascending) row.
__global__ void __launch_bounds__(256)
    dot_rows_kernel(Csr x, Csr y, uint32_t m, double *__restrict__ part,
                    uint32_t *__restrict__ status) {
  __shared__ double red[256 / kWave];
  const uint32_t lane = lane_id(), wib = threadIdx.x / kWave;
  const uint32_t wpb = blockDim.x / kWave;
  double s = 0.0;
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * wpb + wib; r < m; r += gridDim.x * wpb) {
    uint32_t x0, x1, y0, y1;
    // both ranges are always read: a malformed row of one operand leaves the
    // other's range intact (and its own empty)
    const bool x_ok = sp_row(x, r, x0, x1), y_ok = sp_row(y, r, y0, y1);
    if (!x_ok || !y_ok) flags |= kFlagBadIndex;
    for (uint32_t t = x0 + lane; t < x1; t += kWave) {
      const uint32_t c = x.idx[t];
      uint32_t lo = y0, hi = y1;
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2u;
        if (y.idx[mid] < c)
          lo = mid + 1u;
        else
          hi = mid;
      }
      if (lo < y1 && y.idx[lo] == c) s += (double)x.val[t] * (double)y.val[lo];
    }
  }
  s = wave_sum_f64(s);
  if (lane == 0) red[wib] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (uint32_t w = 0; w < wpb; ++w) t += red[w];
    part[blockIdx.x] = t;
  }
  if (flags != 0) atomicOr(status, flags);
}

// *acc += alpha * (sum of the block partials, in block order).
__global__ void __launch_bounds__(256)
    dot_final_kernel(const double *__restrict__ part, uint32_t nb, double alpha,
                     double *__restrict__ acc) {
  __shared__ double red[256];
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (nb + 255u) / 256u;
  double s = 0.0;
  for (uint32_t i = tid * per; i < min(nb, (tid + 1) * per); ++i) s += part[i];
  red[tid] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (uint32_t i = 0; i < 256; ++i) t += red[i];
    *acc += alpha * t;
  }
}

// Blocks for a row-per-wave kernel: as many as stay resident together (the
// rows are dealt out in a grid stride), never more than the rows need.
uint32_t sp_blocks(uint32_t m, const DeviceInfo &dev, int resident_per_cu) {
  const uint64_t want = ((uint64_t)m + kSpWaves - 1) / kSpWaves;
  const uint64_t cap = (uint64_t)dev.cus * (uint64_t)(resident_per_cu > 0 ? resident_per_cu : 1);
  return (uint32_t)(want < cap ? (want > 0 ? want : 1) : cap);
}

template <class K>
int resident_blocks(K kernel, int &cache) {
  if (cache == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kSpWaves * kWave, 0) !=
            hipSuccess ||
        nb <= 0)
      nb = 4;
    cache = nb;
  }
  return cache;
}

int g_count_resident = 0, g_fill_resident = 0;

// Blocks of the heavy-row kernels: two per CU (the fill kernel's LDS holds
// one), never more than the rows.
uint32_t heavy_blocks(uint32_t m, const DeviceInfo &dev) {
  const uint64_t cap = 2ull * (uint64_t)(dev.cus > 0 ? dev.cus : 1);
  return (uint32_t)(m < cap ? (m > 0 ? m : 1) : cap);
}

}  // namespace

uint32_t tr_blocks(uint32_t m, uint32_t q) {
  uint64_t nb = ((uint64_t)m + 255u) / 256u;
  if (nb > kTrMaxBlocks) nb = kTrMaxBlocks;
  const uint64_t by_table = kTrTableBytes / (4ull * (q > 0 ? q : 1));
  if (nb > by_table) nb = by_table;
  return (uint32_t)(nb > 0 ? nb : 1);
}

static size_t tr_table_bytes(uint32_t m, uint32_t q) {
  return align_up((size_t)tr_blocks(m, q) * q * sizeof(uint32_t), 256);
}

static size_t scan_bytes(uint32_t count) {
  return align_up(((size_t)scan_tiles(count) + 1) * sizeof(uint64_t), 256);
}

size_t transpose_workspace(uint32_t m, uint32_t q) { return tr_table_bytes(m, q) + scan_bytes(q); }

size_t matmul_workspace(uint32_t m) { return scan_bytes(m); }

// The rows pass's bitmaps (m x ceil(q / 32) words), then its list of rows
// with more than one value window (a count, then the rows).
static size_t matmul_bitmap_bytes(uint32_t m, uint32_t q) {
  if (q == 0 || q > kSpWinWords * 32u) return 0;  // several column windows: not kept
  return align_up((size_t)m * ((q + 31u) / 32u) * sizeof(uint32_t), 256);
}

size_t matmul_pattern_bytes(uint32_t m, uint32_t q) {
  const size_t bm = matmul_bitmap_bytes(m, q);
  return bm == 0 ? 0 : bm + align_up(((size_t)m + 1) * sizeof(uint32_t), 256);
}

static uint32_t *long_row_list(uint32_t *pattern, uint32_t m, uint32_t q) {
  return pattern == nullptr
             ? nullptr
             : reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(pattern) +
                                            matmul_bitmap_bytes(m, q));
}

size_t dot_workspace() { return kDotBlocks * sizeof(double); }

size_t add_workspace(uint32_t m) { return scan_bytes(m); }

size_t vertex_workspace(uint32_t k, uint32_t n) {
  return align_up(((size_t)k + 1) * sizeof(uint32_t), 256) + align_up((size_t)k * sizeof(float), 256) +
         transpose_workspace(k, n);
}

hipError_t launch_spgemm_count(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                               uint32_t *c_ptr, void *ws, uint32_t *pattern, uint32_t *status,
                               hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  uint32_t *list = long_row_list(pattern, m, q);
  if (list != nullptr) {
    hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(64), 0, stream, list);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (m > 0) {
    const uint32_t nb = sp_blocks(m, dev, resident_blocks(spgemm_count_kernel, g_count_resident));
    hipLaunchKernelGGL(spgemm_count_kernel, dim3(nb), dim3(kSpWaves * kWave), 0,
                       stream, a, b, m, p, q, c_ptr + 1, pattern, list, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (q <= kSpWinWords * 32u && a.nnz >= kHeavyEntries) {
      hipLaunchKernelGGL(spgemm_count_heavy_kernel, dim3(heavy_blocks(m, dev)), dim3(kHvThreads), 0,
                         stream, a, b, m, p, q, c_ptr + 1, pattern, status);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return launch_scan(c_ptr, m, static_cast<uint64_t *>(ws), status, stream);
}

hipError_t launch_spgemm_fill(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                              const uint32_t *c_ptr, uint32_t *c_idx, float *c_val, uint64_t c_cap,
                              const uint32_t *pattern, uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  if (m == 0) return hipSuccess;
  const uint32_t nb = sp_blocks(m, dev, resident_blocks(spgemm_fill_kernel, g_fill_resident));
  hipLaunchKernelGGL(spgemm_fill_kernel, dim3(nb), dim3(kSpWaves * kWave), 0,
                     stream, a, b, m, p, q, c_ptr, c_idx, c_val, c_cap, pattern,
                     long_row_list(const_cast<uint32_t *>(pattern), m, q), status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (q <= kSpWinWords * 32u && a.nnz >= kHeavyEntries) {
    static bool configured = false;  // the kernel's dynamic LDS limit, raised once
    if (!configured) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(&spgemm_fill_heavy_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHvPartBytes);
      if (e != hipSuccess) return e;
      configured = true;
    }
    hipLaunchKernelGGL(spgemm_fill_heavy_kernel, dim3(heavy_blocks(m, dev)), dim3(kHvThreads),
                       kHvPartBytes, stream, a, b, m, p, q, c_ptr, c_idx, c_val, c_cap, pattern,
                       status);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_transpose(Csr a, uint32_t m, uint32_t q, uint32_t *at_ptr, uint32_t *at_idx,
                            float *at_val, void *ws, uint32_t *status, hipStream_t stream) {
  const uint32_t nb = tr_blocks(m, q);
  uint32_t *table = static_cast<uint32_t *>(ws);
  hipError_t e;
  hipLaunchKernelGGL(tr_count_kernel, dim3(nb), dim3(kWave), 0, stream, a, m, q, nb, table,
                     status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const uint32_t cb = (q + 255u) / 256u;
  if (q > 0) {
    hipLaunchKernelGGL(tr_colsum_kernel, dim3(cb), dim3(256), 0, stream, q, nb, table, at_ptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  uint64_t *part = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + tr_table_bytes(m, q));
  if ((e = launch_scan(at_ptr, q, part, status, stream)) != hipSuccess) return e;
  if (q > 0) {
    hipLaunchKernelGGL(tr_base_kernel, dim3(cb), dim3(256), 0, stream, q, nb, table, at_ptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tr_fill_kernel, dim3(nb), dim3(kWave), 0, stream, a, m, q, nb, table,
                     at_idx, at_val);
  return hipGetLastError();
}

int g_add_count_resident = 0, g_add_fill_resident = 0, g_atoms_fill_resident = 0;

hipError_t launch_atoms_count(const uint32_t *atom_idx, const float *atom_val,
                              const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                              uint32_t *at_ptr, void *ws, uint32_t *status, hipStream_t stream) {
  hipError_t e;
  if (n > 0) {
    hipLaunchKernelGGL(atoms_count_kernel, dim3((n + 255u) / 256u), dim3(256), 0, stream, atom_idx,
                       atom_val, atom_cnt, n, k, cap, at_ptr + 1, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_scan(at_ptr, n, static_cast<uint64_t *>(ws), status, stream);
}

hipError_t launch_atoms_fill(const uint32_t *atom_idx, const float *atom_val,
                             const uint32_t *atom_cnt, uint32_t n, uint32_t k, uint32_t cap,
                             const uint32_t *at_ptr, uint32_t *at_idx, float *at_val,
                             uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  if (n == 0) return hipSuccess;
  const uint32_t nb = sp_blocks(n, dev, resident_blocks(atoms_fill_kernel, g_atoms_fill_resident));
  hipLaunchKernelGGL(atoms_fill_kernel, dim3(nb), dim3(kSpWaves * kWave), 0, stream, atom_idx,
                     atom_val, atom_cnt, n, k, cap, at_ptr, at_idx, at_val, status);
  return hipGetLastError();
}

hipError_t launch_add_count(Csr x, Csr y, uint32_t m, uint32_t q, uint32_t *c_ptr, void *ws,
                            uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  if (m > 0) {
    const uint32_t nb = sp_blocks(m, dev, resident_blocks(csr_add_count_kernel, g_add_count_resident));
    hipLaunchKernelGGL(csr_add_count_kernel, dim3(nb), dim3(kSpWaves * kWave), 0, stream, x, y, m,
                       q, c_ptr + 1, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_scan(c_ptr, m, static_cast<uint64_t *>(ws), status, stream);
}

hipError_t launch_add_fill(float alpha, Csr x, float beta, Csr y, uint32_t m, const uint32_t *c_ptr,
                           uint32_t *c_idx, float *c_val, uint64_t c_cap, uint32_t *status,
                           hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  if (m == 0) return hipSuccess;
  const uint32_t nb = sp_blocks(m, dev, resident_blocks(csr_add_fill_kernel, g_add_fill_resident));
  hipLaunchKernelGGL(csr_add_fill_kernel, dim3(nb), dim3(kSpWaves * kWave), 0, stream, alpha, x,
                     beta, y, m, c_ptr, c_idx, c_val, c_cap, status);
  return hipGetLastError();
}

hipError_t launch_vertex(const uint32_t *pick, uint32_t k, uint32_t n, float value, uint32_t *s_ptr,
                         uint32_t *s_idx, float *s_val, void *ws, uint32_t *status,
                         hipStream_t stream) {
  char *w = static_cast<char *>(ws);
  uint32_t *ptr = reinterpret_cast<uint32_t *>(w);
  w += align_up(((size_t)k + 1) * sizeof(uint32_t), 256);
  float *val = reinterpret_cast<float *>(w);
  w += align_up((size_t)k * sizeof(float), 256);
  hipLaunchKernelGGL(vertex_rows_kernel, dim3((k + 1u + 255u) / 256u), dim3(256), 0, stream, k,
                     value, ptr, val);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const Csr rows{ptr, pick, val, k};
  return launch_transpose(rows, k, n, s_ptr, s_idx, s_val, w, status, stream);
}

hipError_t launch_dot(Csr x, Csr y, uint32_t m, double alpha, double *acc, void *ws,
                      uint32_t *status, hipStream_t stream) {
  // <X, Y> = <Y, X>: walk the operand with fewer entries, search the other
  if (x.nnz > y.nnz) {
    const Csr t = x;
    x = y;
    y = t;
  }
  double *part = static_cast<double *>(ws);
  hipLaunchKernelGGL(dot_rows_kernel, dim3(kDotBlocks), dim3(256), 0, stream, x, y, m, part,
                     status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dot_final_kernel, dim3(1), dim3(256), 0, stream, part, kDotBlocks, alpha,
                     acc);
  return hipGetLastError();
}

}  // namespace seacells
