// B-gradient argmin and B step (`fw_argmin_b` and `reduce_argmin_blocks` on
// the source page bixverse-rs 0.6.4, seacells_kernels.rs).
//
//   G[i, c] = sum_m K2B[i, m] AAt[m, c] - K2At[i, c]        (never stored)
//   out[c]  = (min_i G[i, c], lowest i attaining it),  gap = sum B * G
//
// Work unit = (row range, column slice). A wave owns one unit at a time:
// per row it scatters the AAt rows named by the row's K2B entries into a
// dense slice accumulator in LDS (the columns of one AAt row are unique, so
// one scatter instruction never collides), subtracts the K2At row, adds the
// row's B . G term, then folds the slice into running (min, row) pairs held
// in registers, 4 accumulator words per float4 chunk, and clears the slice.
// Rows run in ascending order under a strict `<`, so the lowest row wins a
// tie inside a unit. The unit writes one (order-preserving f32 key << 32 |
// row) per column, which makes "lower value, then lower row" a plain u64
// minimum for the reduce stages, and a stamp with the call's epoch.
//
// Each call first copies AAt into the layout its gather reads:
// - one slice (k <= 2048): every row padded to whole 64-entry chunks of
//   (accumulator byte offset, value); a whole wave gathers one chunk, four
//   runs in flight;
// - narrow slices (k > 2048, at most 1024 columns and ~3.75 MB of AAt
//   each, so one XCD's slices stay in its L2): every (row, slice) run in
//   chunks of 32 (16-bit accumulator position, f32 value); the row's chunks
//   are dealt alternately to the two half-waves, each with its own
//   accumulator. Each slice places its columns in the accumulator in an
//   order of their own (power iteration clustering of AAt), which keeps
//   the scatter's LDS bank conflicts down.
// A segment table seg[s, m] = first position of AAt row m with column
// >= s * slice_w hands each slice its run of every AAt row, and a row-slice
// table does the same for K2At's rows.
//
// The reduce is two kernels: stage 1 takes u64 minima over groups of row
// ranges (coalesced over columns) and checks every stamp and row it
// consumes; stage 2 finishes each column, checks that the winning row is
// below n, and sums the gap partials in a fixed order.
#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kBThreads = 256;
constexpr uint32_t kBUnitsTarget = 8192;
constexpr uint32_t kBMaxS4 = 8;
constexpr uint32_t kReduceCols = 64;  // columns per stage-1 block (one per lane)
constexpr uint32_t kMaxChunks = 64;

constexpr uint32_t kGatherRows = 4;  // AAt runs whose loads are in flight together
constexpr uint32_t kXcds = 8;        // MI355X: 8 XCDs of 32 CUs, each with its own 4 MB L2
constexpr size_t kSliceAatBytes = 15u << 18;  // AAt bytes (at 8 per entry) per slice: 3.75 MB
constexpr uint32_t kSliceCols = 1024;          // columns per slice when k is sliced
constexpr uint32_t kSlicedRowBlocks = 16384;  // row ranges per slice when k is sliced
constexpr uint64_t kKeysBudget = 1ull << 31;  // bytes of partial keys beyond which row ranges shrink
constexpr uint32_t kAccPad = 32;             // dummy slots after each dual accumulator
constexpr uint32_t kStageSlots = kWave + 8;  // LDS staging per wave, in 16-byte slots
constexpr uint32_t kChunkSlots = 2 * kStageSlots - 16;  // (chunk, value) pairs per window
constexpr uint32_t kWalkSteps = 32;   // random-walk steps behind the in-slice column order
constexpr uint32_t kOrderMax = 2048;  // widest slice the order kernel sorts
constexpr uint32_t kBalanceMax = 4096;  // most slices the XCD assignment sorts
constexpr uint32_t kHistRowStep = 16;   // K2B rows sampled for the column histogram

// base[byte_off / 4] with a 32-bit byte offset from a wave-uniform base (the
// array must hold fewer than 2^30 entries)
template <typename T>
__device__ __forceinline__ T load_at(const T *__restrict__ base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}
// the key a unit leaves in a column where no row gave a value below +inf
constexpr uint64_t kNoValueKey = ((uint64_t)0xff800000u << 32) | 0xffffffffull;

// acc[c] += v (LDS read, add, write). One wave's LDS operations execute in
// issue order and the columns of one row are unique, so the sum order per
// column is the program order.
__device__ __forceinline__ void lds_add(float *p, float v) { *p = *p + v; }

__device__ __forceinline__ uint64_t pack_key(float v, uint32_t row) {
  return ((uint64_t)f32_order(v) << 32) | (uint64_t)row;
}

__device__ __forceinline__ bool row_ok(const Csr &m, uint32_t r, uint32_t &lo, uint32_t &hi) {
  lo = m.ptr[r];
  hi = m.ptr[r + 1];
  if (hi > m.nnz || lo > hi) {
    lo = hi = 0;
    return false;
  }
  return true;
}

__global__ void __launch_bounds__(256)
    seg_table_kernel(Csr aat, uint32_t k, uint32_t slice_w, uint32_t n_slices,
                     uint32_t *__restrict__ seg) {
  // slice-major: seg[s * k + m], so the lookups of one slice share lines
  const uint64_t total = (uint64_t)k * ((uint64_t)n_slices + 1);
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint32_t s = (uint32_t)(e / k);
    const uint32_t m = (uint32_t)(e - (uint64_t)s * k);
    uint32_t lo, hi;
    row_ok(aat, m, lo, hi);
    if (s == n_slices) {
      seg[e] = hi;
      continue;
    }
    const uint32_t target = s * slice_w;
    while (lo < hi) {  // first position with column >= target
      const uint32_t mid = lo + (hi - lo) / 2;
      if (aat.idx[mid] < target)
        lo = mid + 1;
      else
        hi = mid;
    }
    seg[e] = lo;
  }
}

// Row-slice table of an n x k operand whose rows are read slice by slice
// (K2At): rs[i * (n_slices + 1) + s] = first position of row i with column
// >= s * slice_w, rs[i * (n_slices + 1) + n_slices] = the row's end, so the
// unit of slice s reads only [rs[.. s], rs[.. s + 1]) of the row. Every
// entry lies inside its row (a binary search of the row, whatever its
// order); a malformed row gets an empty run everywhere and raises BAD_INDEX.
__global__ void __launch_bounds__(256)
    row_slice_kernel(Csr m, uint32_t n_rows, uint32_t slice_w, uint32_t n_slices,
                     uint32_t *__restrict__ rs, uint32_t *__restrict__ status) {
  const uint64_t per = (uint64_t)n_slices + 1;
  const uint64_t total = (uint64_t)n_rows * per;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t flags = 0;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint32_t i = (uint32_t)(e / per);
    const uint32_t s = (uint32_t)(e - (uint64_t)i * per);
    uint32_t lo, hi;
    if (!row_ok(m, i, lo, hi)) flags |= kFlagBadIndex;
    if (s == n_slices) {
      rs[e] = hi;
      continue;
    }
    const uint32_t target = s * slice_w;
    while (lo < hi) {  // first position with column >= target
      const uint32_t mid = lo + (hi - lo) / 2;
      if (m.idx[mid] < target)
        lo = mid + 1;
      else
        hi = mid;
    }
    rs[e] = lo;
  }
  if (flags != 0) atomicOr(status, flags);
}

// ---------------------------------------------------------------------------
// In-slice column order (narrow slices). Where a column sits in the slice
// accumulator sets the LDS bank conflicts of the scatter: the runs of AAt
// are neighbour sets of archetypes, so placing archetypes that share
// neighbours next to each other turns a run's columns into few stretches of
// consecutive words (the chunked copy stores each run in position order).
// It also decides which chunk of its run, and so which of the two half-wave
// accumulators, each term goes to; every sum stays a fixed function of the
// operands. The order comes from power iteration clustering (Lin
// and Cohen, "Power Iteration Clustering", ICML 2010): a start vector of
// hashed column numbers, kWalkSteps steps of the random walk over AAt,
// x <- D^-1 AAt x, which averages x within groups of archetypes that share
// much AAt mass long before it averages across groups; each slice then sorts
// its columns by x (column number on ties). Every step is a fixed-order
// computation, so the order is a function of AAt alone.

// the start vector: a 32-bit integer mix of the column number (the
// murmur3 finaliser), scaled to [0, 1)
__device__ __forceinline__ float walk_start(uint32_t c) {
  uint32_t x = c * 0x9E3779B1u + 1u;
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return (float)x * 0x1p-32f;
}

// One step, one wave per row m: y[m] = sum_c AAt[m,c] x[c] / sum_c AAt[m,c]
// (x = nullptr: the start vector). A row without mass, or malformed (the
// chunked copy reports those), keeps its value.
__global__ void __launch_bounds__(256)
    col_walk_kernel(Csr aat, uint32_t k, const float *__restrict__ x, float *__restrict__ y) {
  const uint32_t lane = lane_id();
  const uint32_t nw = gridDim.x * (blockDim.x / kWave);
  for (uint32_t m = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; m < k; m += nw) {
    uint32_t lo, hi;
    if (!row_ok(aat, m, lo, hi)) lo = hi = 0;
    float sx = 0.0f, sv = 0.0f;
    // four entries per lane in flight (their loads do not wait on each other)
    for (uint32_t q0 = lo + lane; q0 < hi; q0 += 4 * kWave) {
      uint32_t c[4];
      float v[4], xc[4];
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t q = q0 + j * kWave;
        c[j] = q < hi ? aat.idx[q] : k;
        v[j] = q < hi ? aat.val[q] : 0.0f;
      }
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j)
        xc[j] = c[j] < k ? (x != nullptr ? x[c[j]] : walk_start(c[j])) : 0.0f;
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j) {
        if (c[j] < k) {
          sx = __builtin_fmaf(v[j], xc[j], sx);
          sv += v[j];
        }
      }
    }
    sx = wave_sum_f32(sx);
    sv = wave_sum_f32(sv);
    if (lane == 0) {
      const float own = x != nullptr ? x[m] : walk_start(m);
      const float r = sx / sv;
      y[m] = (sv > 0.0f && r == r) ? r : own;
    }
  }
}

// One block per slice: sort the slice's columns by (order key of x, column)
// in LDS (bitonic, a power of two >= the slice width, <= kOrderMax), then
// cpos[c] = position of column c in its slice, pcol[s * slice_w + p] =
// slice-local column at position p. Every column gets a position below the
// slice's width (the padding keys sort last).
__global__ void __launch_bounds__(1024)
    slice_order_kernel(const float *__restrict__ x, uint32_t k, uint32_t slice_w,
                       uint16_t *__restrict__ cpos, uint16_t *__restrict__ pcol) {
  __shared__ uint64_t key[kOrderMax];
  const uint32_t s = blockIdx.x;
  const uint32_t c0 = s * slice_w;
  const uint32_t cw = (k - c0) < slice_w ? (k - c0) : slice_w;
  uint32_t len = 1;
  while (len < cw) len <<= 1;
  for (uint32_t j = threadIdx.x; j < len; j += blockDim.x)
    key[j] = j < cw ? ((uint64_t)f32_order(x[c0 + j]) << 32) | j : ~0ull;
  __syncthreads();
  for (uint32_t size = 2; size <= len; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t j = threadIdx.x; j < len; j += blockDim.x) {
        const uint32_t o = j ^ stride;
        if (o > j) {
          const bool up = (j & size) == 0;
          const uint64_t a = key[j], b = key[o];
          if ((a > b) == up) key[j] = b, key[o] = a;
        }
      }
      __syncthreads();
    }
  }
  for (uint32_t p = threadIdx.x; p < cw; p += blockDim.x) {
    const uint32_t j = (uint32_t)key[p];
    cpos[c0 + j] = (uint16_t)p;
    pcol[(size_t)s * slice_w + p] = (uint16_t)j;
  }
}

// ---------------------------------------------------------------------------
// Which XCD owns which slice (narrow slices, n_slices > kXcds). An XCD
// gathers only its own slices (their AAt stays in its L2), so the kernel
// ends when the XCD with the most work does. The work of slice s is close
// to sum_m ref(m) nq(m, s): ref(m) = the K2B entries with column m (counted
// on every kHistRowStep-th row), nq(m, s) = the chunks of AAt row m in slice
// s (from the run table). The slices are dealt longest first, each to the
// XCD with the least work so far (ties: the lower XCD). Only the speed
// depends on the assignment: every unit writes its own partials.

// hist[m] += 1 for every entry of column m in the sampled rows; one wave per
// row, grid-stride. With k <= kHistLds each block counts into a histogram
// of its own in LDS and adds its non-zero counts to hist once (few device
// atomics); otherwise every entry is a device atomic.
constexpr uint32_t kHistLds = 16384;    // columns an LDS histogram holds (64 KB)
constexpr uint32_t kHistBlocks = 256;   // blocks of the LDS-histogram launch
__global__ void __launch_bounds__(256)
    ref_hist_kernel(Csr k2b, uint32_t n, uint32_t k, uint32_t *__restrict__ hist) {
  extern __shared__ uint32_t lh[];
  const uint32_t lane = lane_id();
  const bool local = k <= kHistLds;
  if (local) {
    for (uint32_t m = threadIdx.x; m < k; m += blockDim.x) lh[m] = 0u;
    __syncthreads();
  }
  const uint32_t nw = gridDim.x * (blockDim.x / kWave);
  for (uint32_t j = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
       (uint64_t)j * kHistRowStep < n; j += nw) {
    uint32_t lo, hi;
    if (!row_ok(k2b, j * kHistRowStep, lo, hi)) continue;
    for (uint32_t q = lo + lane; q < hi; q += kWave) {
      const uint32_t m = k2b.idx[q];
      if (m < k) atomicAdd(local ? lh + m : hist + m, 1u);
    }
  }
  if (local) {
    __syncthreads();
    for (uint32_t m = threadIdx.x; m < k; m += blockDim.x)
      if (lh[m] != 0u) atomicAdd(hist + m, lh[m]);
  }
}

// One block per slice: swork[s] = sum_m hist[m] * nq(m, s)
__global__ void __launch_bounds__(256)
    slice_work_kernel(const uint32_t *__restrict__ hist, const uint32_t *__restrict__ pa_seg,
                      uint32_t k, uint64_t *__restrict__ swork) {
  __shared__ uint64_t part[256];
  const uint32_t s = blockIdx.x;
  const uint32_t *ps = pa_seg + (size_t)s * k;
  uint64_t sum = 0;
  for (uint32_t m = threadIdx.x; m < k; m += blockDim.x) {
    const uint32_t q0 = ps[m], q1 = ps[m + 1];
    sum += (uint64_t)hist[m] * (q1 > q0 ? q1 - q0 : 0u);
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  for (uint32_t off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) swork[s] = part[0];
}

// One block: sort the slices by work (most first, lower slice on ties),
// deal them longest first, then list each XCD's slices in that order.
__global__ void __launch_bounds__(1024)
    xcd_assign_kernel(const uint64_t *__restrict__ swork, uint32_t n_slices,
                      uint32_t *__restrict__ xcd_off, uint32_t *__restrict__ xcd_list) {
  __shared__ uint64_t key[kBalanceMax];
  __shared__ uint8_t owner[kBalanceMax];
  uint32_t len = 1;
  while (len < n_slices) len <<= 1;
  for (uint32_t j = threadIdx.x; j < len; j += blockDim.x) {
    uint64_t kj = ~0ull;
    if (j < n_slices) {
      const uint64_t w = swork[j] >> 8;  // 24 bits of headroom; the order is what matters
      const uint32_t w32 = w > 0xffffffffull ? 0xffffffffu : (uint32_t)w;
      kj = ((uint64_t)(0xffffffffu - w32) << 32) | j;
    }
    key[j] = kj;
  }
  __syncthreads();
  for (uint32_t size = 2; size <= len; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t j = threadIdx.x; j < len; j += blockDim.x) {
        const uint32_t o = j ^ stride;
        if (o > j) {
          const bool up = (j & size) == 0;
          const uint64_t a = key[j], b = key[o];
          if ((a > b) == up) key[j] = b, key[o] = a;
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    uint64_t load[kXcds];
    uint32_t count[kXcds];
    for (uint32_t x = 0; x < kXcds; ++x) load[x] = 0, count[x] = 0;
    for (uint32_t r = 0; r < n_slices; ++r) {
      const uint32_t s = (uint32_t)key[r];
      uint32_t best = 0;
      for (uint32_t x = 1; x < kXcds; ++x)
        if (load[x] < load[best]) best = x;
      owner[r] = (uint8_t)best;
      load[best] += swork[s] + 1;  // + 1: an empty slice still costs its units
      ++count[best];
    }
    uint32_t at = 0;
    for (uint32_t x = 0; x < kXcds; ++x) {
      xcd_off[x] = at;
      at += count[x];
      count[x] = xcd_off[x];
    }
    xcd_off[kXcds] = at;
    for (uint32_t r = 0; r < n_slices; ++r) xcd_list[count[owner[r]]++] = (uint32_t)key[r];
  }
}

// ---------------------------------------------------------------------------
// Padded copy of AAt per slice. The run of AAt row m inside slice s (all of
// the row with one slice) takes ceil(len / ch) chunks of ch entries
// (byte offset of the column in the slice accumulator, value); positions
// past the run point at the dummy slot of the lane that reads them (W +
// position % ch) with value 0, so a gather needs no bounds test and no
// column arithmetic. Chunk 0 is padding only: empty runs read it.
// pa_seg[s * k + m] = first chunk of the run; pa_seg[n_slices * k] = end.

__device__ __forceinline__ uint32_t run_of(const Csr &aat, const uint32_t *seg, uint32_t k,
                                           uint32_t s, uint32_t m, uint32_t &lo, bool &bad) {
  uint32_t hi;
  bad = false;
  if (seg != nullptr) {
    lo = seg[(size_t)s * k + m];
    hi = seg[(size_t)(s + 1) * k + m];
    if (hi < lo) hi = lo;
  } else {
    bad = !row_ok(aat, m, lo, hi);
  }
  return hi - lo;
}

// The run table: chunk counts of every run and their exclusive prefix sum
// (64-bit, checked against the bound the workspace was sized for; past it
// every run is left empty and BAD_INDEX is raised). Three kernels over
// blocks of kScanRuns runs (4 consecutive runs per thread): the blocks'
// counts and sums, a scan of the sums (one block), then each block's
// offsets. bsum holds one sum per block, then the total.
constexpr uint32_t kScanRuns = 1024;

// Exclusive prefix of v over a block of 256 threads; *total gets the sum.
__device__ __forceinline__ uint64_t block_excl_scan_256(uint64_t v, uint64_t *red,
                                                        uint64_t *total) {
  const uint32_t lane = lane_id(), w = threadIdx.x / kWave;
  uint64_t incl = v;
#pragma unroll
  for (uint32_t off = 1; off < kWave; off <<= 1) {
    const uint64_t u = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += u;
  }
  if (lane == kWave - 1) red[w] = incl;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (uint32_t x = 0; x < 4; ++x) {
    if (x < w) before += red[x];
    all += red[x];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__global__ void __launch_bounds__(256)
    pa_count_kernel(Csr aat, const uint32_t *__restrict__ seg, uint32_t k, uint32_t n_slices,
                    uint32_t ch, uint32_t *__restrict__ pa_seg, uint64_t *__restrict__ bsum,
                    uint32_t *__restrict__ status) {
  __shared__ uint64_t red[4];
  const uint64_t total_runs = (uint64_t)k * n_slices;
  const uint64_t e0 = (uint64_t)blockIdx.x * kScanRuns + threadIdx.x * 4u;
  uint64_t sum = 0;
  bool bad_any = false;
  for (uint32_t j = 0; j < 4; ++j) {
    const uint64_t e = e0 + j;
    if (e >= total_runs) break;
    const uint32_t s = (uint32_t)(e / k), m = (uint32_t)(e - (uint64_t)s * k);
    uint32_t lo;
    bool bad;
    const uint32_t len = run_of(aat, seg, k, s, m, lo, bad);
    bad_any |= bad;
    const uint32_t c = (len + ch - 1) / ch;
    pa_seg[e] = c;
    sum += c;
  }
  uint64_t all;
  block_excl_scan_256(sum, red, &all);
  if (threadIdx.x == 0) bsum[blockIdx.x] = all;
  if (bad_any) atomicOr(status, kFlagBadIndex);
}

// One block: exclusive scan of the nb block sums in place; bsum[nb] = the
// total with the padding chunk 0, also written after the last run.
__global__ void __launch_bounds__(256)
    pa_bscan_kernel(uint64_t *__restrict__ bsum, uint32_t nb, uint64_t total_runs,
                    uint64_t pa_chunks, uint32_t *__restrict__ pa_seg,
                    uint32_t *__restrict__ status) {
  __shared__ uint64_t red[4];
  uint64_t carry = 0;
  for (uint32_t b0 = 0; b0 < nb; b0 += 256) {
    const uint32_t b = b0 + threadIdx.x;
    const uint64_t v = b < nb ? bsum[b] : 0u;
    uint64_t all;
    const uint64_t ex = block_excl_scan_256(v, red, &all);
    if (b < nb) bsum[b] = carry + ex;
    carry += all;
  }
  if (threadIdx.x == 0) {
    const uint64_t total = carry + 1;  // + the padding chunk 0
    const bool overflow = total > pa_chunks;
    bsum[nb] = total;
    pa_seg[total_runs] = overflow ? 1u : (uint32_t)total;
    if (overflow) atomicOr(status, kFlagBadIndex);
  }
}

__global__ void __launch_bounds__(256)
    pa_offs_kernel(uint32_t *__restrict__ pa_seg, const uint64_t *__restrict__ bsum,
                   uint32_t nb, uint64_t total_runs, uint64_t pa_chunks) {
  __shared__ uint64_t red[4];
  const uint64_t e0 = (uint64_t)blockIdx.x * kScanRuns + threadIdx.x * 4u;
  uint32_t c[4];
  uint64_t sum = 0;
  for (uint32_t j = 0; j < 4; ++j) {
    c[j] = e0 + j < total_runs ? pa_seg[e0 + j] : 0u;
    sum += c[j];
  }
  uint64_t all;
  uint64_t at = 1 + bsum[blockIdx.x] + block_excl_scan_256(sum, red, &all);
  const bool overflow = bsum[nb] > pa_chunks;
  for (uint32_t j = 0; j < 4; ++j) {
    if (e0 + j >= total_runs) break;
    pa_seg[e0 + j] = overflow ? 1u : (uint32_t)at;
    at += c[j];
  }
}

// One wave per run: its entries, then padding; chunk 0 as padding.
__global__ void __launch_bounds__(256)
    pa_fill_kernel(Csr aat, const uint32_t *__restrict__ seg, uint32_t k, uint32_t n_slices,
                   uint32_t slice_w, uint32_t ch, uint32_t w_acc,
                   const uint32_t *__restrict__ pa_seg, uint2 *__restrict__ pa_ent,
                   uint32_t *__restrict__ status) {
  const uint32_t lane = lane_id();
  const uint64_t nw = (uint64_t)gridDim.x * (blockDim.x / kWave);
  const uint64_t total_runs = (uint64_t)k * n_slices;
  const uint64_t first = (uint64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (first == 0)
    for (uint32_t i = lane; i < ch; i += kWave) pa_ent[i] = make_uint2((w_acc + i) * 4u, 0u);
  uint32_t flags = 0;
  for (uint64_t e = first; e < total_runs; e += nw) {
    const uint32_t s = (uint32_t)(e / k), m = (uint32_t)(e - (uint64_t)s * k);
    const uint32_t c0 = s * slice_w;
    const uint32_t cw = (k - c0) < slice_w ? (k - c0) : slice_w;
    const uint32_t q0 = pa_seg[e], q1 = pa_seg[e + 1];
    uint32_t lo;
    bool bad;
    uint32_t len = run_of(aat, seg, k, s, m, lo, bad);
    const uint64_t room = (uint64_t)(q1 - q0) * ch;  // 0 when the runs were left empty
    if (len > room) len = (uint32_t)room;
    for (uint32_t i = lane; i < room; i += kWave) {
      uint2 v = make_uint2((w_acc + i % ch) * 4u, 0u);
      if (i < len) {
        const uint32_t c = aat.idx[lo + i] - c0;
        if (c < cw)
          v = make_uint2(c * 4u, __float_as_uint(aat.val[lo + i]));
        else
          flags |= kFlagBadIndex;
      }
      pa_ent[(size_t)q0 * ch + i] = v;
    }
  }
  if (flags != 0) atomicOr(status, flags);
}

// Chunked copy of AAt for the narrow-slice gather (two half-waves, one run
// each). The run of AAt row m inside slice s takes ceil(len / 32) chunks of
// 32 entries starting at chunk pc_seg[s * k + m] (the chunk table is built by
// the run-table scan with chunks of 32): the accumulator positions of the entries'
// columns (cpos, the in-slice order) as 16-bit words in pc_col and their
// values in pc_val, so one half-wave load reads exactly one 64-byte run of
// positions and one 128-byte run of values. A run's entries are stored in
// ascending position, so each chunk of a long run covers few stretches of
// consecutive accumulator words. Positions past the run hold 0xffff (the
// gather sends it to the lane's dummy slot) and value 0; chunk 0 is all
// padding (empty runs read it). One wave per run: the run's positions go
// into a bitmap of the slice (at most kOrderMax bits, two per lane), and an
// entry's place is the number of set bits below its own. A column outside
// the slice, or one that appears twice, raises BAD_INDEX.
constexpr uint32_t kPcCh = 32;
constexpr uint32_t kOrderWords = kOrderMax / 32;  // bitmap words per wave
static_assert(kOrderWords == kWave, "one bitmap word per lane");

__global__ void __launch_bounds__(256)
    pc_fill_kernel(Csr aat, const uint32_t *__restrict__ seg, uint32_t k, uint32_t n_slices,
                   uint32_t slice_w, const uint32_t *__restrict__ pc_seg,
                   const uint16_t *__restrict__ cpos, uint16_t *__restrict__ pc_col,
                   float *__restrict__ pc_val, uint32_t *__restrict__ status) {
  const uint32_t lane = lane_id();
  const uint64_t nw = (uint64_t)gridDim.x * (blockDim.x / kWave);
  const uint64_t total_runs = (uint64_t)k * n_slices;
  const uint64_t first = (uint64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  __shared__ uint32_t bits_all[4][kOrderWords];
  __shared__ uint32_t below_all[4][kOrderWords];
  uint32_t *bits = bits_all[(threadIdx.x / kWave) & 3u];
  uint32_t *below = below_all[(threadIdx.x / kWave) & 3u];
  if (first == 0 && lane < kPcCh) pc_col[lane] = 0xffffu, pc_val[lane] = 0.0f;
  uint32_t flags = 0;
  for (uint64_t e = first; e < total_runs; e += nw) {
    const uint32_t s = (uint32_t)(e / k), m = (uint32_t)(e - (uint64_t)s * k);
    const uint32_t c0 = s * slice_w;
    const uint32_t cw = (k - c0) < slice_w ? (k - c0) : slice_w;
    const uint32_t q0 = pc_seg[e], q1 = pc_seg[e + 1];
    uint32_t lo;
    bool bad;
    uint32_t len = run_of(aat, seg, k, s, m, lo, bad);
    const uint64_t room = (uint64_t)(q1 - q0) * kPcCh;  // 0 when the runs were left empty
    if (len > room) len = (uint32_t)room;
    float *vals = pc_val + (size_t)q0 * kPcCh;
    uint16_t *cols = pc_col + (size_t)q0 * kPcCh;
    // the run's positions as a bitmap of the slice
    bits[lane] = 0u;
    wave_lds_sync();
    for (uint32_t i = lane; i < len; i += kWave) {
      const uint32_t c = aat.idx[lo + i] - c0;
      if (c < cw) {
        const uint32_t pos = cpos[c0 + c];
        const uint32_t bit = 1u << (pos & 31u);
        if (atomicOr(bits + (pos >> 5), bit) & bit) flags |= kFlagBadIndex;
      } else {
        flags |= kFlagBadIndex;
      }
    }
    wave_lds_sync();
    // set bits below each word, and in all
    const uint32_t own = __builtin_popcount(bits[lane]);
    uint32_t incl = own;
#pragma unroll
    for (uint32_t off = 1; off < kWave; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += v;
    }
    below[lane] = incl - own;
    const uint32_t placed = readlane_u32(incl, kWave - 1);
    wave_lds_sync();
    for (uint32_t i = lane; i < len; i += kWave) {
      const uint32_t c = aat.idx[lo + i] - c0;
      if (c < cw) {
        const uint32_t pos = cpos[c0 + c];
        const uint32_t r =
            below[pos >> 5] + __builtin_popcount(bits[pos >> 5] & ((1u << (pos & 31u)) - 1u));
        cols[r] = (uint16_t)pos;
        vals[r] = aat.val[lo + i];
      }
    }
    for (uint32_t i = placed + lane; i < room; i += kWave) cols[i] = 0xffffu, vals[i] = 0.0f;
    wave_lds_sync();  // the bitmap is cleared for the next run only after every lane used it
  }
  if (flags != 0) atomicOr(status, flags);
}

// kDual: the two half-waves gather different K2B entries into two
// accumulators (for the short AAt runs of narrow slices); each column then
// sums the even-numbered entries of the row in one accumulator and the odd
// ones in the other, each in K2B order, and adds the two at the end.
template <uint32_t S4, bool kDual, uint32_t kPairs>
__global__ void __launch_bounds__(kBThreads)
    fw_b_partials_kernel(Csr k2b, Csr aat, Csr k2at, Csr b, uint32_t n, uint32_t k,
                         uint32_t slice_w, uint32_t n_slices, uint32_t n_row_blocks,
                         const uint32_t *__restrict__ seg, const uint32_t *__restrict__ pa_seg,
                         const uint2 *__restrict__ pa_ent, const uint16_t *__restrict__ pc_col,
                         const float *__restrict__ pc_val, const uint16_t *__restrict__ cpos,
                         const uint16_t *__restrict__ pcol,
                         const uint32_t *__restrict__ k2at_rs, uint64_t *__restrict__ part_key,
                         float *__restrict__ part_gap, uint32_t *__restrict__ stamps,
                         uint32_t *__restrict__ xcd_work, const uint32_t *__restrict__ xcd_off,
                         const uint32_t *__restrict__ xcd_list, uint32_t epoch,
                         uint32_t *__restrict__ status) {
  constexpr uint32_t W = 256 * S4;  // accumulator columns (>= slice_w)
  // a window's padding slots stay inside the stage
  static_assert(kChunkSlots + 2 * kPairs <= 2 * kStageSlots, "stage slots");
  constexpr uint32_t NC = 4 * S4;   // columns per lane
  constexpr uint32_t NACC = kDual ? 2 : 1;
  extern __shared__ float lds_acc[];
  const uint32_t lane = lane_id();
  const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t wpb = blockDim.x / kWave;
  // dual: each accumulator is followed by one dummy slot per lane of its
  // half (so the second one also starts 32 floats off the bank pattern of
  // the first), then the staged entry triples
  constexpr uint32_t ACC2 = W + kAccPad;
  constexpr uint32_t WAVE_FLOATS = kDual ? 2 * ACC2 + kStageSlots * 4 : W + kWave;
  float *acc = lds_acc + (size_t)wib * WAVE_FLOATS;
  uint4 *stage = reinterpret_cast<uint4 *>(acc + 2 * ACC2);
  const uint32_t half = kDual ? (lane >> 5) : 0u;
  const uint32_t hl = kDual ? (lane & 31u) : lane;  // lane within its half
  float *acc_h = acc + half * ACC2;                   // this half's accumulator
  // narrow slices: gather the staged chunks [t0, t1) (a whole number of
  // steps), chunk s to half s % 2, kPairs per half in flight
  auto gather_steps = [&](const uint2 *cst, uint32_t t0, uint32_t t1) {
    for (uint32_t t = t0; t < t1; t += 2 * kPairs) {
      uint32_t ca[kPairs];
      float xs[kPairs], va[kPairs];
#pragma unroll
      for (uint32_t g = 0; g < kPairs; ++g) {
        const uint2 cx = cst[t + 2 * g + half];
        xs[g] = __uint_as_float(cx.y);
        const uint32_t p = cx.x * kPcCh + hl;
        ca[g] = load_at(pc_col, p * 2u);
        va[g] = load_at(pc_val, p * 4u);
      }
      // padding entries have position 0xffff and go to this lane's dummy
      // slot past the accumulator (positions are slice-local, so nothing
      // lands outside it; the dummy only ever takes + 0)
#pragma unroll
      for (uint32_t g = 0; g < kPairs; ++g) {
        float *q = acc_h + min(ca[g], W + hl);
        *q = __builtin_fmaf(xs[g], va[g], *q);
      }
    }
  };

  // Blocks are dealt to the XCDs round-robin, so block b runs on XCD
  // b % kXcds. Each XCD takes its own slices (all row blocks of them: the
  // ones the assignment gave it, else every kXcds-th), or, with fewer slices
  // than XCDs, its share of the row blocks of one slice, and walks them
  // slice after slice: the AAt columns an XCD gathers stay in its L2. (On
  // another placement only the speed changes.)
  const uint32_t xcd = blockIdx.x % kXcds;
  uint32_t sl0, sl_step, rb0, rb_step, my_sl;
  const uint32_t *my_list = nullptr;
  if (xcd_off != nullptr) {
    const uint32_t o0 = xcd_off[xcd], o1 = xcd_off[xcd + 1];
    my_list = xcd_list + o0;
    my_sl = o1 > o0 ? o1 - o0 : 0u;
    sl0 = 0, sl_step = 1, rb0 = 0, rb_step = 1;
  } else {
    if (n_slices >= kXcds) {
      sl0 = xcd, sl_step = kXcds, rb0 = 0, rb_step = 1;
    } else {
      sl0 = xcd % n_slices, sl_step = kXcds, rb0 = xcd / n_slices, rb_step = kXcds / n_slices;
    }
    my_sl = sl0 < n_slices ? (n_slices - sl0 + sl_step - 1) / sl_step : 0u;
  }
  const uint32_t my_rb = rb0 < n_row_blocks ? (n_row_blocks - rb0 + rb_step - 1) / rb_step : 0u;
  const uint32_t my_units = my_sl * my_rb;
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const float inf = __builtin_inff();
  uint32_t flags = 0;

#pragma unroll
  for (uint32_t a = 0; a < NACC; ++a)
#pragma unroll
    for (uint32_t s4 = 0; s4 < S4; ++s4)
      *reinterpret_cast<float4 *>(acc + a * ACC2 + s4 * 256 + lane * 4) = zero4;
  if constexpr (kDual) {
    if (lane < kAccPad) acc[W + lane] = 0.0f, acc[ACC2 + W + lane] = 0.0f;
  } else {
    acc[W + lane] = 0.0f;  // the dummy slots padding entries add 0 to
  }
  wave_lds_sync();

  // units in slice-major order. With several slices they are taken one at
  // a time from the XCD's counter, so the XCD's waves sweep one slice before
  // the next; a single slice keeps a fixed order (one unit per wave or so).
  const bool dynamic = n_slices > 1;
  const uint32_t wx = (blockIdx.x / kXcds) * wpb + wib;
  const uint32_t nwx = (gridDim.x / kXcds) * wpb;
  for (uint32_t pass = 0;; ++pass) {
    uint32_t u = wx + pass * nwx;
    if (dynamic) {
      if (lane == 0) u = atomicAdd(xcd_work + xcd, 1u);
      u = __builtin_amdgcn_readfirstlane(u);
    }
    if (u >= my_units) break;
    const uint32_t js = u / my_rb;
    const uint32_t rb = rb0 + (u - js * my_rb) * rb_step;
    uint32_t sl = sl0 + js * sl_step;
    if (my_list != nullptr) {
      sl = my_list[js];
      if (sl >= n_slices) {  // an assignment out of range: skip it (the reduce reports it)
        flags |= kFlagBadIndex;
        continue;
      }
    }
    const uint32_t unit = rb * n_slices + sl;
    const uint32_t c0 = sl * slice_w;
    const uint32_t cw = (k - c0) < slice_w ? (k - c0) : slice_w;
    const uint32_t r0 = (uint32_t)(((uint64_t)n * rb) / n_row_blocks);
    const uint32_t r1 = (uint32_t)(((uint64_t)n * (rb + 1)) / n_row_blocks);

    float bv[NC];
    uint32_t bi[NC];
#pragma unroll
    for (uint32_t j = 0; j < NC; ++j) bv[j] = inf, bi[j] = 0xffffffffu;
    float gsum = 0.0f;

    for (uint32_t i = r0; i < r1; ++i) {
      // -- acc[c] = sum_m K2B[i, m] AAt[m, c] over this slice
      uint32_t carry = 0;  // narrow slices: staged chunks left for the next batch
      uint32_t e0, e1;
      if (!row_ok(k2b, i, e0, e1)) flags |= kFlagBadIndex;
      const uint32_t *pseg = pa_seg + (size_t)sl * k;  // the run table of this slice
      for (uint32_t eb = e0; eb < e1; eb += kWave) {
        const uint32_t e = eb + lane;
        // this entry's run of AAt: first chunk q0 and chunks nq of the
        // slice's chunked copy
        uint32_t q0 = 0, nq = 0;
        float x = 0.0f;
        if (e < e1) {
          const uint32_t m = k2b.idx[e];
          x = k2b.val[e];
          if (m < k) {
            q0 = pseg[m];
            nq = pseg[m + 1] - q0;
          } else {
            flags |= kFlagBadIndex;
          }
        }
        if (nq == 0) q0 = 0;  // empty: the padding chunk (adds 0 to dummy slots)
        const uint32_t cnt = (e1 - eb) < kWave ? (e1 - eb) : kWave;
        if constexpr (kDual) {
          // The chunks of the row's runs, flattened in K2B order, are dealt
          // alternately to the two half-waves (chunk s to half s % 2),
          // kPairs per half in flight: every half-wave load reads one whole
          // chunk (32 entries, one 128-byte line of values) whatever the runs'
          // lengths. Each half accumulates into its own array, so a column
          // sums its terms of the even-numbered chunks in one and of the
          // odd-numbered ones in the other, each in K2B order; the fold adds
          // the two. (chunk, K2B value) pairs go through LDS in windows of
          // at most kChunkSlots; slots past the row's last chunk hold the
          // padding chunk 0 with coefficient 0.
          const uint32_t my_nq = lane < cnt ? nq : 0u;
          uint32_t incl = my_nq;
#pragma unroll
          for (uint32_t off = 1; off < kWave; off <<= 1) {
            const uint32_t v = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += v;
          }
          const uint32_t pos = incl - my_nq;
          const uint32_t total = readlane_u32(incl, kWave - 1);
          uint2 *cst = reinterpret_cast<uint2 *>(stage);
          // the row's chunk sequence runs on across its batches: a window
          // holds the chunks carried over from the last one, then new ones;
          // whole steps of 2 kPairs chunks are gathered and the rest (fewer
          // than a step) is carried again, so only the row's last step
          // holds padding
          for (uint32_t done = 0; done < total;) {
            const uint32_t take =
                (total - done) < (kChunkSlots - carry) ? (total - done) : (kChunkSlots - carry);
            for (uint32_t j = pos < done ? done - pos : 0u; j < my_nq && pos + j < done + take; ++j)
              cst[carry + pos + j - done] = make_uint2(q0 + j, __float_as_uint(x));
            wave_lds_sync();
            const uint32_t avail = carry + take;
            const uint32_t full = avail / (2 * kPairs) * (2 * kPairs);
            gather_steps(cst, 0, full);
            carry = avail - full;
            uint2 left = make_uint2(0u, 0u);
            if (lane < carry) left = cst[full + lane];
            wave_lds_sync();
            if (lane < carry) cst[lane] = left;
            wave_lds_sync();
            done += take;
          }
          continue;
        }
        // kGatherRows runs in flight at a time (their first three chunks); the
        // adds still go entry after entry, so every column sums its terms in
        // K2B order and the result does not depend on the timing
        for (uint32_t u = 0; u < cnt; u += kGatherRows) {
          uint32_t gq[kGatherRows], gn[kGatherRows];
          float xs[kGatherRows];
          uint2 ea[kGatherRows], eb[kGatherRows], ec[kGatherRows];
#pragma unroll
          for (uint32_t g = 0; g < kGatherRows; ++g) {
            const uint32_t src = (u + g) < kWave ? (u + g) : (kWave - 1);
            const bool on = (u + g) < cnt;
            gq[g] = on ? readlane_u32(q0, src) : 0u;
            gn[g] = on ? readlane_u32(nq, src) : 0u;
            xs[g] = readlane_f32(x, src);
            ea[g] = load_at(pa_ent + (size_t)gq[g] * kWave, lane * 8u);
            eb[g] = ec[g] = make_uint2(0u, 0u);
            if (gn[g] > 1) eb[g] = load_at(pa_ent + (size_t)(gq[g] + 1) * kWave, lane * 8u);
            if (gn[g] > 2) ec[g] = load_at(pa_ent + (size_t)(gq[g] + 2) * kWave, lane * 8u);
          }
          // the three chunks of one run hold distinct columns (padding lanes
          // point at their own dummy slot and add 0): their old values are
          // read together, then written (one LDS round trip per run)
#pragma unroll
          for (uint32_t g = 0; g < kGatherRows; ++g) {
            float *q = reinterpret_cast<float *>(reinterpret_cast<char *>(acc) + ea[g].x);
            float *qb = reinterpret_cast<float *>(reinterpret_cast<char *>(acc) + eb[g].x);
            float *qc = reinterpret_cast<float *>(reinterpret_cast<char *>(acc) + ec[g].x);
            const float oa = *q;
            const float ob = gn[g] > 1 ? *qb : 0.0f;
            const float oc = gn[g] > 2 ? *qc : 0.0f;
            *q = __builtin_fmaf(xs[g], __uint_as_float(ea[g].y), oa);
            if (gn[g] > 1) *qb = __builtin_fmaf(xs[g], __uint_as_float(eb[g].y), ob);
            if (gn[g] > 2) *qc = __builtin_fmaf(xs[g], __uint_as_float(ec[g].y), oc);
            for (uint32_t j = 3; j < gn[g]; ++j) {
              const uint2 eg = load_at(pa_ent + (size_t)(gq[g] + j) * kWave, lane * 8u);
              float *qj = reinterpret_cast<float *>(reinterpret_cast<char *>(acc) + eg.x);
              *qj = __builtin_fmaf(xs[g], __uint_as_float(eg.y), *qj);
            }
          }
        }
      }
      if constexpr (kDual) {
        // the row's last chunks, with padding up to a whole step
        if (carry != 0) {
          uint2 *cst = reinterpret_cast<uint2 *>(stage);
          if (lane >= carry && lane < 2 * kPairs) cst[lane] = make_uint2(0u, 0u);
          wave_lds_sync();
          gather_steps(cst, 0, 2 * kPairs);
        }
        wave_lds_sync();
      }
      // -- acc[c] -= K2At[i, c] (with several slices, only this slice's run
      // of the row, from the row-slice table)
      uint32_t q0, q1;
      if (k2at_rs != nullptr) {
        const size_t r = (size_t)i * (n_slices + 1) + sl;
        q0 = k2at_rs[r];
        q1 = k2at_rs[r + 1];
        if (q1 < q0) q1 = q0;
      } else if (!row_ok(k2at, i, q0, q1)) {
        flags |= kFlagBadIndex;
      }
      for (uint32_t q = q0 + lane; q < q1; q += kWave) {
        const uint32_t c = k2at.idx[q] - c0;
        if (c < cw) lds_add(acc + (kDual ? (uint32_t)cpos[c0 + c] : c), -k2at.val[q]);
      }
      wave_lds_sync();
      // -- gap += sum_c B[i, c] G[i, c]
      if (b.ptr != nullptr) {
        uint32_t g0, g1;
        if (!row_ok(b, i, g0, g1)) flags |= kFlagBadIndex;
        for (uint32_t q = g0 + lane; q < g1; q += kWave) {
          const uint32_t c = b.idx[q] - c0;
          if (c < cw) {
            const uint32_t pc = kDual ? (uint32_t)cpos[c0 + c] : c;
            gsum += b.val[q] * (kDual ? acc[pc] + acc[ACC2 + pc] : acc[pc]);
          }
        }
      }
      // -- running minimum per column (strict `<`: lowest row wins), clear
#pragma unroll
      for (uint32_t s4 = 0; s4 < S4; ++s4) {
        const uint32_t cb = s4 * 256 + lane * 4;
        float4 *slot = reinterpret_cast<float4 *>(acc + cb);
        float4 v = *slot;
        if constexpr (kDual) {
          float4 *slot2 = reinterpret_cast<float4 *>(acc + ACC2 + cb);
          const float4 v2 = *slot2;
          v.x += v2.x, v.y += v2.y, v.z += v2.z, v.w += v2.w;
          *slot2 = zero4;
        }
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j) {
          if (cb + j < cw && vv[j] < bv[4 * s4 + j]) {
            bv[4 * s4 + j] = vv[j];
            bi[4 * s4 + j] = i;
          }
        }
        *slot = zero4;
      }
      wave_lds_sync();
    }

    // -- this unit's partials (the minima are held by accumulator position;
    // narrow slices write each to its column)
    uint64_t *out = part_key + (size_t)rb * k + c0;
    const uint16_t *pc = kDual ? pcol + (size_t)sl * slice_w : nullptr;
#pragma unroll
    for (uint32_t s4 = 0; s4 < S4; ++s4) {
      const uint32_t cb = s4 * 256 + lane * 4;
#pragma unroll
      for (uint32_t j = 0; j < 4; ++j)
        if (cb + j < cw)
          out[kDual ? (uint32_t)pc[cb + j] : cb + j] = pack_key(bv[4 * s4 + j], bi[4 * s4 + j]);
    }
    const float g = wave_sum_f32(gsum);
    if (lane == 0) {
      part_gap[unit] = g;
      stamps[unit] = epoch;
    }
  }
  // some flags are raised by single lanes: every lane that saw one reports it
  if (flags != 0) atomicOr(status, flags);
}

// Stage 1: block (column group x, row-range chunk y); 4 waves x 64 lanes.
// Lane l of every wave owns column x * 64 + l; wave w takes row ranges
// rb = chunk_lo + w, + 4, ... . Keys are u64 minima, so the order in which
// row ranges are combined does not matter. Every partial it consumes is
// checked: the unit's stamp must be this call's epoch, and the key's row
// must lie in the unit's row range [n rb / NB, n (rb + 1) / NB) (tested
// without a division: n rb < (row + 1) NB <= n (rb + 1)). A unit whose
// column never saw a value below +inf left (+inf, ~0): no finite value.
__global__ void __launch_bounds__(256)
    fw_b_reduce1_kernel(const uint64_t *__restrict__ part_key, const uint32_t *__restrict__ stamps,
                        uint32_t n, uint32_t n_row_blocks, uint32_t n_slices, uint32_t slice_w,
                        uint32_t n_chunks, uint32_t k, uint32_t epoch,
                        const float *__restrict__ part_gap, uint64_t *__restrict__ part2,
                        double *__restrict__ gap2, uint32_t *__restrict__ status) {
  __shared__ uint64_t red[4][kReduceCols];
  __shared__ double gred[256];
  const uint32_t lane = lane_id();
  const uint32_t w = threadIdx.x / kWave;
  const uint32_t c = blockIdx.x * kReduceCols + lane;
  const uint32_t ch = blockIdx.y;
  const uint32_t lo = (uint32_t)(((uint64_t)n_row_blocks * ch) / n_chunks);
  const uint32_t hi = (uint32_t)(((uint64_t)n_row_blocks * (ch + 1)) / n_chunks);
  uint64_t best = ~0ull;
  uint32_t flags = 0;
  if (c < k) {
    const uint32_t sl = c / slice_w;
    for (uint32_t rb = lo + w; rb < hi; rb += 4) {
      const uint64_t key = part_key[(size_t)rb * k + c];
      best = key < best ? key : best;
      if (stamps[(size_t)rb * n_slices + sl] != epoch) flags |= kFlagPartialsInvalid;
      const uint64_t row1 = (uint64_t)(uint32_t)key + 1u;
      if (key == kNoValueKey)
        flags |= kFlagNonfinite;
      else if (!((uint64_t)n * rb < row1 * n_row_blocks &&
                 row1 * n_row_blocks <= (uint64_t)n * (rb + 1u)))
        flags |= kFlagPartialsInvalid;
    }
  }
  red[w][lane] = best;
  __syncthreads();
  if (w == 0 && c < k) {
    uint64_t m = red[0][lane];
    for (uint32_t x = 1; x < 4; ++x) m = red[x][lane] < m ? red[x][lane] : m;
    part2[(size_t)ch * k + c] = m;
  }
  if (flags != 0) atomicOr(status, flags);
  // the first column group also sums this chunk's share of the gap
  // partials (f64, a fixed order: strided per thread, then a tree)
  if (blockIdx.x == 0) {
    const uint64_t units = (uint64_t)n_row_blocks * n_slices;
    const uint32_t u0 = (uint32_t)(units * ch / n_chunks);
    const uint32_t u1 = (uint32_t)(units * (ch + 1) / n_chunks);
    double s = 0.0;
    for (uint32_t u = u0 + threadIdx.x; u < u1; u += 256) s += (double)part_gap[u];
    gred[threadIdx.x] = s;
    __syncthreads();
    for (uint32_t h = 128; h > 0; h >>= 1) {
      if (threadIdx.x < h) gred[threadIdx.x] += gred[threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x == 0) gap2[ch] = gred[0];
  }
}

// Stage 2: one thread per column over the chunk minima; the last block's
// first thread adds the chunks' gap sums in chunk order.
__global__ void __launch_bounds__(256)
    fw_b_reduce2_kernel(const uint64_t *__restrict__ part2, uint32_t n_chunks,
                        const double *__restrict__ gap2, uint32_t n, uint32_t k,
                        float *__restrict__ out_val, uint32_t *__restrict__ out_idx,
                        float *__restrict__ gap, uint32_t *__restrict__ status) {
  const uint32_t col_blocks = (k + 255) / 256;
  if (blockIdx.x < col_blocks) {
    const uint32_t c = blockIdx.x * 256 + threadIdx.x;
    if (c >= k) return;
    uint64_t best = ~0ull;
    for (uint32_t ch = 0; ch < n_chunks; ++ch) {
      const uint64_t key = part2[(size_t)ch * k + c];
      best = key < best ? key : best;
    }
    const uint32_t row = (uint32_t)best;
    const float v = f32_unorder((uint32_t)(best >> 32));
    uint32_t flags = 0;
    // (+inf, ~0): no row gave this column a finite value (stage 1 flagged it)
    if (row >= n && best != kNoValueKey) flags |= kFlagPartialsInvalid;
    if (!__builtin_isfinite(v)) flags |= kFlagNonfinite;
    out_val[c] = v;
    out_idx[c] = row;
    if (flags != 0) atomicOr(status, flags);
  } else if (threadIdx.x == 0 && gap != nullptr) {
    double s = 0.0;
    for (uint32_t ch = 0; ch < n_chunks; ++ch) s += gap2[ch];
    *gap = (float)s;
  }
}

// Full Frank-Wolfe duality gap of the B subproblem: sum(B * G) - sum_c
// min_i G[i, c]. One block: the chunks' gap sums are added exactly as the
// final reduce adds them (chunk order, f64), the column minima in f64.
__global__ void __launch_bounds__(256)
    fw_b_fw_gap_kernel(const double *__restrict__ gap2, uint32_t n_chunks,
                       const float *__restrict__ out_val, uint32_t k,
                       float *__restrict__ fw_gap) {
  __shared__ double red[256];
  double v = 0.0;
  for (uint32_t c = threadIdx.x; c < k; c += 256) v += (double)out_val[c];
  red[threadIdx.x] = v;
  __syncthreads();
  for (uint32_t w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (uint32_t ch = 0; ch < n_chunks; ++ch) s += gap2[ch];
    *fw_gap = (float)(s - red[0]);
  }
}

// B step on padded B^T rows, one thread per archetype.
__global__ void __launch_bounds__(256)
    fw_b_apply_kernel(uint32_t *__restrict__ bt_idx, float *__restrict__ bt_val,
                      uint32_t *__restrict__ bt_cnt, uint32_t n, uint32_t k, uint32_t cap_b,
                      const uint32_t *__restrict__ arg_idx, float gamma,
                      uint32_t *__restrict__ status) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= k) return;
  uint32_t *idx = bt_idx + (size_t)c * cap_b;
  float *val = bt_val + (size_t)c * cap_b;
  const uint32_t cnt = bt_cnt[c];
  const uint32_t i = arg_idx[c];
  if (cnt > cap_b || i >= n) {
    atomicOr(status, kFlagBadIndex);
    return;
  }
  uint32_t pos = 0;
  while (pos < cnt && idx[pos] < i) ++pos;
  const bool present = pos < cnt && idx[pos] == i;
  if (!present && cnt == cap_b) {
    atomicOr(status, kFlagBCapOverflow);
    return;
  }
  const float keep = 1.0f - gamma;
  for (uint32_t s = 0; s < cnt; ++s) val[s] *= keep;
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

__global__ void status_clear_kernel(uint32_t *__restrict__ status) { *status = 0u; }

__global__ void xcd_work_zero_kernel(uint32_t *__restrict__ p, uint32_t count) {
  if (threadIdx.x < count) p[threadIdx.x] = 0u;
}

__global__ void __launch_bounds__(256)
    hist_zero_kernel(uint32_t *__restrict__ p, uint32_t count) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = 0u;
}

template <uint32_t S4, bool kDual>
hipError_t launch_partials(const BPlan &p, Csr k2b, Csr aat, Csr k2at, Csr b, uint32_t n,
                           uint32_t k, const uint32_t *seg, const uint32_t *pa_seg,
                           const uint2 *pa_ent, const uint16_t *pc_col, const float *pc_val,
                           const uint16_t *cpos, const uint16_t *pcol,
                           const uint32_t *k2at_rs, uint64_t *keys,
                           float *gap_part, uint32_t *stamps, uint32_t *xcd_work,
                           const uint32_t *xcd_off, const uint32_t *xcd_list, uint32_t epoch,
                           uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  const uint32_t lds = (kBThreads / kWave) *
                       (kDual ? 2 * (256 * S4 + kAccPad) + kStageSlots * 4 : 256 * S4 + kWave) *
                       sizeof(float);
  // narrow slices: kGatherRows pairs of runs in flight, or twice as many
  // when that keeps as many blocks resident (the wider accumulators are
  // register-bound already)
  auto k_std = &fw_b_partials_kernel<S4, kDual, kGatherRows>;
  auto k_deep = k_std;
  if constexpr (kDual) k_deep = &fw_b_partials_kernel<S4, true, 2 * kGatherRows>;
  static int bpc = -1;
  static bool deep = false;
  if (bpc < 0) {
    int v = 0, v2 = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void *>(k_std),
                                                     kBThreads, lds);
    if (e != hipSuccess) return e;
    if (kDual) {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &v2, reinterpret_cast<const void *>(k_deep), kBThreads, lds);
      if (e != hipSuccess) return e;
    }
    deep = kDual && v2 >= v;
    bpc = v < 1 ? 1 : v;
  }
  const uint64_t units = (uint64_t)p.n_row_blocks * p.n_slices;
  const uint64_t want = (units + 3) / 4;
  const uint64_t resident = (uint64_t)dev.cus * (uint64_t)bpc;
  uint64_t blocks = want < resident ? want : resident;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;  // the same number of blocks on every XCD
  hipLaunchKernelGGL(deep ? k_deep : k_std, dim3((uint32_t)blocks), dim3(kBThreads), lds,
                     stream, k2b, aat, k2at, b, n, k, p.slice_w, p.n_slices, p.n_row_blocks, seg,
                     pa_seg, pa_ent, pc_col, pc_val, cpos, pcol, k2at_rs, keys, gap_part, stamps,
                     xcd_work, xcd_off, xcd_list, epoch, status);
  return hipGetLastError();
}

}  // namespace

// Slices: one when k fits one accumulator (k <= 2048); otherwise enough
// that each holds at most kSliceCols columns (the running minima of wider
// slices take registers that cost resident waves) and at most ~3.75 MB of
// AAt at 8 bytes per entry (its chunked copy, ~6 bytes per entry plus
// padding, stays within one XCD's 4 MB L2), as 2, 4 or a multiple of 8
// slices so that they spread evenly over the XCDs.
static uint32_t slices_for(uint32_t k, uint64_t aat_nnz) {
  const uint32_t wmax = 256u * kBMaxS4;
  if (k <= wmax) return 1;
  uint64_t s = ((uint64_t)k + kSliceCols - 1) / kSliceCols;
  const uint64_t by_l2 = (aat_nnz * 8 + kSliceAatBytes - 1) / kSliceAatBytes;
  if (by_l2 > s) s = by_l2;
  if (s <= 2) return 2;
  if (s <= 4) return 4;
  s = (s + kXcds - 1) / kXcds * kXcds;
  const uint64_t most = ((uint64_t)k + 3) / 4;  // slices of at least 4 columns
  return (uint32_t)(s < most ? s : most);
}

static BPlan plan_with_slices(uint32_t n, uint32_t k, uint32_t n_slices, uint64_t aat_nnz) {
  BPlan p{};
  p.n_slices = n_slices;
  p.slice_w = (uint32_t)align_up((k + n_slices - 1) / n_slices, 4);
  p.n_slices = (k + p.slice_w - 1) / p.slice_w;
  p.s4 = (p.slice_w + 255u) / 256u;
  uint64_t rb = p.n_slices > 1 ? kSlicedRowBlocks : kBUnitsTarget;
  // the partial keys take n_row_blocks * k * 8 bytes: fewer row ranges for
  // a very large k (one at least)
  const uint64_t rb_budget = kKeysBudget / ((uint64_t)k * sizeof(uint64_t));
  if (rb > rb_budget) rb = rb_budget;
  if (rb > n) rb = n;
  if (rb < 1) rb = 1;
  p.n_row_blocks = (uint32_t)rb;
  p.n_chunks = p.n_row_blocks < kMaxChunks ? p.n_row_blocks : kMaxChunks;
  const size_t units = (size_t)p.n_row_blocks * p.n_slices;
  size_t off = 0;
  p.off_keys = off;
  off = align_up(off + (size_t)p.n_row_blocks * k * sizeof(uint64_t), 256);
  p.off_part2 = off;
  off = align_up(off + (size_t)p.n_chunks * k * sizeof(uint64_t), 256);
  p.off_gap = off;
  off = align_up(off + units * sizeof(float), 256);
  p.off_gap2 = off;
  off = align_up(off + (size_t)p.n_chunks * sizeof(double), 256);
  p.off_stamp = off;
  off = align_up(off + units * sizeof(uint32_t), 256);
  p.off_work = off;
  off = align_up(off + kXcds * sizeof(uint32_t), 256);
  p.off_seg = off;
  if (p.n_slices > 1) off = align_up(off + (size_t)k * (p.n_slices + 1) * sizeof(uint32_t), 256);
  p.off_rs = off;
  if (p.n_slices > 1) off = align_up(off + (size_t)n * (p.n_slices + 1) * sizeof(uint32_t), 256);
  // AAt copied per slice in chunks: narrow slices gather two short runs per
  // wave instruction (one per half-wave) from chunks of 32 entries (16-bit
  // accumulator positions and f32 values apart, addressed with 32-bit byte
  // offsets); otherwise chunks of 64 (accumulator byte offset, value) pairs.
  // A run of len entries takes ceil(len / ch) <= len / ch + 1 chunks and an
  // empty run none, so all runs take at most nnz / ch + min(runs, nnz)
  // chunks, plus chunk 0 (padding)
  const uint64_t runs = (uint64_t)k * p.n_slices;
  const uint64_t nonempty = runs < aat_nnz ? runs : aat_nnz;
  const uint64_t pc_chunks = (aat_nnz + kPcCh - 1) / kPcCh + nonempty + 1;
  p.dual = p.n_slices > 1 && pc_chunks < (1ull << 25) && p.slice_w <= kOrderMax;
  p.pa_ch = p.dual ? kPcCh : kWave;
  p.pa_chunks = p.dual ? pc_chunks : (aat_nnz + kWave - 1) / kWave + nonempty + 1;
  p.off_pa_seg = off;
  off = align_up(off + (runs + 1) * sizeof(uint32_t), 256);
  p.off_pa_bsum = off;  // the run-table scan: one sum per kScanRuns runs, then the total
  off = align_up(off + ((runs + kScanRuns - 1) / kScanRuns + 1) * sizeof(uint64_t), 256);
  p.off_pa_ent = off;
  if (!p.dual) off = align_up(off + (size_t)p.pa_chunks * p.pa_ch * sizeof(uint2), 256);
  p.off_pc_col = off;
  if (p.dual) off = align_up(off + (size_t)p.pa_chunks * kPcCh * sizeof(uint16_t), 256);
  p.off_pc_val = off;
  if (p.dual) off = align_up(off + (size_t)p.pa_chunks * kPcCh * sizeof(float), 256);
  p.off_walk = off;
  if (p.dual) off = align_up(off + 2 * (size_t)k * sizeof(float), 256);
  p.off_cpos = off;
  if (p.dual) off = align_up(off + (size_t)k * sizeof(uint16_t), 256);
  p.off_pcol = off;
  if (p.dual) off = align_up(off + (size_t)p.n_slices * p.slice_w * sizeof(uint16_t), 256);
  // the XCDs' slices, when some XCD owns more than one (with one slice each
  // there is nothing to even out)
  p.balance = p.dual && p.n_slices > kXcds && p.n_slices <= kBalanceMax;
  p.off_hist = off;
  if (p.balance) off = align_up(off + (size_t)k * sizeof(uint32_t), 256);
  p.off_swork = off;
  if (p.balance) off = align_up(off + (size_t)p.n_slices * sizeof(uint64_t), 256);
  p.off_xcd_off = off;
  if (p.balance) off = align_up(off + (kXcds + 1) * sizeof(uint32_t), 256);
  p.off_xcd_list = off;
  if (p.balance) off = align_up(off + (size_t)p.n_slices * sizeof(uint32_t), 256);
  p.ws_bytes = off;
  return p;
}

BPlan plan_b(uint32_t n, uint32_t k, uint64_t aat_nnz) {
  return plan_with_slices(n, k, slices_for(k, aat_nnz), aat_nnz);
}

hipError_t launch_status_clear(uint32_t *status, hipStream_t stream) {
  hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(1), 0, stream, status);
  return hipGetLastError();
}

hipError_t launch_fw_b(const BPlan &p, Csr k2b, Csr aat, Csr k2at, Csr b, uint32_t n,
                       uint32_t k, float *out_val, uint32_t *out_idx, float *gap,
                       float *fw_gap, void *ws, uint32_t *status, uint32_t epoch,
                       hipStream_t stream) {
  char *base = static_cast<char *>(ws);
  uint64_t *keys = reinterpret_cast<uint64_t *>(base + p.off_keys);
  float *gap_part = reinterpret_cast<float *>(base + p.off_gap);
  uint32_t *stamps = reinterpret_cast<uint32_t *>(base + p.off_stamp);
  uint32_t *seg = p.n_slices > 1 ? reinterpret_cast<uint32_t *>(base + p.off_seg) : nullptr;
  uint32_t *pa_seg = reinterpret_cast<uint32_t *>(base + p.off_pa_seg);
  uint2 *pa_ent = reinterpret_cast<uint2 *>(base + p.off_pa_ent);
  uint32_t *xcd_work = reinterpret_cast<uint32_t *>(base + p.off_work);
  uint32_t *k2at_rs = p.n_slices > 1 ? reinterpret_cast<uint32_t *>(base + p.off_rs) : nullptr;
  hipError_t e;
  if (k2at_rs != nullptr) {
    const uint64_t total = (uint64_t)n * (p.n_slices + 1);
    const uint64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(row_slice_kernel, dim3((uint32_t)(blocks < 65536u ? blocks : 65536u)),
                       dim3(256), 0, stream, k2at, n, p.slice_w, p.n_slices, k2at_rs, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (seg != nullptr) {
    const uint64_t total = (uint64_t)k * (p.n_slices + 1);
    const uint64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(seg_table_kernel, dim3((uint32_t)(blocks < 65536u ? blocks : 65536u)),
                       dim3(256), 0, stream, aat, k, p.slice_w, p.n_slices, seg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the chunked copy of AAt per slice (run table, then the entries)
  const bool dual = p.dual;
  uint16_t *pc_col = reinterpret_cast<uint16_t *>(base + p.off_pc_col);
  float *pc_val = reinterpret_cast<float *>(base + p.off_pc_val);
  uint16_t *cpos = dual ? reinterpret_cast<uint16_t *>(base + p.off_cpos) : nullptr;
  uint16_t *pcol = dual ? reinterpret_cast<uint16_t *>(base + p.off_pcol) : nullptr;
  if (dual) {
    // the in-slice column order: the walk, then one sort per slice
    float *walk = reinterpret_cast<float *>(base + p.off_walk);
    const uint32_t blocks = (k + 3) / 4;  // 4 waves per block, one row each
    const dim3 grid(blocks < 65535u ? blocks : 65535u);
    for (uint32_t t = 0; t < kWalkSteps; ++t) {
      const float *x = t == 0 ? nullptr : walk + (size_t)((t + 1) & 1) * k;
      hipLaunchKernelGGL(col_walk_kernel, grid, dim3(256), 0, stream, aat, k, x,
                         walk + (size_t)(t & 1) * k);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(slice_order_kernel, dim3(p.n_slices), dim3(1024), 0, stream,
                       walk + (size_t)((kWalkSteps - 1) & 1) * k, k, p.slice_w, cpos, pcol);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const uint64_t runs = (uint64_t)k * p.n_slices;
    const uint32_t nb = (uint32_t)((runs + kScanRuns - 1) / kScanRuns);
    uint64_t *bsum = reinterpret_cast<uint64_t *>(base + p.off_pa_bsum);
    hipLaunchKernelGGL(pa_count_kernel, dim3(nb), dim3(256), 0, stream, aat, seg, k, p.n_slices,
                       p.pa_ch, pa_seg, bsum, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pa_bscan_kernel, dim3(1), dim3(256), 0, stream, bsum, nb, runs,
                       p.pa_chunks, pa_seg, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pa_offs_kernel, dim3(nb), dim3(256), 0, stream, pa_seg, bsum, nb, runs,
                       p.pa_chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const uint64_t runs = (uint64_t)k * p.n_slices;
    const uint64_t blocks = (runs + 3) / 4;  // 4 waves per block, one run each
    const dim3 grid((uint32_t)(blocks < 65535u ? blocks : 65535u));
    if (dual)
      hipLaunchKernelGGL(pc_fill_kernel, grid, dim3(256), 0, stream, aat, seg, k, p.n_slices,
                         p.slice_w, pa_seg, cpos, pc_col, pc_val, status);
    else
      hipLaunchKernelGGL(pa_fill_kernel, grid, dim3(256), 0, stream, aat, seg, k, p.n_slices,
                         p.slice_w, p.pa_ch, 256u * p.s4, pa_seg, pa_ent, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // which XCD owns which slice
  const uint32_t *xcd_off = nullptr, *xcd_list = nullptr;
  if (p.balance) {
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + p.off_hist);
    uint64_t *swork = reinterpret_cast<uint64_t *>(base + p.off_swork);
    uint32_t *off = reinterpret_cast<uint32_t *>(base + p.off_xcd_off);
    uint32_t *list = reinterpret_cast<uint32_t *>(base + p.off_xcd_list);
    const uint32_t zb = (k + 255) / 256;
    hipLaunchKernelGGL(hist_zero_kernel, dim3(zb < 4096u ? zb : 4096u), dim3(256), 0, stream,
                       hist, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const uint64_t sampled = ((uint64_t)n + kHistRowStep - 1) / kHistRowStep;
    const uint64_t hb = (sampled + 3) / 4;  // 4 waves per block, one row each
    const bool local = k <= kHistLds;
    const uint64_t cap = local ? kHistBlocks : 16384u;
    hipLaunchKernelGGL(ref_hist_kernel, dim3((uint32_t)(hb < cap ? (hb > 0 ? hb : 1) : cap)),
                       dim3(256), local ? (size_t)k * sizeof(uint32_t) : 0, stream, k2b, n, k,
                       hist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(slice_work_kernel, dim3(p.n_slices), dim3(256), 0, stream, hist, pa_seg,
                       k, swork);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(xcd_assign_kernel, dim3(1), dim3(1024), 0, stream, swork, p.n_slices, off,
                       list);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    xcd_off = off;
    xcd_list = list;
  }
  hipLaunchKernelGGL(xcd_work_zero_kernel, dim3(1), dim3(64), 0, stream, xcd_work, kXcds);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (p.s4) {
#define SEACELLS_B_CASE(S)                                                                      \
  case S:                                                                                       \
    e = dual ? launch_partials<S, true>(p, k2b, aat, k2at, b, n, k, seg, pa_seg, pa_ent,       \
                                        pc_col, pc_val, cpos, pcol, k2at_rs, keys, gap_part,    \
                                        stamps, xcd_work, xcd_off, xcd_list, epoch, status,     \
                                        stream)                                                 \
             : launch_partials<S, false>(p, k2b, aat, k2at, b, n, k, seg, pa_seg, pa_ent,      \
                                         pc_col, pc_val, cpos, pcol, k2at_rs, keys, gap_part,   \
                                         stamps, xcd_work, xcd_off, xcd_list, epoch, status,    \
                                         stream);                                               \
    break;
    SEACELLS_B_CASE(1)
    SEACELLS_B_CASE(2)
    SEACELLS_B_CASE(3)
    SEACELLS_B_CASE(4)
    SEACELLS_B_CASE(5)
    SEACELLS_B_CASE(6)
    SEACELLS_B_CASE(7)
    SEACELLS_B_CASE(8)
#undef SEACELLS_B_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_fw_b_reduce(p, n, k, out_val, out_idx, gap, fw_gap, ws, status, epoch, stream);
}

hipError_t launch_fw_b_reduce(const BPlan &p, uint32_t n, uint32_t k, float *out_val,
                              uint32_t *out_idx, float *gap, float *fw_gap, void *ws,
                              uint32_t *status, uint32_t epoch, hipStream_t stream) {
  char *base = static_cast<char *>(ws);
  const uint64_t *keys = reinterpret_cast<const uint64_t *>(base + p.off_keys);
  uint64_t *part2 = reinterpret_cast<uint64_t *>(base + p.off_part2);
  const float *gap_part = reinterpret_cast<const float *>(base + p.off_gap);
  double *gap2 = reinterpret_cast<double *>(base + p.off_gap2);
  const uint32_t *stamps = reinterpret_cast<const uint32_t *>(base + p.off_stamp);
  hipError_t e;
  const dim3 g1((k + kReduceCols - 1) / kReduceCols, p.n_chunks);
  hipLaunchKernelGGL(fw_b_reduce1_kernel, g1, dim3(256), 0, stream, keys, stamps, n,
                     p.n_row_blocks, p.n_slices, p.slice_w, p.n_chunks, k, epoch, gap_part, part2,
                     gap2, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(fw_b_reduce2_kernel, dim3((k + 255) / 256 + 1), dim3(256), 0, stream, part2,
                     p.n_chunks, gap2, n, k, out_val, out_idx, gap, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (fw_gap != nullptr) {
    hipLaunchKernelGGL(fw_b_fw_gap_kernel, dim3(1), dim3(256), 0, stream, gap2, p.n_chunks,
                       out_val, k, fw_gap);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_fw_b_apply(uint32_t *bt_idx, float *bt_val, uint32_t *bt_cnt, uint32_t n,
                             uint32_t k, uint32_t cap_b, const uint32_t *arg_idx, float gamma,
                             uint32_t *status, hipStream_t stream) {
  hipLaunchKernelGGL(fw_b_apply_kernel, dim3((k + 255) / 256), dim3(256), 0, stream, bt_idx,
                     bt_val, bt_cnt, n, k, cap_b, arg_idx, gamma, status);
  return hipGetLastError();
}

}  // namespace seacells
