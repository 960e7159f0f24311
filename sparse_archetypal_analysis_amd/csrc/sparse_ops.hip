// Sparse operations that build the Frank-Wolfe operands on the device: the
// page's host routines `csr_matmul_csr` (product of two CSR matrices, each
// output row sorted), `transpose_sparse` (rows of the transpose in ascending
// order of the original rows), and the sums the RSS identity needs
// (||K - K B A||^2 = <K, K> - 2 <K^2 B, A^T> + <B^T K^2 B, A A^T>).
//
// Product C = A B, one wave per row of A:
//   a bitmap of the row's output columns is built in LDS (a window of
//   16384 columns at a time), a popcount prefix over it gives every column
//   its rank, and the products are added into an LDS slot per rank (a window
//   of 2048 ranks at a time), then written out in column order. The entries
//   of A's row are taken one after the other and each B row is spread over
//   the lanes (the columns of one row are unique, so a lane-parallel add
//   never collides): every output sums its products in A-entry order, then
//   B-entry order, in f32 with fma. The output keeps every column that some
//   product reaches (a sum that cancels to 0 stays as an explicit 0).
// Transpose: rows are cut into R blocks; one wave per block counts its
//   entries per column, the counts become per-(block, column) write
//   positions, and each wave writes its rows in order, so a transposed row
//   lists the original rows in ascending order (no atomics on positions).
// Inner product <X, Y> over two matrices of the same shape: one wave per row
//   looks each X entry up in Y's row (binary search), products in f64; the
//   rows' partial sums are added in a fixed order.
#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kSpWaves = 4;        // waves per block
constexpr uint32_t kSpWinWords = 512;   // bitmap words per column window (16384 columns)
constexpr uint32_t kSpSlots = 2048;     // value slots per rank window
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

// Exclusive prefix sum over the wave (lane order).
__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t x, uint32_t lane) {
  uint32_t incl = x;
  for (uint32_t off = 1; off < kWave; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  return incl - x;
}

// Mark in bits[] (window starting at column w0, nw words) every column some
// product of A's row [a0, a1) reaches. Returns the flags seen.
__device__ __forceinline__ uint32_t mark_columns(const Csr &a, const Csr &b, uint32_t p,
                                                 uint32_t q, uint32_t a0, uint32_t a1,
                                                 uint32_t w0, uint32_t nw, uint32_t *bits,
                                                 uint32_t lane) {
  uint32_t flags = 0;
  for (uint32_t e = a0; e < a1; ++e) {
    const uint32_t j = a.idx[e];
    uint32_t b0, b1;
    if (j >= p || !sp_row(b, j, b0, b1)) {
      flags |= kFlagBadIndex;
      continue;
    }
    for (uint32_t t = b0 + lane; t < b1; t += kWave) {
      const uint32_t c = b.idx[t];
      if (c >= q) {
        flags |= kFlagBadIndex;
        continue;
      }
      const uint32_t rel = c - w0;
      if (rel < nw * 32u) atomicOr(&bits[rel >> 5], 1u << (rel & 31u));
    }
  }
  return flags;
}

// Output columns per row of A B into cnt[r] (the caller's row pointer + 1).
__global__ void __launch_bounds__(kSpWaves * kWave)
    spgemm_count_kernel(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                        uint32_t *__restrict__ cnt, uint32_t *__restrict__ status) {
  __shared__ uint32_t bits_all[kSpWaves][kSpWinWords];
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t *bits = bits_all[wib];
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * kSpWaves + wib; r < m; r += gridDim.x * kSpWaves) {
    uint32_t a0, a1;
    if (!sp_row(a, r, a0, a1)) flags |= kFlagBadIndex;
    uint64_t total = 0;
    for (uint64_t w0 = 0; w0 < q; w0 += (uint64_t)kSpWinWords * 32u) {
      const uint32_t nw = (uint32_t)u64min(kSpWinWords, (q - w0 + 31u) / 32u);
      for (uint32_t w = lane; w < nw; w += kWave) bits[w] = 0u;
      wave_lds_sync();
      flags |= mark_columns(a, b, p, q, a0, a1, (uint32_t)w0, nw, bits, lane);
      wave_lds_sync();
      uint32_t part = 0;
      for (uint32_t w = lane; w < nw; w += kWave) part += __popc(bits[w]);
      total += wave_sum_u32(part);
      wave_lds_sync();
    }
    if (lane == 0) cnt[r] = total > 0xffffffffull ? 0xffffffffu : (uint32_t)total;
  }
  if (flags != 0) atomicOr(status, flags);
}

// One block: ptr[0] = 0, ptr[1 .. count] becomes the inclusive prefix sum of
// itself (64-bit, so a total of 2^31 or more is caught: then the flag is set
// and every pointer is 0, so a later pass over them writes nothing).
__global__ void __launch_bounds__(1024)
    scan_counts_kernel(uint32_t *__restrict__ ptr, uint32_t count, uint32_t too_large_flag,
                       uint32_t *__restrict__ status) {
  __shared__ uint64_t part[1024];
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (count + 1023u) / 1024u;
  const uint32_t i0 = min(tid * per, count), i1 = min(i0 + per, count);
  uint64_t sum = 0;
  for (uint32_t i = i0; i < i1; ++i) sum += ptr[1 + i];
  part[tid] = sum;
  __syncthreads();
  for (uint32_t off = 1; off < 1024; off <<= 1) {
    const uint64_t v = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const bool too_large = part[1023] >= 0x80000000ull;
  uint64_t at = part[tid] - sum;
  for (uint32_t i = i0; i < i1; ++i) {
    at += ptr[1 + i];
    ptr[1 + i] = too_large ? 0u : (uint32_t)at;
  }
  if (tid == 0) {
    ptr[0] = 0u;
    if (too_large) atomicOr(status, too_large_flag);
  }
}

// Columns and values of A B into the rows the count pass sized.
__global__ void __launch_bounds__(kSpWaves * kWave)
    spgemm_fill_kernel(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                       const uint32_t *__restrict__ c_ptr, uint32_t *__restrict__ c_idx,
                       float *__restrict__ c_val, uint32_t *__restrict__ status) {
  __shared__ uint32_t bits_all[kSpWaves][kSpWinWords];
  __shared__ uint32_t rank_all[kSpWaves][kSpWinWords];
  __shared__ float acc_all[kSpWaves][kSpSlots];
  const uint32_t lane = lane_id();
  const uint32_t wib = threadIdx.x / kWave;
  uint32_t *bits = bits_all[wib];
  uint32_t *rank = rank_all[wib];
  float *acc = acc_all[wib];
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * kSpWaves + wib; r < m; r += gridDim.x * kSpWaves) {
    const uint32_t base = c_ptr[r], end = c_ptr[r + 1];
    const uint32_t cnt = end >= base ? end - base : 0u;
    uint32_t a0, a1;
    if (!sp_row(a, r, a0, a1)) flags |= kFlagBadIndex;
    uint32_t done = 0;
    for (uint64_t w0l = 0; w0l < q; w0l += (uint64_t)kSpWinWords * 32u) {
      const uint32_t w0 = (uint32_t)w0l;
      const uint32_t nw = (uint32_t)u64min(kSpWinWords, (q - w0l + 31u) / 32u);
      for (uint32_t w = lane; w < nw; w += kWave) bits[w] = 0u;
      wave_lds_sync();
      flags |= mark_columns(a, b, p, q, a0, a1, w0, nw, bits, lane);
      wave_lds_sync();
      // ranks: each lane takes a contiguous run of words
      const uint32_t per = (nw + kWave - 1) / kWave;
      const uint32_t v0w = min(lane * per, nw), v1w = min(v0w + per, nw);
      uint32_t part = 0;
      for (uint32_t w = v0w; w < v1w; ++w) part += __popc(bits[w]);
      uint32_t run = wave_excl_scan_u32(part, lane);
      const uint32_t nwin = wave_sum_u32(part);
      for (uint32_t w = v0w; w < v1w; ++w) {
        rank[w] = run;
        run += __popc(bits[w]);
      }
      wave_lds_sync();
      for (uint32_t s0 = 0; s0 < nwin; s0 += kSpSlots) {
        const uint32_t ns = min(kSpSlots, nwin - s0);
        for (uint32_t s = lane; s < ns; s += kWave) acc[s] = 0.0f;
        wave_lds_sync();
        for (uint32_t e = a0; e < a1; ++e) {
          const uint32_t j = a.idx[e];
          const float av = a.val[e];
          uint32_t b0, b1;
          if (j >= p || !sp_row(b, j, b0, b1)) continue;  // flagged by the marking pass
          for (uint32_t t = b0 + lane; t < b1; t += kWave) {
            const uint32_t c = b.idx[t];
            const uint32_t rel = c - w0;
            if (c >= q || rel >= nw * 32u) continue;
            const uint32_t w = rel >> 5, bit = 1u << (rel & 31u);
            const uint32_t pos = rank[w] + __popc(bits[w] & (bit - 1u)) - s0;
            if (pos < ns) acc[pos] = __builtin_fmaf(av, b.val[t], acc[pos]);
          }
          wave_lds_sync();
        }
        // out in column order: the lane owning word w writes its set bits
        for (uint32_t w = lane; w < nw; w += kWave) {
          uint32_t x = bits[w];
          uint32_t pos = rank[w];
          while (x != 0u) {
            const uint32_t bpos = (uint32_t)__builtin_ctz(x);
            x &= x - 1u;
            const uint32_t slot = pos - s0;
            if (slot < ns && done + pos < cnt) {
              c_idx[(size_t)base + done + pos] = w0 + w * 32u + bpos;
              c_val[(size_t)base + done + pos] = acc[slot];
            }
            ++pos;
          }
        }
        wave_lds_sync();
      }
      done += nwin;
    }
    if (done != cnt) flags |= kFlagBadIndex;  // row pointers not those of the count pass
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
    if (!sp_row(x, r, x0, x1) || !sp_row(y, r, y0, y1)) flags |= kFlagBadIndex;
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

uint32_t sp_blocks(uint32_t m, const DeviceInfo &dev) {
  // enough blocks to fill the device a few times over, never more than rows need
  const uint64_t want = ((uint64_t)m + kSpWaves - 1) / kSpWaves;
  const uint64_t cap = (uint64_t)dev.cus * 8u;
  return (uint32_t)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

uint32_t tr_blocks(uint32_t m, uint32_t q) {
  uint64_t nb = ((uint64_t)m + 255u) / 256u;
  if (nb > kTrMaxBlocks) nb = kTrMaxBlocks;
  const uint64_t by_table = kTrTableBytes / (4ull * (q > 0 ? q : 1));
  if (nb > by_table) nb = by_table;
  return (uint32_t)(nb > 0 ? nb : 1);
}

size_t transpose_workspace(uint32_t m, uint32_t q) {
  return align_up((size_t)tr_blocks(m, q) * q * sizeof(uint32_t), 256);
}

size_t dot_workspace() { return kDotBlocks * sizeof(double); }

hipError_t launch_spgemm_count(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                               uint32_t *c_ptr, uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  if (m > 0) {
    hipLaunchKernelGGL(spgemm_count_kernel, dim3(sp_blocks(m, dev)), dim3(kSpWaves * kWave), 0,
                       stream, a, b, m, p, q, c_ptr + 1, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, stream, c_ptr, m,
                     kFlagOutputTooLarge, status);
  return hipGetLastError();
}

hipError_t launch_spgemm_fill(Csr a, Csr b, uint32_t m, uint32_t p, uint32_t q,
                              const uint32_t *c_ptr, uint32_t *c_idx, float *c_val,
                              uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(spgemm_fill_kernel, dim3(sp_blocks(m, dev)), dim3(kSpWaves * kWave), 0,
                     stream, a, b, m, p, q, c_ptr, c_idx, c_val, status);
  return hipGetLastError();
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
  hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, stream, at_ptr, q,
                     kFlagOutputTooLarge, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (q > 0) {
    hipLaunchKernelGGL(tr_base_kernel, dim3(cb), dim3(256), 0, stream, q, nb, table, at_ptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tr_fill_kernel, dim3(nb), dim3(kWave), 0, stream, a, m, q, nb, table,
                     at_idx, at_val);
  return hipGetLastError();
}

hipError_t launch_dot(Csr x, Csr y, uint32_t m, double alpha, double *acc, void *ws,
                      uint32_t *status, hipStream_t stream) {
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
