// A update: the per-cell Frank-Wolfe column solve (`fw_columns_a_gpu` on the
// source page bixverse-rs 0.6.4, seacells_kernels.rs).
//
// One wave64 owns one cell at a time (persistent waves, grid-stride over
// cells). Its state is the dense k-vector of the gradient, held in LDS
// (or in a workspace slice when k is too large for LDS), plus the cell's
// atom list in LDS.
//
// The state is kept as g = s * h with a scalar s, where g = t1 . a - t2 is
// the page's gradient (t2 = row of K2B). A step
//     g <- (1 - gamma) g + gamma (t1[idx, :] - t2)
// becomes s <- (1 - gamma) s and h <- h + (gamma / s) (t1[idx, :] - t2):
// the (1 - gamma) scaling of all k entries, which the page pays as a dense
// pass per step, is a scalar update here, and each step only touches the
// non-zeros of one t1 row and of t2. gamma = 1 restarts from
// h = t1[idx, :] - t2, s = 1. Since s > 0, argmin g = argmin h.
//
// The argmin is a float4 scan of h (lowest column within a lane under a
// strict `<`), then a wave-wide minimum of the (order-preserving f32 key,
// column) pair, which gives the lowest column on a tie as the page requires.
#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kABlockMaxThreads = 256;

// Clamp a CSR row range to the stored entries; a malformed row pointer
// becomes an empty row and a flag instead of a stray access.
__device__ __forceinline__ void row_range(const Csr &m, uint32_t r, uint32_t &lo, uint32_t &hi,
                                          uint32_t &flags) {
  lo = m.ptr[r];
  hi = m.ptr[r + 1];
  if (hi > m.nnz || lo > hi) {
    flags |= kFlagBadIndex;
    lo = hi = 0;
  }
}

template <bool kHInLds>
__global__ void __launch_bounds__(kABlockMaxThreads)
    fw_a_columns_kernel(Csr t1, Csr k2b, Csr ap, uint32_t n, uint32_t k, uint32_t kpad, uint32_t T,
                        uint32_t cap, const float *__restrict__ gamma,
                        uint32_t *__restrict__ atom_idx, float *__restrict__ atom_val,
                        uint32_t *__restrict__ atom_cnt, uint32_t *__restrict__ trace,
                        float *__restrict__ h_ws, uint32_t lds_words_per_wave,
                        uint32_t *__restrict__ status) {
  extern __shared__ uint32_t lds[];
  const uint32_t lane = lane_id();
  const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t wpb = blockDim.x / kWave;
  const uint32_t gwave = blockIdx.x * wpb + wib;
  const uint32_t nwaves = gridDim.x * wpb;
  uint32_t *wl = lds + (size_t)wib * lds_words_per_wave;
  float *h;
  uint32_t *s_aidx;
  if constexpr (kHInLds) {
    h = reinterpret_cast<float *>(wl);
    s_aidx = wl + kpad;
  } else {
    h = h_ws + (size_t)gwave * kpad;
    s_aidx = wl;
  }
  float *s_aval = reinterpret_cast<float *>(s_aidx + cap);
  const float inf = __builtin_inff();
  uint32_t flags = 0;

  for (uint32_t cell = gwave; cell < n; cell += nwaves) {
    // -- clear: h = 0 on [0, k), +inf on the padding [k, kpad)
    for (uint32_t c = lane * 4; c < kpad; c += 4 * kWave) {
      float4 z;
      z.x = (c + 0 < k) ? 0.0f : inf;
      z.y = (c + 1 < k) ? 0.0f : inf;
      z.z = (c + 2 < k) ? 0.0f : inf;
      z.w = (c + 3 < k) ? 0.0f : inf;
      *reinterpret_cast<float4 *>(h + c) = z;
    }
    // -- seed the atoms from A_prev's column
    uint32_t s0, s1;
    row_range(ap, cell, s0, s1, flags);
    uint32_t cnt = s1 - s0;
    if (cnt > cap) {
      flags |= kFlagCapOverflow;
      cnt = cap;
    }
    for (uint32_t s = lane; s < cnt; s += kWave) {
      s_aidx[s] = ap.idx[s0 + s];
      s_aval[s] = ap.val[s0 + s];
    }
    wave_lds_sync();
    // -- h = t1 . a_prev : one t1 row per seed, scaled by its weight
    for (uint32_t s = s0; s < s1; ++s) {
      const uint32_t m = ap.idx[s];
      const float am = ap.val[s];
      if (m >= k) {
        flags |= kFlagBadIndex;
        continue;
      }
      uint32_t p0, p1;
      row_range(t1, m, p0, p1, flags);
      for (uint32_t p = p0 + lane; p < p1; p += kWave) {
        const uint32_t c = t1.idx[p];
        if (c < k) h[c] += am * t1.val[p];
      }
      wave_lds_sync();
    }
    // -- h -= t2 (this cell's row of K2B)
    uint32_t q0, q1;
    row_range(k2b, cell, q0, q1, flags);
    for (uint32_t q = q0 + lane; q < q1; q += kWave) {
      const uint32_t c = k2b.idx[q];
      if (c < k) h[c] -= k2b.val[q];
    }
    wave_lds_sync();

    float sc = 1.0f;  // g = sc * h
    for (uint32_t t = 0; t < T; ++t) {
      // -- argmin_c h[c], lowest column on a tie
      float bv = inf;
      uint32_t bi = 0xffffffffu;
      for (uint32_t c = lane * 4; c < kpad; c += 4 * kWave) {
        const float4 v = *reinterpret_cast<const float4 *>(h + c);
        if (v.x < bv) bv = v.x, bi = c;
        if (v.y < bv) bv = v.y, bi = c + 1;
        if (v.z < bv) bv = v.z, bi = c + 2;
        if (v.w < bv) bv = v.w, bi = c + 3;
      }
      uint32_t idx = wave_argmin(bv, bi);
      if (idx >= k) {  // only when no entry compares below +inf (NaN state)
        flags |= kFlagNonfinite;
        idx = 0;
      }
      if (trace != nullptr && lane == 0) trace[(size_t)cell * T + t] = idx;

      const float gam = gamma != nullptr ? gamma[t] : 2.0f / (float)(t + 2u);
      if (!(gam > 0.0f && gam <= 1.0f)) flags |= kFlagBadGamma;
      const float keep = 1.0f - gam;

      // -- atoms: scale every weight, add gamma at idx or append idx
      bool found = false;
      for (uint32_t s = lane; s < cnt; s += kWave) {
        float v = s_aval[s] * keep;
        if (s_aidx[s] == idx) {
          v += gam;
          found = true;
        }
        s_aval[s] = v;
      }
      if (__ballot(found) == 0) {
        if (cnt < cap) {
          if (lane == 0) {
            s_aidx[cnt] = idx;
            s_aval[cnt] = gam;
          }
          ++cnt;
        } else {
          flags |= kFlagCapOverflow;
        }
      }

      // -- state: lazy scale, or restart when gamma == 1
      float alpha;
      if (keep == 0.0f) {
        for (uint32_t c = lane * 4; c < kpad; c += 4 * kWave) {
          float4 z;
          z.x = (c + 0 < k) ? 0.0f : inf;
          z.y = (c + 1 < k) ? 0.0f : inf;
          z.z = (c + 2 < k) ? 0.0f : inf;
          z.w = (c + 3 < k) ? 0.0f : inf;
          *reinterpret_cast<float4 *>(h + c) = z;
        }
        sc = 1.0f;
        alpha = 1.0f;
        wave_lds_sync();
      } else {
        sc *= keep;
        if (sc < 0x1p-64f) {  // fold the scale back in before h grows too large
          for (uint32_t c = lane * 4; c < kpad; c += 4 * kWave) {
            float4 v = *reinterpret_cast<float4 *>(h + c);
            v.x *= sc, v.y *= sc, v.z *= sc, v.w *= sc;
            *reinterpret_cast<float4 *>(h + c) = v;
          }
          sc = 1.0f;
          wave_lds_sync();
        }
        alpha = gam / sc;
      }
      // -- h += alpha * t1[idx, :]  (columns of one row are unique)
      uint32_t p0, p1;
      row_range(t1, idx, p0, p1, flags);
      for (uint32_t p = p0 + lane; p < p1; p += kWave) {
        const uint32_t c = t1.idx[p];
        if (c < k) h[c] += alpha * t1.val[p];
      }
      wave_lds_sync();
      // -- h -= alpha * t2
      for (uint32_t q = q0 + lane; q < q1; q += kWave) {
        const uint32_t c = k2b.idx[q];
        if (c < k) h[c] -= alpha * k2b.val[q];
      }
      wave_lds_sync();
    }

    // -- write the atoms
    const size_t base = (size_t)cell * cap;
    for (uint32_t s = lane; s < cnt; s += kWave) {
      atom_idx[base + s] = s_aidx[s];
      atom_val[base + s] = s_aval[s];
    }
    if (lane == 0) atom_cnt[cell] = cnt;
    wave_lds_sync();
  }
  flags = __builtin_amdgcn_readfirstlane(flags);
  if (flags != 0 && lane == 0) atomicOr(status, flags);
}

template <bool kHInLds>
hipError_t configure(uint32_t lds_bytes, uint32_t threads, int *blocks_per_cu) {
  static bool set[2] = {false, false};
  hipError_t e = hipSuccess;
  auto fn = reinterpret_cast<const void *>(&fw_a_columns_kernel<kHInLds>);
  if (!set[kHInLds]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytesPerCU);
    if (e != hipSuccess) return e;
    set[kHInLds] = true;
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, threads, lds_bytes);
}

}  // namespace

APlan plan_a(uint32_t n, uint32_t k, uint32_t T, uint32_t cap) {
  (void)T;
  APlan p{};
  p.kpad = (k + 3u) & ~3u;
  const size_t atom_words = align_up(2 * (size_t)cap, 4);
  const size_t lds_words = align_up((size_t)p.kpad + atom_words, 4);
  if (lds_words * 4 <= kLdsBytesPerCU) {
    p.h_in_lds = true;
    p.lds_per_wave = (uint32_t)(lds_words * 4);
    uint32_t w = (uint32_t)(kLdsBytesPerCU / p.lds_per_wave);
    p.waves_per_block = w >= 4 ? 4 : (w >= 2 ? 2 : 1);
    p.global_waves = 0;
    p.ws_bytes = 0;
  } else {
    p.h_in_lds = false;
    p.lds_per_wave = (uint32_t)(atom_words * 4);
    const uint32_t w = (uint32_t)(kLdsBytesPerCU / p.lds_per_wave);  // >= 1: cap checked by the caller
    p.waves_per_block = w >= 4 ? 4 : (w >= 2 ? 2 : 1);
    const uint32_t gw = n < 8192u ? n : 8192u;
    p.global_waves = (gw + p.waves_per_block - 1) / p.waves_per_block * p.waves_per_block;
    p.ws_bytes = align_up((size_t)p.global_waves * p.kpad * sizeof(float), 256);
  }
  return p;
}

hipError_t launch_fw_a(const APlan &plan, Csr t1, Csr k2b, Csr ap, uint32_t n, uint32_t k,
                       uint32_t T, uint32_t cap, const float *gamma, uint32_t *atom_idx,
                       float *atom_val, uint32_t *atom_cnt, uint32_t *trace, void *ws,
                       uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  const uint32_t wpb = plan.waves_per_block;
  const uint32_t threads = wpb * kWave;
  const uint32_t lds_bytes = wpb * plan.lds_per_wave;
  const uint32_t lds_words_per_wave = plan.lds_per_wave / 4;
  if (plan.h_in_lds) {
    int bpc = 0;
    e = configure<true>(lds_bytes, threads, &bpc);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    const uint64_t want = (n + wpb - 1) / wpb;
    const uint64_t cap_blocks = (uint64_t)dev.cus * (uint64_t)bpc;
    const uint32_t blocks = (uint32_t)(want < cap_blocks ? want : cap_blocks);
    hipLaunchKernelGGL(fw_a_columns_kernel<true>, dim3(blocks), dim3(threads), lds_bytes, stream,
                       t1, k2b, ap, n, k, plan.kpad, T, cap, gamma,
                       atom_idx, atom_val, atom_cnt, trace, nullptr, lds_words_per_wave, status);
  } else {
    int bpc = 0;
    e = configure<false>(lds_bytes, threads, &bpc);
    if (e != hipSuccess) return e;
    const uint32_t blocks = plan.global_waves / wpb;
    hipLaunchKernelGGL(fw_a_columns_kernel<false>, dim3(blocks), dim3(threads), lds_bytes, stream,
                       t1, k2b, ap, n, k, plan.kpad, T, cap, gamma,
                       atom_idx, atom_val, atom_cnt, trace, static_cast<float *>(ws),
                       lds_words_per_wave, status);
  }
  return hipGetLastError();
}

}  // namespace seacells
