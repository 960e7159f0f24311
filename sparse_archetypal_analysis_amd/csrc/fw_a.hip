// A update: the per-cell Frank-Wolfe column solve (`fw_columns_a_gpu` on the
// source page bixverse-rs 0.6.4, seacells_kernels.rs).
//
// One wave64 owns one cell at a time (persistent waves, grid-stride over
// cells). Its state is the dense k-vector of the gradient, held in LDS (or
// in a workspace slice when k is too large for LDS); the cell's atoms live
// in registers (two slots per lane) or, for a large capacity, in LDS.
//
// The state is kept as g = s * h with a scalar s, where g = t1 . a - t2 is
// the page's gradient (t2 = the cell's row of K2B). A step
//     g <- (1 - gamma) g + gamma (t1[idx, :] - t2)
// becomes s <- (1 - gamma) s and h <- h + (gamma / s) (t1[idx, :] - t2):
// the (1 - gamma) scaling of all k entries, which the page pays as a dense
// pass per step, is a scalar update here, and each step only touches the
// non-zeros of one t1 row and of t2. gamma = 1 restarts from
// h = t1[idx, :] - t2, s = 1. Since s > 0, argmin g = argmin h. The scalar
// schedule (gamma, 1 - gamma, gamma / s, restarts, and folding s back into
// h when it underflows) is the same for every cell, so each block computes
// it once into LDS.
//
// Argmin. While every product added into h is >= 0 (kernel data: t1, K2B
// and A_prev are non-negative), h[c] >= 0 for every c outside supp(t2). If
// the minimum of h over supp(t2) is negative it is then the global minimum,
// and it comes for free from the pass that subtracts t2 each step (lowest
// column among equal values). Otherwise, and always once a negative product
// has been added (until the next restart), a dense scan decides. Both give
// the index a dense scan of the same f32 state gives.
//
// Dense scan: uniform-trip float4 chunks (the state is padded with +inf to a
// multiple of 256 columns, with at least one padding column), per-chunk
// min3, the first chunk holding each lane's minimum, then a wave minimum of
// the order-preserving f32 key and of the column among the lanes holding it
// (lowest column on a tie, -0 == +0).
//
// Lanes with nothing to do in a sparse pass point at the first padding
// column (value +inf, added weight 0), so the passes run with uniform trip
// counts and no per-lane branches.
#include <stdlib.h>

#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kABlockMaxThreads = 256;
constexpr uint32_t kSchedMax = 256;    // steps whose schedule is tabulated in LDS
constexpr uint32_t kT2Regs = 4;        // chunks of 64 t2 entries held in registers
constexpr uint32_t kAtomSlots = 2;     // atom slots per lane when atoms live in registers
constexpr uint32_t kNone = 0xffffffffu;

struct StepSched {
  float gam;    // gamma_t
  float keep;   // 1 - gamma_t; 0 means restart
  float alpha;  // gamma_t / s_t after any restart or fold
  float fold;   // > 0: multiply h by this before the update (scale folded back)
};

__device__ __forceinline__ StepSched sched_step(const float *gamma, uint32_t t, float &s,
                                                uint32_t &flags) {
  StepSched r;
  r.gam = gamma != nullptr ? gamma[t] : 2.0f / (float)(t + 2u);
  if (!(r.gam > 0.0f && r.gam <= 1.0f)) flags |= kFlagBadGamma;
  r.keep = 1.0f - r.gam;
  r.fold = 0.0f;
  if (r.keep == 0.0f) {
    s = 1.0f;
    r.alpha = 1.0f;
  } else {
    s *= r.keep;
    if (s < 0x1p-64f) {  // fold the scale back in before h grows too large
      r.fold = s;
      s = 1.0f;
    }
    r.alpha = r.gam / s;
  }
  return r;
}

// Fill h with 0 on [0, k) and +inf on the padding [k, nch * 256).
__device__ __forceinline__ void clear_state(float *h, uint32_t k, uint32_t nch, uint32_t lane) {
  const float inf = __builtin_inff();
  for (uint32_t i = 0; i < nch; ++i) {
    const uint32_t c = i * 256 + lane * 4;
    float4 z;
    z.x = (c + 0 < k) ? 0.0f : inf;
    z.y = (c + 1 < k) ? 0.0f : inf;
    z.z = (c + 2 < k) ? 0.0f : inf;
    z.w = (c + 3 < k) ? 0.0f : inf;
    *reinterpret_cast<float4 *>(h + c) = z;
  }
}

// Exact argmin of h over [0, nch * 256) (padding holds +inf).
__device__ __forceinline__ uint32_t dense_argmin(const float *h, uint32_t nch, uint32_t lane) {
  const float *p = h + lane * 4;
  float bv = __builtin_inff();
  uint32_t bch = 0;
  for (uint32_t i = 0; i < nch; ++i) {
    const float4 v = *reinterpret_cast<const float4 *>(p + i * 256);
    const float m = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
    if (m < bv) bv = m, bch = i;
  }
  const uint32_t key = f32_order(bv);
  const uint32_t best = wave_min_u32(key);
  uint32_t cand = kNone;
  if (key == best) {
    const float4 v = *reinterpret_cast<const float4 *>(p + bch * 256);
    const uint32_t j = (v.x == bv) ? 0u : (v.y == bv) ? 1u : (v.z == bv) ? 2u : 3u;
    cand = bch * 256 + lane * 4 + j;
  }
  return wave_min_u32(cand);
}

template <bool kHInLds, bool kRegAtoms>
__global__ void __launch_bounds__(kABlockMaxThreads)
    fw_a_columns_kernel(const uint32_t *__restrict__ t1_ptr, const uint32_t *__restrict__ t1_idx,
                        const float *__restrict__ t1_val, uint32_t t1_nnz,
                        const uint32_t *__restrict__ k2b_ptr, const uint32_t *__restrict__ k2b_idx,
                        const float *__restrict__ k2b_val, uint32_t k2b_nnz,
                        const uint32_t *__restrict__ ap_ptr, const uint32_t *__restrict__ ap_idx,
                        const float *__restrict__ ap_val, uint32_t ap_nnz, uint32_t n,
                        uint32_t k, uint32_t kscan, uint32_t T, uint32_t cap,
                        const float *__restrict__ gamma, uint32_t *__restrict__ atom_idx,
                        float *__restrict__ atom_val, uint32_t *__restrict__ atom_cnt,
                        uint32_t *__restrict__ trace, float *__restrict__ state_ws,
                        uint32_t sched_words, uint32_t lds_words_per_wave, uint32_t dense_only,
                        uint32_t *__restrict__ status) {
  extern __shared__ uint32_t lds[];
  const uint32_t lane = lane_id();
  const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t wpb = blockDim.x / kWave;
  const uint32_t gwave = blockIdx.x * wpb + wib;
  const uint32_t nwaves = gridDim.x * wpb;
  uint32_t flags = 0;

  // -- the step schedule, once per block
  const StepSched *sched = reinterpret_cast<const StepSched *>(lds);
  if (sched_words != 0) {
    if (threadIdx.x == 0) {
      StepSched *w = reinterpret_cast<StepSched *>(lds);
      float s = 1.0f;
      uint32_t f = 0;
      for (uint32_t t = 0; t < T; ++t) w[t] = sched_step(gamma, t, s, f);
      lds[sched_words - 1] = f;
    }
    __syncthreads();
    flags |= lds[sched_words - 1];
  }

  uint32_t *wl = lds + sched_words + (size_t)wib * lds_words_per_wave;
  float *h = kHInLds ? reinterpret_cast<float *>(wl) : state_ws + (size_t)gwave * kscan;
  uint32_t *s_aidx = kHInLds ? wl + kscan : wl;          // LDS atoms (large cap only)
  float *s_aval = reinterpret_cast<float *>(s_aidx + ((cap + 3u) & ~3u));
  const uint32_t nch = kscan / 256;
  const uint32_t dummy = k;  // first padding column: holds +inf
  const float inf = __builtin_inff();

  // h += alpha * (row r of t1); columns of one row are unique, so no two
  // lanes touch the same column. Returns whether some product was negative.
  auto scatter_row = [&](uint32_t r, float alpha) -> bool {
    uint32_t p0 = t1_ptr[r], p1 = t1_ptr[r + 1];
    if (p1 > t1_nnz || p0 > p1) {
      flags |= kFlagBadIndex;
      p0 = p1 = 0;
    }
    const uint32_t nit = (p1 - p0 + kWave - 1) / kWave;
    bool lane_neg = false;
    for (uint32_t i = 0; i < nit; ++i) {
      const uint32_t p = p0 + i * kWave + lane;
      const bool valid = p < p1;
      const uint32_t pc = valid ? p : p1 - 1;
      uint32_t c = t1_idx[pc];
      float v = t1_val[pc];
      if (c >= k) {
        if (valid) flags |= kFlagBadIndex;
        c = dummy;
        v = 0.0f;
      }
      if (!valid) c = dummy, v = 0.0f;
      h[c] = h[c] + alpha * v;
      lane_neg |= (v < 0.0f);
    }
    return __ballot(lane_neg) != 0;
  };

  for (uint32_t cell = gwave; cell < n; cell += nwaves) {
    // -- t2 = this cell's K2B row: the first kT2Regs * 64 entries in registers
    uint32_t q0 = k2b_ptr[cell], q1 = k2b_ptr[cell + 1];
    if (q1 > k2b_nnz || q0 > q1) {
      flags |= kFlagBadIndex;
      q0 = q1 = 0;
    }
    const uint32_t nq_chunks = (q1 - q0 + kWave - 1) / kWave;
    const uint32_t nchk = nq_chunks < kT2Regs ? nq_chunks : kT2Regs;
    uint32_t t2c[kT2Regs];
    float t2v[kT2Regs];
#pragma unroll
    for (uint32_t r = 0; r < kT2Regs; ++r) {
      t2c[r] = dummy;
      t2v[r] = 0.0f;
      if (r < nchk) {
        const uint32_t q = q0 + r * kWave + lane;
        if (q < q1) {
          const uint32_t c = k2b_idx[q];
          if (c < k)
            t2c[r] = c, t2v[r] = k2b_val[q];
          else
            flags |= kFlagBadIndex;
        }
      }
    }
    const uint32_t q_extra = q0 + kT2Regs * kWave;  // entries past the registers

    clear_state(h, k, nch, lane);

    // -- seed the atoms from A_prev's column
    uint32_t s0 = ap_ptr[cell], s1 = ap_ptr[cell + 1];
    if (s1 > ap_nnz || s0 > s1) {
      flags |= kFlagBadIndex;
      s0 = s1 = 0;
    }
    uint32_t cnt = s1 - s0;
    if (cnt > cap) {
      flags |= kFlagCapOverflow;
      cnt = cap;
    }
    uint32_t aidx[kAtomSlots];
    float aval[kAtomSlots];
    if constexpr (kRegAtoms) {
#pragma unroll
      for (uint32_t j = 0; j < kAtomSlots; ++j) {
        const uint32_t s = j * kWave + lane;
        aidx[j] = s < cnt ? ap_idx[s0 + s] : kNone;
        aval[j] = s < cnt ? ap_val[s0 + s] : 0.0f;
      }
    } else {
      for (uint32_t s = lane; s < cnt; s += kWave) {
        s_aidx[s] = ap_idx[s0 + s];
        s_aval[s] = ap_val[s0 + s];
      }
    }
    wave_lds_sync();

    // -- h = t1 . a_prev : one t1 row per seed, scaled by its weight
    bool mono = dense_only == 0;
    for (uint32_t s = s0; s < s1; ++s) {
      const uint32_t m = ap_idx[s];
      const float am = ap_val[s];
      if (m >= k) {
        flags |= kFlagBadIndex;
        continue;
      }
      if (am < 0.0f) mono = false;
      if (scatter_row(m, am)) mono = false;
      wave_lds_sync();
    }

    // -- h -= alpha * t2, and the minimum of h over supp(t2)
    float mval;
    uint32_t midx;
    auto t2_pass = [&](float alpha) {
      float bv = inf;
      uint32_t bi = kNone, br = 0;
#pragma unroll
      for (uint32_t r = 0; r < kT2Regs; ++r) {
        if (r < nchk) {
          const uint32_t c = t2c[r];
          const float hn = h[c] - alpha * t2v[r];
          h[c] = hn;
          if (hn < bv) bv = hn, bi = c, br = r;
        }
      }
      uint32_t nr = nchk;
      for (uint32_t qb = q_extra; qb < q1; qb += kWave, ++nr) {  // rows longer than 256
        const uint32_t q = qb + lane;
        if (q < q1) {
          const uint32_t c = k2b_idx[q];
          if (c < k) {
            const float hn = h[c] - alpha * k2b_val[q];
            h[c] = hn;
            if (hn < bv) bv = hn, bi = c, br = nr;
          }
        }
      }
      // minimum value key over the wave, then the lowest column holding it:
      // entries are ascending in (chunk, lane) order, so the first chunk with
      // a matching lane and, in it, the lowest matching lane win
      const uint32_t key = f32_order(bv);
      const uint32_t best = wave_min_u32(key);
      mval = f32_unorder(best);
      midx = kNone;
      for (uint32_t r = 0; r < nr; ++r) {
        const uint64_t m = __ballot(key == best && br == r && bi != kNone);
        if (m != 0) {
          midx = readlane_u32(bi, (uint32_t)__builtin_ctzll(m));
          break;
        }
      }
    };
    t2_pass(1.0f);
    wave_lds_sync();

    float s_run = 1.0f;
    for (uint32_t t = 0; t < T; ++t) {
      const StepSched sc = sched_words != 0 ? sched[t] : sched_step(gamma, t, s_run, flags);

      // -- argmin_c h[c], lowest column on a tie
      uint32_t idx = (mono && mval < 0.0f) ? midx : dense_argmin(h, nch, lane);
      if (idx >= k) {  // only when no entry compares below +inf (NaN state)
        flags |= kFlagNonfinite;
        idx = 0;
      }
      if (trace != nullptr && lane == 0) trace[(size_t)cell * T + t] = idx;

      // -- atoms: scale every weight, add gamma at idx or append idx
      bool hit = false;
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < kAtomSlots; ++j) {
          float v = aval[j] * sc.keep;
          if (aidx[j] == idx) v += sc.gam, hit = true;
          aval[j] = v;
        }
      } else {
        for (uint32_t s = lane; s < cnt; s += kWave) {
          float v = s_aval[s] * sc.keep;
          if (s_aidx[s] == idx) v += sc.gam, hit = true;
          s_aval[s] = v;
        }
      }
      if (__ballot(hit) == 0) {
        if (cnt < cap) {
          if constexpr (kRegAtoms) {
            const uint32_t j = cnt / kWave, l = cnt % kWave;
#pragma unroll
            for (uint32_t jj = 0; jj < kAtomSlots; ++jj)
              if (jj == j && lane == l) aidx[jj] = idx, aval[jj] = sc.gam;
          } else if (lane == 0) {
            s_aidx[cnt] = idx;
            s_aval[cnt] = sc.gam;
          }
          ++cnt;
        } else {
          flags |= kFlagCapOverflow;
        }
      }

      // -- state: restart when gamma == 1, fold the scale back in when due
      if (sc.keep == 0.0f) {
        clear_state(h, k, nch, lane);
        mono = dense_only == 0;
      } else if (sc.fold > 0.0f) {
        for (uint32_t i = 0; i < nch; ++i) {
          float4 *q = reinterpret_cast<float4 *>(h + i * 256 + lane * 4);
          float4 v = *q;
          v.x *= sc.fold, v.y *= sc.fold, v.z *= sc.fold, v.w *= sc.fold;
          *q = v;
        }
        mono = false;
      }
      wave_lds_sync();
      // -- h += alpha * t1[idx, :]
      if (scatter_row(idx, sc.alpha)) mono = false;
      wave_lds_sync();
      // -- h -= alpha * t2
      t2_pass(sc.alpha);
      wave_lds_sync();
    }

    // -- write the atoms
    const size_t base = (size_t)cell * cap;
    if constexpr (kRegAtoms) {
#pragma unroll
      for (uint32_t j = 0; j < kAtomSlots; ++j) {
        const uint32_t s = j * kWave + lane;
        if (s < cnt) {
          atom_idx[base + s] = aidx[j];
          atom_val[base + s] = aval[j];
        }
      }
    } else {
      for (uint32_t s = lane; s < cnt; s += kWave) {
        atom_idx[base + s] = s_aidx[s];
        atom_val[base + s] = s_aval[s];
      }
    }
    if (lane == 0) atom_cnt[cell] = cnt;
    wave_lds_sync();
  }
  // some flags are raised by single lanes: every lane that saw one reports it
  if (flags != 0) atomicOr(status, flags);
}

template <bool kHInLds, bool kRegAtoms>
hipError_t launch_variant(const APlan &plan, const DeviceInfo &dev, Csr t1, Csr k2b, Csr ap,
                          uint32_t n, uint32_t k, uint32_t T, uint32_t cap, const float *gamma,
                          uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                          uint32_t *trace, void *ws, uint32_t dense_only, uint32_t *status,
                          hipStream_t stream) {
  static bool configured = false;
  auto fn = reinterpret_cast<const void *>(&fw_a_columns_kernel<kHInLds, kRegAtoms>);
  const uint32_t wpb = plan.waves_per_block;
  const uint32_t threads = wpb * kWave;
  const uint32_t lds_bytes = plan.sched_words * 4 + wpb * plan.lds_per_wave;
  hipError_t e;
  if (!configured) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytesPerCU);
    if (e != hipSuccess) return e;
    configured = true;
  }
  uint32_t blocks;
  if (kHInLds) {
    int bpc = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, fn, threads, lds_bytes);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    const uint64_t want = (n + wpb - 1) / wpb;
    const uint64_t cap_blocks = (uint64_t)dev.cus * (uint64_t)bpc;
    blocks = (uint32_t)(want < cap_blocks ? want : cap_blocks);
  } else {
    blocks = plan.global_waves / wpb;  // each wave owns one workspace slice
  }
  hipLaunchKernelGGL((fw_a_columns_kernel<kHInLds, kRegAtoms>), dim3(blocks), dim3(threads),
                     lds_bytes, stream, t1.ptr, t1.idx, t1.val, t1.nnz, k2b.ptr, k2b.idx,
                     k2b.val, k2b.nnz, ap.ptr, ap.idx, ap.val, ap.nnz, n, k, plan.kpad, T, cap,
                     gamma, atom_idx, atom_val, atom_cnt, trace, static_cast<float *>(ws),
                     plan.sched_words, plan.lds_per_wave / 4, dense_only, status);
  return hipGetLastError();
}

bool dense_only_requested() {
  const char *v = getenv("SEACELLS_A_DENSE_ARGMIN");
  return v != nullptr && v[0] == '1';
}

}  // namespace

APlan plan_a(uint32_t n, uint32_t k, uint32_t T, uint32_t cap) {
  APlan p{};
  p.kpad = (uint32_t)align_up((size_t)k + 1, 256);  // scan length, >= 1 padding column
  p.reg_atoms = cap <= kAtomSlots * kWave;
  const size_t atom_words = p.reg_atoms ? 0 : 2 * align_up(cap, 4);
  p.sched_words = T <= kSchedMax ? (uint32_t)(T * (sizeof(StepSched) / 4) + 4) : 0u;
  const size_t budget = kLdsBytesPerCU - (size_t)p.sched_words * 4;
  const size_t lds_words = align_up((size_t)p.kpad + atom_words, 4);
  if (lds_words * 4 <= budget) {
    p.h_in_lds = true;
    p.lds_per_wave = (uint32_t)(lds_words * 4);
    const uint32_t w = (uint32_t)(budget / p.lds_per_wave);
    p.waves_per_block = w >= 4 ? 4 : (w >= 2 ? 2 : 1);
    p.global_waves = 0;
    p.ws_words_per_wave = 0;
    p.ws_bytes = 0;
  } else {
    p.h_in_lds = false;
    p.lds_per_wave = (uint32_t)(atom_words * 4);
    const uint32_t w = p.lds_per_wave ? (uint32_t)(budget / p.lds_per_wave) : 4u;
    p.waves_per_block = w >= 4 ? 4 : (w >= 2 ? 2 : w);  // 0: atoms alone exceed LDS
    if (p.waves_per_block == 0) return p;
    const uint32_t gw = n < 8192u ? n : 8192u;
    p.global_waves = (gw + p.waves_per_block - 1) / p.waves_per_block * p.waves_per_block;
    p.ws_words_per_wave = p.kpad;
    p.ws_bytes = align_up((size_t)p.global_waves * p.ws_words_per_wave * 4, 256);
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
  const uint32_t dense_only = dense_only_requested() ? 1u : 0u;
#define SEACELLS_A_ARGS \
  plan, dev, t1, k2b, ap, n, k, T, cap, gamma, atom_idx, atom_val, atom_cnt, trace, ws, \
      dense_only, status, stream
  if (plan.h_in_lds)
    return plan.reg_atoms ? launch_variant<true, true>(SEACELLS_A_ARGS)
                          : launch_variant<true, false>(SEACELLS_A_ARGS);
  return plan.reg_atoms ? launch_variant<false, true>(SEACELLS_A_ARGS)
                        : launch_variant<false, false>(SEACELLS_A_ARGS);
#undef SEACELLS_A_ARGS
}

}  // namespace seacells
