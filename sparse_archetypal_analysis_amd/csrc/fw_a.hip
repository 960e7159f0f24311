// A update: the per-cell Frank-Wolfe column solve (`fw_columns_a_gpu` on the
// source page bixverse-rs 0.6.4, seacells_kernels.rs).
//
// A lane group of G lanes (G = 16, 32 or 64; 64 / G cells per wave64) owns
// one cell at a time; waves are persistent and grid-stride over cells. A
// cell's state is the dense k-vector of the gradient, held in LDS (or in a
// workspace slice when k is too large for LDS); its atoms live in registers
// (up to 128 per cell) or, for a larger capacity, in LDS. The per-step work
// of one cell is small (one sparse t1 row and the cell's K2B row), so
// several cells share each instruction: the fixed cost of a step (two group
// reductions, atom update, control) is paid once per 64 / G cells.
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
// Dense scan: float4 chunks (the state is padded with +inf to a multiple of
// 4G columns, with at least one padding column), per-chunk min3, the first
// chunk holding each lane's minimum, then a group minimum of the
// order-preserving f32 key and of the column among the lanes holding it
// (lowest column on a tie, -0 == +0).
//
// Lanes with nothing to do in a sparse pass point at the first padding
// column (value +inf, added weight 0).
#include <stdlib.h>

#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kABlockMaxThreads = 256;
constexpr uint32_t kSchedMax = 256;   // steps whose schedule is tabulated in LDS
constexpr uint32_t kT2Regs = 4;       // chunks of G t2 entries held in registers
constexpr uint32_t kRegAtomMax = 128; // atoms per cell held in registers
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

// Minimum of a u32 over each group of G consecutive lanes; every lane of a
// group receives its group's minimum. Same butterfly as wave_min_u32,
// stopped at the group width.
template <uint32_t G>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0xB1, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x4E, 0xF, 0xF, false));
  if constexpr (G >= 8)
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x141, 0xF, 0xF, false));
  if constexpr (G >= 16)
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)x, 0x140, 0xF, 0xF, false));
  if constexpr (G >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = min(x, min((uint32_t)r[0], (uint32_t)r[1]));
  }
  if constexpr (G >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = min(x, min((uint32_t)r[0], (uint32_t)r[1]));
    return __builtin_amdgcn_readfirstlane(x);  // wave-uniform: keeps what follows scalar
  }
  return x;
}

// (ptr[r], ptr[r + 1]) for this lane's group, where r is uniform within each
// group: one scalar load per group (through the scalar cache), then a select.
template <uint32_t G>
__device__ __forceinline__ void group_load_pair(const uint32_t *__restrict__ ptr, uint32_t r,
                                                uint32_t grp, uint32_t &lo, uint32_t &hi) {
  constexpr uint32_t CPW = kWave / G;
  uint32_t l = 0, h = 0;
#pragma unroll
  for (uint32_t g = 0; g < CPW; ++g) {
    const uint32_t rg = __builtin_amdgcn_readlane((int)r, g * G);
    const uint32_t a = ptr[rg], b = ptr[rg + 1];
    if (g == 0 || grp == g) l = a, h = b;
  }
  lo = l;
  hi = h;
}

// ptr[r] for this lane's group (r uniform within each group), as above.
template <uint32_t G, typename V>
__device__ __forceinline__ V group_load(const V *__restrict__ ptr, uint32_t r, uint32_t grp) {
  constexpr uint32_t CPW = kWave / G;
  V out{};
#pragma unroll
  for (uint32_t g = 0; g < CPW; ++g) {
    const uint32_t rg = __builtin_amdgcn_readlane((int)r, g * G);
    const V a = ptr[rg];
    if (g == 0 || grp == g) out = a;
  }
  return out;
}

// Bits of the lanes of this lane's group in a 64-bit ballot.
template <uint32_t G>
__device__ __forceinline__ uint64_t group_mask(uint32_t grp) {
  if constexpr (G == 64) return ~0ull;
  return ((1ull << G) - 1ull) << (grp * G);
}

// Fill h with 0 on [0, k) and +inf on the padding [k, kscan).
template <uint32_t G>
__device__ __forceinline__ void clear_state(float *h, uint32_t k, uint32_t nch, uint32_t gl) {
  const float inf = __builtin_inff();
  for (uint32_t i = 0; i < nch; ++i) {
    const uint32_t c = i * 4 * G + gl * 4;
    float4 z;
    z.x = (c + 0 < k) ? 0.0f : inf;
    z.y = (c + 1 < k) ? 0.0f : inf;
    z.z = (c + 2 < k) ? 0.0f : inf;
    z.w = (c + 3 < k) ? 0.0f : inf;
    *reinterpret_cast<float4 *>(h + c) = z;
  }
}

// Exact argmin of each group's h over [0, nch * 4G) (padding holds +inf).
template <uint32_t G>
__device__ __forceinline__ uint32_t dense_argmin(const float *h, uint32_t nch, uint32_t gl) {
  const float *p = h + gl * 4;
  float bv = __builtin_inff();
  uint32_t bch = 0;
  for (uint32_t i = 0; i < nch; ++i) {
    const float4 v = *reinterpret_cast<const float4 *>(p + i * 4 * G);
    const float m = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
    if (m < bv) bv = m, bch = i;
  }
  const uint32_t key = f32_order(bv);
  const uint32_t best = group_min_u32<G>(key);
  uint32_t cand = kNone;
  if (key == best) {
    const float4 v = *reinterpret_cast<const float4 *>(p + bch * 4 * G);
    const uint32_t j = (v.x == bv) ? 0u : (v.y == bv) ? 1u : (v.z == bv) ? 2u : 3u;
    cand = bch * 4 * G + gl * 4 + j;
  }
  return group_min_u32<G>(cand);
}

// One cell per wave64 (k above 1024): every per-cell value is wave-uniform
// and stays on the scalar unit (row pointers through the scalar cache,
// uniform trip counts, a ballot walk for the index of the t2 minimum).
constexpr uint32_t kWaveAtomSlots = 2;  // atom slots per lane in registers

template <bool kHInLds, bool kRegAtoms>
__global__ void __launch_bounds__(kABlockMaxThreads)
    fw_a_wave_kernel(const uint32_t *__restrict__ t1_ptr, const uint32_t *__restrict__ t1_idx,
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

    clear_state<kWave>(h, k, nch, lane);

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
    uint32_t aidx[kWaveAtomSlots];
    float aval[kWaveAtomSlots];
    if constexpr (kRegAtoms) {
#pragma unroll
      for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
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
      uint32_t idx = (mono && mval < 0.0f) ? midx : dense_argmin<kWave>(h, nch, lane);
      if (idx >= k) {  // only when no entry compares below +inf (NaN state)
        flags |= kFlagNonfinite;
        idx = 0;
      }
      if (trace != nullptr && lane == 0) trace[(size_t)cell * T + t] = idx;

      // -- atoms: scale every weight, add gamma at idx or append idx
      bool hit = false;
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
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
            for (uint32_t jj = 0; jj < kWaveAtomSlots; ++jj)
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
        clear_state<kWave>(h, k, nch, lane);
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
      for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
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


template <uint32_t G, bool kHInLds, bool kRegAtoms>
__global__ void __launch_bounds__(kABlockMaxThreads)
    fw_a_group_kernel(const uint32_t *__restrict__ t1_ptr, const uint32_t *__restrict__ t1_idx,
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
  constexpr uint32_t CPW = kWave / G;           // cells per wave
  constexpr uint32_t AS = kRegAtomMax / G;      // register atom slots per lane
  extern __shared__ uint32_t lds[];
  const uint32_t lane = lane_id();
  const uint32_t grp = lane / G, gl = lane % G;
  const uint64_t gmask = group_mask<G>(grp);
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

  const uint32_t cap4 = (cap + 3u) & ~3u;
  uint32_t *wl = lds + sched_words + (size_t)wib * lds_words_per_wave;
  float *h = kHInLds ? reinterpret_cast<float *>(wl) + (size_t)grp * kscan
                     : state_ws + ((size_t)gwave * CPW + grp) * kscan;
  uint32_t *s_aidx = (kHInLds ? wl + (size_t)CPW * kscan : wl) + (size_t)grp * 2 * cap4;
  float *s_aval = reinterpret_cast<float *>(s_aidx + cap4);
  const uint32_t nch = kscan / (4 * G);
  const uint32_t dummy = k;  // first padding column: holds +inf
  const float inf = __builtin_inff();

  // h += alpha * (row r of t1), r per group; columns of one row are unique,
  // so no two lanes of a group touch the same column. Returns (per lane)
  // whether the group added a negative product.
  auto scatter_row = [&](bool on, uint32_t r, float alpha) -> bool {
    uint32_t p0 = 0, p1 = 0;
    group_load_pair<G>(t1_ptr, on ? r : 0u, grp, p0, p1);
    if (!on) p0 = p1 = 0;
    {
      if (p1 > t1_nnz || p0 > p1) {
        flags |= kFlagBadIndex;
        p0 = p1 = 0;
      }
    }
    bool lane_neg = false;
    for (uint32_t i = 0;; ++i) {
      const uint32_t p = p0 + i * G + gl;
      const bool valid = p < p1;
      if (__ballot(valid) == 0) break;
      uint32_t c = dummy;
      float v = 0.0f;
      if (valid) {
        c = t1_idx[p];
        v = t1_val[p];
        if (c >= k) {
          flags |= kFlagBadIndex;
          c = dummy;
          v = 0.0f;
        }
      }
      h[c] = h[c] + alpha * v;
      lane_neg |= (v < 0.0f);
    }
    return (__ballot(lane_neg) & gmask) != 0;
  };

  for (uint32_t base = gwave * CPW; base < n; base += nwaves * CPW) {
    // idle groups of the last round shadow the last cell and write nothing
    const bool active = base + grp < n;
    const uint32_t cell = active ? base + grp : n - 1;

    // -- t2 = this cell's K2B row: the first kT2Regs * G entries in registers
    uint32_t q0, q1;
    group_load_pair<G>(k2b_ptr, cell, grp, q0, q1);
    if (q1 > k2b_nnz || q0 > q1) {
      flags |= kFlagBadIndex;
      q0 = q1 = 0;
    }
    uint32_t t2c[kT2Regs];
    float t2v[kT2Regs];
    uint32_t nchk = 0;  // register chunks in use by some group of the wave
#pragma unroll
    for (uint32_t r = 0; r < kT2Regs; ++r) {
      t2c[r] = dummy;
      t2v[r] = 0.0f;
      const uint32_t q = q0 + r * G + gl;
      const bool valid = q < q1;
      if (__ballot(q0 + r * G < q1) != 0) nchk = r + 1;
      if (valid) {
        const uint32_t c = k2b_idx[q];
        if (c < k)
          t2c[r] = c, t2v[r] = k2b_val[q];
        else
          flags |= kFlagBadIndex;
      }
    }
    const uint32_t q_extra = q0 + kT2Regs * G;  // entries past the registers

    clear_state<G>(h, k, nch, gl);

    // -- seed the atoms from A_prev's column
    uint32_t s0, s1;
    group_load_pair<G>(ap_ptr, cell, grp, s0, s1);
    if (s1 > ap_nnz || s0 > s1) {
      flags |= kFlagBadIndex;
      s0 = s1 = 0;
    }
    uint32_t cnt = s1 - s0;
    if (cnt > cap) {
      flags |= kFlagCapOverflow;
      cnt = cap;
    }
    uint32_t aidx[AS];
    float aval[AS];
    if constexpr (kRegAtoms) {
#pragma unroll
      for (uint32_t j = 0; j < AS; ++j) {
        const uint32_t s = j * G + gl;
        aidx[j] = s < cnt ? ap_idx[s0 + s] : kNone;
        aval[j] = s < cnt ? ap_val[s0 + s] : 0.0f;
      }
    } else {
      for (uint32_t s = gl; s < cnt; s += G) {
        s_aidx[s] = ap_idx[s0 + s];
        s_aval[s] = ap_val[s0 + s];
      }
    }
    wave_lds_sync();

    // -- h = t1 . a_prev : one t1 row per seed, scaled by its weight
    bool mono = dense_only == 0;
    for (uint32_t i = 0;; ++i) {
      const bool has = s0 + i < s1;
      if (__ballot(has) == 0) break;
      uint32_t m = group_load<G>(ap_idx, has ? s0 + i : 0u, grp);
      float am = group_load<G>(ap_val, has ? s0 + i : 0u, grp);
      if (!has) m = dummy, am = 0.0f;
      if (has && m >= k) flags |= kFlagBadIndex;
      const bool ok = has && m < k;
      if (ok && am < 0.0f) mono = false;
      // groups without a seed here add nothing
      if (scatter_row(ok, ok ? m : 0u, am)) mono = false;
      wave_lds_sync();
    }

    // -- h -= alpha * t2, and the minimum of h over supp(t2) per group
    float mval;
    uint32_t midx;
    auto t2_pass = [&](float alpha) {
      float bv = inf;
      uint32_t bi = kNone;
#pragma unroll
      for (uint32_t r = 0; r < kT2Regs; ++r) {
        if (r < nchk) {
          const uint32_t c = t2c[r];
          const float hn = h[c] - alpha * t2v[r];
          h[c] = hn;
          if (hn < bv) bv = hn, bi = c;
        }
      }
      for (uint32_t qb = q_extra;; qb += G) {  // rows longer than kT2Regs * G
        const uint32_t q = qb + gl;
        const bool valid = q < q1;
        if (__ballot(valid) == 0) break;
        if (valid) {
          const uint32_t c = k2b_idx[q];
          if (c < k) {
            const float hn = h[c] - alpha * k2b_val[q];
            h[c] = hn;
            if (hn < bv) bv = hn, bi = c;
          }
        }
      }
      // group minimum of the value key, then the lowest column holding it
      const uint32_t key = f32_order(bv);
      const uint32_t best = group_min_u32<G>(key);
      mval = f32_unorder(best);
      midx = group_min_u32<G>(key == best ? bi : kNone);
    };
    t2_pass(1.0f);
    wave_lds_sync();

    float s_run = 1.0f;
    for (uint32_t t = 0; t < T; ++t) {
      const StepSched sc = sched_words != 0 ? sched[t] : sched_step(gamma, t, s_run, flags);

      // -- argmin_c h[c] per group, lowest column on a tie
      const bool sparse_ok = mono && mval < 0.0f;
      uint32_t idx = midx;
      if (__ballot(!sparse_ok) != 0) {
        const uint32_t d = dense_argmin<G>(h, nch, gl);
        if (!sparse_ok) idx = d;
      }
      if (idx >= k) {  // only when no entry compares below +inf (NaN state)
        flags |= kFlagNonfinite;
        idx = 0;
      }
      if (trace != nullptr && gl == 0 && active) trace[(size_t)cell * T + t] = idx;

      // -- atoms: scale every weight, add gamma at idx or append idx
      bool hit = false;
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < AS; ++j) {
          if (j * G < cap) {
            float v = aval[j] * sc.keep;
            if (aidx[j] == idx) v += sc.gam, hit = true;
            aval[j] = v;
          }
        }
      } else {
        for (uint32_t s = gl; s < cnt; s += G) {
          float v = s_aval[s] * sc.keep;
          if (s_aidx[s] == idx) v += sc.gam, hit = true;
          s_aval[s] = v;
        }
      }
      if ((__ballot(hit) & gmask) == 0) {
        if (cnt < cap) {
          if constexpr (kRegAtoms) {
            const uint32_t j = cnt / G, l = cnt % G;
#pragma unroll
            for (uint32_t jj = 0; jj < AS; ++jj)
              if (jj == j && gl == l) aidx[jj] = idx, aval[jj] = sc.gam;
          } else if (gl == 0) {
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
        clear_state<G>(h, k, nch, gl);
        mono = dense_only == 0;
      } else if (sc.fold > 0.0f) {
        for (uint32_t i = 0; i < nch; ++i) {
          float4 *q = reinterpret_cast<float4 *>(h + i * 4 * G + gl * 4);
          float4 v = *q;
          v.x *= sc.fold, v.y *= sc.fold, v.z *= sc.fold, v.w *= sc.fold;
          *q = v;
        }
        mono = false;
      }
      wave_lds_sync();
      // -- h += alpha * t1[idx, :]
      if (scatter_row(true, idx, sc.alpha)) mono = false;
      wave_lds_sync();
      // -- h -= alpha * t2
      t2_pass(sc.alpha);
      wave_lds_sync();
    }

    // -- write the atoms
    if (active) {
      const size_t obase = (size_t)cell * cap;
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < AS; ++j) {
          const uint32_t s = j * G + gl;
          if (s < cnt) {
            atom_idx[obase + s] = aidx[j];
            atom_val[obase + s] = aval[j];
          }
        }
      } else {
        for (uint32_t s = gl; s < cnt; s += G) {
          atom_idx[obase + s] = s_aidx[s];
          atom_val[obase + s] = s_aval[s];
        }
      }
      if (gl == 0) atom_cnt[cell] = cnt;
    }
    wave_lds_sync();
  }
  // some flags are raised by single lanes: every lane that saw one reports it
  if (flags != 0) atomicOr(status, flags);
}

template <uint32_t G, bool kHInLds, bool kRegAtoms>
hipError_t launch_variant(const APlan &plan, const DeviceInfo &dev, Csr t1, Csr k2b, Csr ap,
                          uint32_t n, uint32_t k, uint32_t T, uint32_t cap, const float *gamma,
                          uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                          uint32_t *trace, void *ws, uint32_t dense_only, uint32_t *status,
                          hipStream_t stream) {
  static bool configured = false;
  auto kern = [] {
    if constexpr (G == kWave)
      return &fw_a_wave_kernel<kHInLds, kRegAtoms>;
    else
      return &fw_a_group_kernel<G, kHInLds, kRegAtoms>;
  }();
  auto fn = reinterpret_cast<const void *>(kern);
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
  const uint32_t cpw = kWave / G;
  if (kHInLds) {
    int bpc = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, fn, threads, lds_bytes);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    const uint64_t want = ((uint64_t)n + (uint64_t)wpb * cpw - 1) / ((uint64_t)wpb * cpw);
    const uint64_t cap_blocks = (uint64_t)dev.cus * (uint64_t)bpc;
    blocks = (uint32_t)(want < cap_blocks ? want : cap_blocks);
  } else {
    blocks = plan.global_waves / wpb;  // each wave owns workspace slices
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads),
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

// Lanes per cell: from the environment for experiments, else by k.
uint32_t group_width(uint32_t k) {
  const char *v = getenv("SEACELLS_A_GROUP");
  if (v != nullptr) {
    const int g = atoi(v);
    if (g == 16 || g == 32 || g == 64) return (uint32_t)g;
  }
  // small k: several cells per wave amortise the per-step fixed cost; large
  // k: one cell per wave keeps the dense fallback scan short
  if (k <= 512) return 16;
  if (k <= 1024) return 32;
  return 64;
}

}  // namespace

APlan plan_a(uint32_t n, uint32_t k, uint32_t T, uint32_t cap) {
  APlan p{};
  p.group = group_width(k);
  const uint32_t cpw = kWave / p.group;
  p.kpad = (uint32_t)align_up((size_t)k + 1, 4 * p.group);  // >= 1 padding column
  p.reg_atoms = cap <= kRegAtomMax;
  const size_t atom_words = p.reg_atoms ? 0 : (size_t)cpw * 2 * align_up(cap, 4);
  p.sched_words = T <= kSchedMax ? (uint32_t)(T * (sizeof(StepSched) / 4) + 4) : 0u;
  const size_t budget = kLdsBytesPerCU - (size_t)p.sched_words * 4;
  const size_t lds_words = align_up((size_t)cpw * p.kpad + atom_words, 4);
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
    const uint32_t cells = n < 8192u ? n : 8192u;
    const uint32_t gw = (cells + cpw - 1) / cpw;
    p.global_waves = (gw + p.waves_per_block - 1) / p.waves_per_block * p.waves_per_block;
    p.ws_words_per_wave = cpw * p.kpad;
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
#define SEACELLS_A_GROUP(GW)                                                                \
  if (plan.group == GW) {                                                                   \
    if (plan.h_in_lds)                                                                      \
      return plan.reg_atoms ? launch_variant<GW, true, true>(SEACELLS_A_ARGS)               \
                            : launch_variant<GW, true, false>(SEACELLS_A_ARGS);             \
    return plan.reg_atoms ? launch_variant<GW, false, true>(SEACELLS_A_ARGS)                \
                          : launch_variant<GW, false, false>(SEACELLS_A_ARGS);              \
  }
  SEACELLS_A_GROUP(16)
  SEACELLS_A_GROUP(32)
  SEACELLS_A_GROUP(64)
#undef SEACELLS_A_GROUP
#undef SEACELLS_A_ARGS
  return hipErrorInvalidValue;
}

}  // namespace seacells
