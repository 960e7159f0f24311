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
#include "common.hpp"

namespace seacells {
namespace {

constexpr uint32_t kABlockMaxThreads = 256;
constexpr uint32_t kSchedMax = 256;   // steps whose schedule is tabulated in LDS
constexpr uint32_t kT2Regs = 4;       // chunks of G t2 entries held in registers
constexpr uint32_t kRegAtomMax = 128; // atoms per cell held in registers
constexpr uint32_t kNone = 0xffffffffu;
constexpr uint32_t kZeroKey = 0x80000000u;  // f32_order of -0 and +0
constexpr uint32_t kInfKey = 0xff800000u;   // f32_order of +inf
constexpr uint32_t kSupportMinK = 2048;     // support state from this k on
constexpr uint32_t kSupWavesPerBlock = 4;
constexpr uint32_t kSupDefaultWaves = 24;   // resident waves per CU the LDS is sized for
constexpr uint32_t kSupWideWaves = 16;      // the same with 512 t2 entries in registers
constexpr uint32_t kSupLongWaves = 8;       // the same for the pass over long K2B rows
constexpr uint32_t kSupMinHc = 256;         // smallest useful t2 capacity
constexpr uint32_t kSupMaxHc = 8192;
constexpr float kRenormFloor = 1e-15f;      // the page's A_RENORM_FLOOR

// base[byte_off / sizeof(T)] with a 32-bit byte offset from a wave-uniform
// base: one offset register serves loads from several arrays (valid while
// the array holds fewer than 2^30 four-byte entries).
template <typename T>
__device__ __forceinline__ T load_at(const T *__restrict__ base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

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

// The step schedule of a block, written by one thread: T entries, then in
// the last two of the sched_words words the scale s after the last step
// (g = s h for the returned column) and the OR of the flags.
__device__ void build_schedule(uint32_t *lds, uint32_t sched_words, const float *gamma,
                               uint32_t T) {
  StepSched *w = reinterpret_cast<StepSched *>(lds);
  float s = 1.0f;
  uint32_t f = 0;
  for (uint32_t t = 0; t < T; ++t) w[t] = sched_step(gamma, t, s, f);
  lds[sched_words - 2] = __float_as_uint(s);
  lds[sched_words - 1] = f;
}

// Sum over each group of G consecutive lanes (every lane of a group gets it).
template <uint32_t G>
__device__ __forceinline__ float group_sum_f32(float x) {
  for (int off = G / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Minimum of a u32 over each group of G consecutive lanes; every lane of a
// group receives its group's minimum (G = 64: wave_min_u32, uniform). The
// in-row steps are wave_min_u32's, stopped at the group width; a 32-lane
// group ends with a permlane16 swap, which gives both its rows the result.
template <uint32_t G>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t x) {
  if constexpr (G == 64) return wave_min_u32(x);
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
  // a lane with no value below +inf (padding, or a NaN state) offers none:
  // a group with no such value returns kNone (>= k)
  if (key == best && bv < __builtin_inff()) {
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

// kPrune: after every step, drop the atoms at or below the threshold and
// renormalise (the page's pruning variant); the scale s is then per cell.
template <bool kHInLds, bool kRegAtoms, bool kPrune>
__global__ void __launch_bounds__(kABlockMaxThreads)
    fw_a_wave_kernel(const uint32_t *__restrict__ pt_ptr, const uint2 *__restrict__ pt_ent,
                        const uint32_t *__restrict__ k2b_ptr, const uint32_t *__restrict__ k2b_idx,
                        const float *__restrict__ k2b_val, uint32_t k2b_nnz,
                        const uint32_t *__restrict__ ap_ptr, const uint32_t *__restrict__ ap_idx,
                        const float *__restrict__ ap_val, uint32_t ap_nnz, uint32_t n,
                        uint32_t k, uint32_t kscan, uint32_t T, uint32_t cap,
                        const float *__restrict__ gamma, uint32_t *__restrict__ atom_idx,
                        float *__restrict__ atom_val, uint32_t *__restrict__ atom_cnt,
                        uint32_t *__restrict__ trace, float *__restrict__ fw_gap,
                        float *__restrict__ state_ws,
                        uint32_t sched_words, uint32_t lds_words_per_wave, uint32_t dense_only,
                        const uint32_t *__restrict__ cell_list,
                        const uint32_t *__restrict__ cell_count, float prune_thr,
                        uint32_t *__restrict__ status) {
  extern __shared__ uint32_t lds[];
  const uint32_t lane = lane_id();
  const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t wpb = blockDim.x / kWave;
  const uint32_t gwave = blockIdx.x * wpb + wib;
  const uint32_t nwaves = gridDim.x * wpb;
  uint32_t flags = 0;
  // cells: 0 .. n-1, or the first *cell_count entries of cell_list
  uint32_t ncells = n;
  if (cell_list != nullptr) {
    const uint32_t c = *cell_count;
    ncells = c < n ? c : n;
  }

  // -- the step schedule, once per block
  const StepSched *sched = reinterpret_cast<const StepSched *>(lds);
  if (sched_words != 0) {
    if (threadIdx.x == 0) build_schedule(lds, sched_words, gamma, T);
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

  // h += alpha * (row r of t1), from the padded copy: whole chunks of 64
  // (column byte offset, value) pairs, padding entries pointing at the +inf
  // column with value 0. Columns of one row are unique, so no two lanes
  // touch the same column; two chunks are in flight together (their reads
  // before their writes: distinct columns, or the +inf column, which stays
  // +inf). Returns whether the row holds a negative value.
  char *hb = reinterpret_cast<char *>(h);
  auto scatter_row = [&](uint32_t r, float alpha) -> bool {
    const uint32_t e0 = pt_ptr[r], e1 = pt_ptr[r + 1];
    const uint32_t c0 = e0 >> 1, c1 = e1 >> 1;
    uint32_t ch = c0;
    for (; ch + 1 < c1; ch += 2) {
      const uint2 ea = load_at(pt_ent + (size_t)ch * kWave, lane * 8u);
      const uint2 eb = load_at(pt_ent + (size_t)(ch + 1) * kWave, lane * 8u);
      float *pa = reinterpret_cast<float *>(hb + ea.x);
      float *pb = reinterpret_cast<float *>(hb + eb.x);
      const float ha = *pa, hv = *pb;
      *pa = __builtin_fmaf(alpha, __uint_as_float(ea.y), ha);
      *pb = __builtin_fmaf(alpha, __uint_as_float(eb.y), hv);
    }
    if (ch < c1) {
      const uint2 e = load_at(pt_ent + (size_t)ch * kWave, lane * 8u);
      float *hp = reinterpret_cast<float *>(hb + e.x);
      *hp = __builtin_fmaf(alpha, __uint_as_float(e.y), *hp);
    }
    return (e0 & 1u) != 0u;
  };

  for (uint32_t slot = gwave; slot < ncells; slot += nwaves) {
    const uint32_t cell = cell_list != nullptr ? cell_list[slot] : slot;
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
    bool mneg = false;  // that minimum is negative (then midx holds its column)
    uint32_t midx = kNone;
    auto t2_pass = [&](float alpha) {
      float bv = inf;
      uint32_t bi = kNone, br = 0;
      auto reg_chunk = [&](uint32_t r) {
        const uint32_t c = t2c[r];
        const float hn = __builtin_fmaf(-alpha, t2v[r], h[c]);
        h[c] = hn;
        if (hn < bv) bv = hn, bi = c, br = r;
      };
      // the register chunks, nested so that a short row tests its length once
      static_assert(kT2Regs == 4, "the nesting below holds four register chunks");
      uint32_t nr = nchk;
      if (nchk > 0) {
        reg_chunk(0);
        if (nchk > 1) {
          reg_chunk(1);
          if (nchk > 2) {
            reg_chunk(2);
            if (nchk > 3) {
              reg_chunk(3);
              for (uint32_t qb = q_extra; qb < q1; qb += kWave, ++nr) {  // rows longer than 256
                const uint32_t q = qb + lane;
                if (q < q1) {
                  const uint32_t c = k2b_idx[q];
                  if (c < k) {
                    const float hn = __builtin_fmaf(-alpha, k2b_val[q], h[c]);
                    h[c] = hn;
                    if (hn < bv) bv = hn, bi = c, br = nr;
                  }
                }
              }
            }
          }
        }
      }
      // minimum over the wave, then the lowest column holding it: entries
      // are ascending in (chunk, lane) order, so the first chunk with a
      // matching lane and, in it, the lowest matching lane win. Only a
      // negative minimum is used (the dense scan decides otherwise), so the
      // key is ~bits: ordered like the values among negative numbers, and
      // above every negative number for the others (-0 and +inf included).
      // bv is never NaN (a NaN never compares below it), so the minimum is
      // negative exactly when the smallest key lies below that of -0.
      const uint32_t key = ~__float_as_uint(bv);
      const uint32_t best = wave_min_u32(key);
      mneg = best < 0x7fffffffu;
      uint64_t m = __ballot(key == best);  // never empty: every lane takes part
      if (nr > 1) {
        for (uint32_t r = 0; r < nr; ++r) {
          const uint64_t mr = m & __ballot(br == r);
          if (mr != 0) {
            m = mr;
            break;
          }
        }
      }
      midx = readlane_u32(bi, (uint32_t)__builtin_ctzll(m | (1ull << 63)));
    };
    t2_pass(1.0f);
    wave_lds_sync();

    float s_run = 1.0f;
    float s_cell = 1.0f;  // this cell's scale (pruning only)
    for (uint32_t t = 0; t < T; ++t) {
      const StepSched sc = sched_words != 0 ? sched[t] : sched_step(gamma, t, s_run, flags);

      // -- argmin_c h[c], lowest column on a tie
      uint32_t idx = (mono && mneg) ? midx : dense_argmin<kWave>(h, nch, lane);
      if (idx >= k) {  // only when no entry compares below +inf (NaN state)
        flags |= kFlagNonfinite;
        idx = 0;
      }
      if (trace != nullptr && lane == 0) trace[(size_t)cell * T + t] = idx;

      // -- atoms: scale every weight, add gamma at idx or append idx
      uint64_t hits = 0;  // lanes whose slot holds idx
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
          if (j * kWave < cap) {  // (a wave-uniform test: one slot per lane when cap <= 64)
            const bool at = aidx[j] == idx;
            aval[j] = at ? __builtin_fmaf(aval[j], sc.keep, sc.gam) : aval[j] * sc.keep;
            hits |= __ballot(at);
          }
        }
      } else {
        bool hit = false;
        for (uint32_t s = lane; s < cnt; s += kWave) {
          const bool at = s_aidx[s] == idx;
          s_aval[s] = at ? __builtin_fmaf(s_aval[s], sc.keep, sc.gam) : s_aval[s] * sc.keep;
          hit |= at;
        }
        hits = __ballot(hit);
      }
      if (hits == 0) {
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
      // (with pruning the scale is this cell's own: s_k = s * (1 - gamma))
      float alpha = sc.alpha, fold = sc.fold, s_k = 1.0f;
      if constexpr (kPrune) {
        s_k = sc.keep == 0.0f ? 1.0f : s_cell * sc.keep;
        fold = 0.0f;
        if (sc.keep != 0.0f && s_k < 0x1p-64f) fold = s_k, s_k = 1.0f;
        alpha = sc.gam / s_k;
      }
      if (sc.keep == 0.0f) {
        clear_state<kWave>(h, k, nch, lane);
        mono = dense_only == 0;
      } else if (fold > 0.0f) {
        for (uint32_t i = 0; i < nch; ++i) {
          float4 *q = reinterpret_cast<float4 *>(h + i * 256 + lane * 4);
          float4 v = *q;
          v.x *= fold, v.y *= fold, v.z *= fold, v.w *= fold;
          *q = v;
        }
        mono = false;
      }
      wave_lds_sync();
      // -- h += alpha * t1[idx, :]
      if (scatter_row(idx, alpha)) mono = false;
      wave_lds_sync();
      float beta = alpha;
      if constexpr (kPrune) {
        // -- drop: every non-zero weight with |a| <= threshold goes to 0 (its
        // slot stays), and its t1 row leaves w, slot by slot
        for (uint32_t c0 = 0; c0 < cnt; c0 += kWave) {
          float dv = 0.0f;
          uint32_t dm = 0;
          bool drop = false;
          if constexpr (kRegAtoms) {
#pragma unroll
            for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
              if (j * kWave == c0) {
                const float v = aval[j];
                drop = c0 + lane < cnt && v != 0.0f && !(v > prune_thr || v < -prune_thr);
                if (drop) dv = v, dm = aidx[j], aval[j] = 0.0f;
              }
            }
          } else {
            const uint32_t sl = c0 + lane;
            if (sl < cnt) {
              const float v = s_aval[sl];
              drop = v != 0.0f && !(v > prune_thr || v < -prune_thr);
              if (drop) dv = v, dm = s_aidx[sl], s_aval[sl] = 0.0f;
            }
          }
          for (uint64_t msk = __ballot(drop); msk != 0; msk &= msk - 1) {
            const uint32_t l = (uint32_t)__builtin_ctzll(msk);
            const uint32_t m = readlane_u32(dm, l);
            const float d = readlane_f32(dv, l);
            if (m < k) {
              scatter_row(m, -d / s_k);
              mono = false;  // products leave w: only a dense scan decides
            }
            wave_lds_sync();
          }
        }
        // -- renormalise: a and w by 1 / sum(a) unless the sum is at or below
        // the floor; in g = s h form the factor goes into s, and the t2 term,
        // which it must not scale, gets a correction in the pass below
        float part = 0.0f;
        if constexpr (kRegAtoms) {
#pragma unroll
          for (uint32_t j = 0; j < kWaveAtomSlots; ++j) part += aval[j];
        } else {
          for (uint32_t sl = lane; sl < cnt; sl += kWave) part += s_aval[sl];
        }
        const float total = wave_sum_f32(part);  // the same in every lane
        float r = 1.0f;
        if (total > kRenormFloor) {
          r = 1.0f / total;
          beta = alpha - (1.0f - total) / s_k;
          if constexpr (kRegAtoms) {
#pragma unroll
            for (uint32_t j = 0; j < kWaveAtomSlots; ++j) aval[j] *= r;
          } else {
            for (uint32_t sl = lane; sl < cnt; sl += kWave) s_aval[sl] *= r;
          }
        }
        s_cell = s_k * r;
        wave_lds_sync();
      }
      // -- h -= beta * t2
      t2_pass(beta);
      wave_lds_sync();
    }

    // -- the Frank-Wolfe duality gap of the returned column:
    // <g, a> - min_c g[c] with g = s h (atoms of weight 0 add nothing)
    float gap_out = 0.0f;
    if (fw_gap != nullptr) {
      float s_t;
      if constexpr (kPrune)
        s_t = s_cell;
      else
        s_t = sched_words != 0 ? __uint_as_float(lds[sched_words - 2]) : s_run;
      const uint32_t gi = (mono && mneg) ? midx : dense_argmin<kWave>(h, nch, lane);
      float part = 0.0f;
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
          const uint32_t m = aidx[j];
          if (j * kWave + lane < cnt && m < k && aval[j] != 0.0f)
            part = __builtin_fmaf(aval[j], h[m], part);
        }
      } else {
        for (uint32_t sl = lane; sl < cnt; sl += kWave) {
          const uint32_t m = s_aidx[sl];
          const float am = s_aval[sl];
          if (m < k && am != 0.0f) part = __builtin_fmaf(am, h[m], part);
        }
      }
      const float gmin = gi < k ? h[gi] : __builtin_nanf("");
      gap_out = s_t * (wave_sum_f32(part) - gmin);
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
    if (lane == 0) {
      atom_cnt[cell] = cnt;
      if (fw_gap != nullptr) fw_gap[cell] = gap_out;
    }
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
                        uint32_t *__restrict__ trace, float *__restrict__ fw_gap,
                        float *__restrict__ state_ws,
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
    if (threadIdx.x == 0) build_schedule(lds, sched_words, gamma, T);
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
      h[c] = __builtin_fmaf(alpha, v, h[c]);
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
          const float hn = __builtin_fmaf(-alpha, t2v[r], h[c]);
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
            const float hn = __builtin_fmaf(-alpha, k2b_val[q], h[c]);
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
            const bool at = aidx[j] == idx;
            aval[j] = at ? __builtin_fmaf(aval[j], sc.keep, sc.gam) : aval[j] * sc.keep;
            hit |= at;
          }
        }
      } else {
        for (uint32_t s = gl; s < cnt; s += G) {
          const bool at = s_aidx[s] == idx;
          s_aval[s] = at ? __builtin_fmaf(s_aval[s], sc.keep, sc.gam) : s_aval[s] * sc.keep;
          hit |= at;
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

    // -- the Frank-Wolfe duality gap of the returned column (per group)
    float gap_out = 0.0f;
    if (fw_gap != nullptr) {
      const float s_t = sched_words != 0 ? __uint_as_float(lds[sched_words - 2]) : s_run;
      const bool sparse_ok = mono && mval < 0.0f;
      uint32_t gi = midx;
      if (__ballot(!sparse_ok) != 0) {
        const uint32_t d = dense_argmin<G>(h, nch, gl);
        if (!sparse_ok) gi = d;
      }
      float part = 0.0f;
      if constexpr (kRegAtoms) {
#pragma unroll
        for (uint32_t j = 0; j < AS; ++j) {
          const uint32_t m = aidx[j];
          if (j * G + gl < cnt && m < k && aval[j] != 0.0f)
            part = __builtin_fmaf(aval[j], h[m], part);
        }
      } else {
        for (uint32_t sl = gl; sl < cnt; sl += G) {
          const uint32_t m = s_aidx[sl];
          const float am = s_aval[sl];
          if (m < k && am != 0.0f) part = __builtin_fmaf(am, h[m], part);
        }
      }
      const float gmin = gi < k ? h[gi] : __builtin_nanf("");
      gap_out = s_t * (group_sum_f32<G>(part) - gmin);
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
      if (gl == 0) {
        atom_cnt[cell] = cnt;
        if (fw_gap != nullptr) fw_gap[cell] = gap_out;
      }
    }
    wave_lds_sync();
  }
  // some flags are raised by single lanes: every lane that saw one reports it
  if (flags != 0) atomicOr(status, flags);
}

// ---------------------------------------------------------------------------
// Padded copy of t1 for the one-cell-per-wave kernel.
//
// pt_ptr[r] = 2 * (first chunk of row r) | (row r holds a value < 0), with
// pt_ptr[k] = 2 * (all chunks); a row of len entries takes ceil(len / 64)
// chunks of 64 entries (column * 4, value bits). Entries past the row end
// point at column k (the state's +inf padding) with value 0. A malformed
// row (end past nnz or before its start) or column (>= k) raises
// BAD_INDEX; such a row is left empty and such an entry becomes padding.
// If the chunks would exceed the bound the workspace was sized for (only
// possible with malformed row pointers), every row is left empty.

// One block: chunk counts per row and their exclusive prefix sum.
__global__ void __launch_bounds__(1024)
    pad_rows_kernel(const uint32_t *__restrict__ t1_ptr, uint32_t t1_nnz, uint32_t k,
                    uint32_t pad_chunks, uint32_t *__restrict__ pt_ptr,
                    uint32_t *__restrict__ status) {
  __shared__ uint64_t part[1024];
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (k + 1023u) / 1024u;
  const uint32_t r0 = tid * per < k ? tid * per : k;
  const uint32_t r1 = r0 + per < k ? r0 + per : k;
  auto chunks = [&](uint32_t r) -> uint32_t {
    const uint32_t p0 = t1_ptr[r], p1 = t1_ptr[r + 1];
    if (p1 > t1_nnz || p0 > p1) return 0xffffffffu;
    return (p1 - p0 + kWave - 1) / kWave;
  };
  uint64_t sum = 0;
  uint32_t bad = 0;
  for (uint32_t r = r0; r < r1; ++r) {
    const uint32_t c = chunks(r);
    if (c == 0xffffffffu) bad = 1; else sum += c;
  }
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 1024 partial sums (in 64 bits: malformed row
  // pointers can make them large; the total is checked below)
  for (uint32_t off = 1; off < 1024; off <<= 1) {
    const uint64_t v = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const uint64_t total = part[1023];
  __shared__ uint32_t any_bad;
  if (tid == 0) any_bad = 0;
  __syncthreads();
  if (bad) atomicOr(&any_bad, 1u);
  __syncthreads();
  const bool overflow = total > pad_chunks;
  uint64_t at = part[tid] - sum;
  for (uint32_t r = r0; r < r1; ++r) {
    uint32_t c = chunks(r);
    if (c == 0xffffffffu) c = 0;
    pt_ptr[r] = overflow ? 0u : (uint32_t)at << 1;
    at += c;
  }
  if (tid == 1023) pt_ptr[k] = overflow ? 0u : (uint32_t)total << 1;
  if (tid == 0 && (any_bad || overflow)) atomicOr(status, kFlagBadIndex);
}

// One wave per row: the row's entries into its chunks, padding after them;
// a negative value sets the row's low bit.
__global__ void __launch_bounds__(256)
    pad_fill_kernel(const uint32_t *__restrict__ t1_ptr, const uint32_t *__restrict__ t1_idx,
                    const float *__restrict__ t1_val, uint32_t t1_nnz, uint32_t k,
                    uint32_t *__restrict__ pt_ptr, uint2 *__restrict__ pt_ent,
                    uint32_t *__restrict__ status) {
  const uint32_t lane = lane_id();
  const uint32_t nw = gridDim.x * (blockDim.x / kWave);
  uint32_t flags = 0;
  for (uint32_t r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; r < k; r += nw) {
    const uint32_t c0 = pt_ptr[r] >> 1, c1 = pt_ptr[r + 1] >> 1;
    uint32_t p0 = t1_ptr[r], p1 = t1_ptr[r + 1];
    if (p1 > t1_nnz || p0 > p1) p0 = p1 = 0;
    // never more entries than the chunks hold (pointers left empty above)
    const uint32_t len = min(p1 - p0, (c1 - c0) * kWave);
    bool neg = false;
    for (uint32_t i = lane; i < (c1 - c0) * kWave; i += kWave) {
      uint2 e = make_uint2(k * 4u, 0u);
      if (i < len) {
        const uint32_t c = t1_idx[p0 + i];
        const float v = t1_val[p0 + i];
        if (c < k) {
          e = make_uint2(c * 4u, __float_as_uint(v));
          neg |= v < 0.0f;
        } else {
          flags |= kFlagBadIndex;
        }
      }
      pt_ent[(size_t)c0 * kWave + i] = e;
    }
    if (__ballot(neg) != 0 && lane == 0) atomicOr(&pt_ptr[r], 1u);
  }
  if (flags != 0) atomicOr(status, flags);
}

// ---------------------------------------------------------------------------
// Support state for large k (one cell per wave64).
//
// With non-negative data, g outside supp(t2) is a sum of non-negative
// products, so the argmin needs the state only on supp(t2) (the cell's K2B
// row, at most hc_cap entries) plus, for columns outside it, whether any
// non-zero product has landed there since the last restart. Per cell the
// wave keeps in LDS:
//   rec[w]  for each 32-column word w: the supp(t2) bits of the word and the
//           position in the row of its first entry, so a column's position
//           is rec.y + popcount of the bits below it;
//   cov[w]  bits of the columns outside supp(t2) that hold a non-zero
//           product (the padding columns >= k are marked as well);
//   hc[p]   h at the p-th column of supp(t2).
// That is ~12 bytes per 32 columns + 4 per t2 entry instead of 4 per column.
// Every value of hc is produced by the same operations, in the same order,
// as the dense state's value at that column, so the picks are the dense
// kernel's picks:
//   min over supp(t2) < 0   -> that minimum (the dense rule);
//   otherwise the minimum is 0 if any column holds 0: the lowest column
//   outside cov and supp(t2), or of supp(t2) with hc == 0.
// A cell leaves this path (it is queued for the dense kernel, which redoes
// it from the start) on anything the support state cannot represent: a
// negative product, a K2B row longer than hc_cap or not strictly ascending,
// a malformed row or index, a scale fold, a step with no zero and a
// positive minimum, or an invalid step size.
// Work lists of one support pass (device pointers into the workspace).
struct SupQueues {
  const uint32_t *in_list;  // cells to take, or nullptr for 0 .. n-1 (or `order`)
  const uint32_t *in_cnt;   // entries of in_list
  uint32_t *work;           // next entry to take (starts at 0)
  // without in_list: the cells in a locality order, dealt to the XCDs in
  // contiguous segments (xcd_work: one counter per segment), or nullptr
  const uint32_t *order;
  uint32_t *xcd_work;
  uint32_t *long_list;      // cells whose K2B row exceeds hc_cap, or nullptr: to dense_list
  uint32_t *long_cnt;
  uint32_t *dense_list;     // cells for the dense kernel
  uint32_t *dense_cnt;
};


constexpr uint32_t kAXcds = 8;  // MI355X: 8 XCDs, each with its own L2

// Locality order of the cells for the support pass: cells sorted (counting
// sort) by the column of the largest entry of their K2B row (the lowest
// such column on a tie), i.e. the archetype with the most B mass within two
// kernel hops: cells with the same key lie close together and pick
// overlapping atoms. Only the order in which cells are processed changes:
// every cell's outputs are the same whatever the order. One wave per cell.
__global__ void __launch_bounds__(256)
    cell_key_kernel(const uint32_t *__restrict__ k2b_ptr, const uint32_t *__restrict__ k2b_idx,
                    const float *__restrict__ k2b_val, uint32_t k2b_nnz, uint32_t n, uint32_t k,
                    uint32_t *__restrict__ keys, uint32_t *__restrict__ hist) {
  const uint32_t lane = lane_id();
  const uint32_t wpb = blockDim.x / kWave;
  const uint32_t nw = gridDim.x * wpb;
  for (uint32_t c = blockIdx.x * wpb + threadIdx.x / kWave; c < n; c += nw) {
    const uint32_t lo = k2b_ptr[c], hi = k2b_ptr[c + 1];
    uint32_t key = k;  // empty or malformed rows go last
    if (lo < hi && hi <= k2b_nnz) {
      uint32_t bk = 0xffffffffu, bc = 0xffffffffu;  // ~order(value), column
      // four entries per lane in flight
      for (uint32_t p0 = lo + lane; p0 < hi; p0 += 4 * kWave) {
        uint32_t kv[4], col[4];
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j) {
          const uint32_t p = p0 + j * kWave;
          kv[j] = p < hi ? ~f32_order(k2b_val[p]) : 0xffffffffu;  // larger value, smaller key
          col[j] = p < hi ? k2b_idx[p] : 0xffffffffu;
        }
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j)
          if (kv[j] < bk || (kv[j] == bk && col[j] < bc)) bk = kv[j], bc = col[j];
      }
      const uint32_t best = wave_min_u32(bk);
      const uint32_t col = wave_min_u32(bk == best ? bc : 0xffffffffu);
      if (col < k) key = col;
    }
    if (lane == 0) {
      keys[c] = key;
      atomicAdd(hist + key, 1u);
    }
  }
}

// One block: exclusive prefix sum of the k + 1 bucket counts, in place.
__global__ void __launch_bounds__(1024) key_scan_kernel(uint32_t *__restrict__ hist, uint32_t m) {
  __shared__ uint32_t part[1024];
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (m + 1023) / 1024;
  const uint32_t e0 = tid * per < m ? tid * per : m;
  const uint32_t e1 = e0 + per < m ? e0 + per : m;
  uint32_t sum = 0;
  for (uint32_t e = e0; e < e1; ++e) sum += hist[e];
  part[tid] = sum;
  __syncthreads();
  for (uint32_t off = 1; off < 1024; off <<= 1) {
    const uint32_t v = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  uint32_t at = part[tid] - sum;
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t c = hist[e];
    hist[e] = at;
    at += c;
  }
}

// order[pos] = cell, pos taken from the cell's bucket (any order inside it)
__global__ void __launch_bounds__(256)
    cell_scatter_kernel(const uint32_t *__restrict__ keys, uint32_t n,
                        uint32_t *__restrict__ offs, uint32_t *__restrict__ order) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < n; c += stride)
    order[atomicAdd(offs + keys[c], 1u)] = c;
}

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t *__restrict__ p, uint32_t m) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < m; i += stride) p[i] = 0u;
}

constexpr uint32_t kTailPos = 0x80000000u;  // marks a t2 position (not a column) in the pass
constexpr uint32_t kRowBatch = 4;   // chunks of a t1 row whose loads are in flight together
constexpr uint32_t kT2Batch = 4;    // chunks of K2B past the registers re-read together

// a compile-time count passed to a generic lambda
template <uint32_t N>
struct Count {
  static constexpr uint32_t value = N;
};

// TR: chunks of 64 t2 entries held in registers (the rest are re-read).
// kPrune: the pruning variant; a step that drops an atom sends the cell to
// the dense kernel, the renormalisation is done here as the dense kernel does.
template <uint32_t TR, bool kPrune>
__global__ void __launch_bounds__(kABlockMaxThreads)
    fw_a_support_kernel(const uint32_t *__restrict__ pt_ptr, const uint2 *__restrict__ pt_ent,
                        const uint32_t *__restrict__ k2b_ptr, const uint32_t *__restrict__ k2b_idx,
                        const float *__restrict__ k2b_val, uint32_t k2b_nnz,
                        const uint32_t *__restrict__ ap_ptr, const uint32_t *__restrict__ ap_idx,
                        const float *__restrict__ ap_val, uint32_t ap_nnz, uint32_t n,
                        uint32_t k, uint32_t T, uint32_t cap, const float *__restrict__ gamma,
                        uint32_t *__restrict__ atom_idx, float *__restrict__ atom_val,
                        uint32_t *__restrict__ atom_cnt, uint32_t *__restrict__ trace,
                        float *__restrict__ fw_gap, uint32_t nwords, uint32_t hc_cap,
                        uint32_t sched_words,
                        uint32_t lds_words_per_wave, SupQueues q, float prune_thr,
                        uint32_t *__restrict__ status) {
  extern __shared__ uint32_t lds[];
  const uint32_t lane = lane_id();
  const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // -- the step schedule, once per block (the dense kernel reports its flags)
  const StepSched *sched = reinterpret_cast<const StepSched *>(lds);
  if (threadIdx.x == 0) build_schedule(lds, sched_words, gamma, T);
  __syncthreads();
  const bool sched_ok = lds[sched_words - 1] == 0u;
  uint32_t flags = 0;

  uint32_t *wl = lds + sched_words + (size_t)wib * lds_words_per_wave;
  uint2 *rec = reinterpret_cast<uint2 *>(wl);     // nwords + 1 (the last one stays 0)
  uint32_t *cov = wl + 2 * (nwords + 1);           // nwords + 1
  float *hc = reinterpret_cast<float *>(cov + nwords + 1);  // hc_cap + one dummy per lane
  const uint32_t pad_bits = (k & 31u) != 0u ? ~((1u << (k & 31u)) - 1u) : 0u;
  const float inf = __builtin_inff();

  // Each lane owns one dummy slot past the state, which takes the products
  // of entries outside supp(t2) and is never read as a value, and the bitmap
  // ends in one all-zero word (the padding column k lands in it or in the
  // last word's unused bits), so lanes without an entry take the same path
  // as the others and no branch splits a batch.
  float *hdummy = hc + hc_cap + lane;

  // h += alpha * t1[row] on supp(t2), the row being chunks [c0, c1) of the
  // padded copy of t1 (64 entries each, every column checked by the copy;
  // padding entries hold column k and value 0, whose bitmap bit is never
  // set); marks the other columns that receive a non-zero product when
  // `cover`. The row goes in batches of kRowBatch chunks, then one batch of
  // the 1 to 3 chunks left: all loads of a batch are in flight together,
  // then all bitmap lookups, then all state reads, then the writes (the
  // positions of one row are distinct).
  auto scatter_row = [&](uint32_t c0, uint32_t c1, float alpha, bool cover, uint32_t nq) {
    const uint32_t nit = c1 - c0;
    // one batch of NB chunks from chunk i0 on (all of them within the row)
    auto batch = [&](auto nb, uint32_t i0) {
      constexpr uint32_t NB = decltype(nb)::value;
      uint32_t cc[NB];
      float vv[NB];
#pragma unroll
      for (uint32_t b = 0; b < NB; ++b) {
        const uint2 e = load_at(pt_ent, ((c0 + i0 + b) * kWave + lane) * 8u);
        cc[b] = e.x >> 2;
        vv[b] = __uint_as_float(e.y);
      }
      uint2 rw[NB];
#pragma unroll
      for (uint32_t b = 0; b < NB; ++b) rw[b] = rec[cc[b] >> 5];
      float *hp[NB];
      float hv[NB];
      bool in_t2[NB];
#pragma unroll
      for (uint32_t b = 0; b < NB; ++b) {
        const uint32_t bit = 1u << (cc[b] & 31u);
        const uint32_t pos = rw[b].y + __popc(rw[b].x & (bit - 1u));
        in_t2[b] = (rw[b].x & bit) != 0u;  // (then pos < nq: the bits are supp(t2)'s)
        hp[b] = in_t2[b] ? hc + pos : hdummy;
        hv[b] = *hp[b];
      }
#pragma unroll
      for (uint32_t b = 0; b < NB; ++b) *hp[b] = __builtin_fmaf(alpha, vv[b], hv[b]);
      if (cover) {
#pragma unroll
        for (uint32_t b = 0; b < NB; ++b)
          if (!in_t2[b] && alpha * vv[b] != 0.0f) atomicOr(&cov[cc[b] >> 5], 1u << (cc[b] & 31u));
      }
    };
    // full batches, then one batch of exactly the chunks left
    uint32_t i0 = 0;
    for (; i0 + kRowBatch <= nit; i0 += kRowBatch) batch(Count<kRowBatch>{}, i0);
    const uint32_t rest = nit - i0;
    static_assert(kRowBatch == 4, "the tail below covers 1 to 3 chunks");
    if (rest == 3)
      batch(Count<3>{}, i0);
    else if (rest == 2)
      batch(Count<2>{}, i0);
    else if (rest == 1)
      batch(Count<1>{}, i0);
  };

  uint32_t ncells = n;
  if (q.in_list != nullptr) {
    const uint32_t c = *q.in_cnt;
    ncells = c < n ? c : n;
  }
  // With a locality order, the XCD this block runs on (blocks are dealt to
  // the XCDs round-robin) takes its own segment of the order first, so the
  // cells in flight on one XCD are neighbours and share the t1 rows of
  // their atoms in that XCD's L2; then it helps with the other segments.
  // (On another placement only the speed changes.)
  const bool by_order = q.in_list == nullptr && q.order != nullptr;
  uint32_t seg = blockIdx.x % kAXcds, segs_left = kAXcds;
  for (;;) {
    // cells are taken one at a time from a counter: no block waits for a
    // slot while others idle, and expensive cells spread by themselves
    uint32_t cell;
    if (by_order) {
      cell = kNone;
      while (segs_left > 0) {
        const uint32_t lo = (uint32_t)(((uint64_t)n * seg) / kAXcds);
        const uint32_t hi = (uint32_t)(((uint64_t)n * (seg + 1)) / kAXcds);
        uint32_t s = 0;
        if (lane == 0) s = atomicAdd(q.xcd_work + seg, 1u);
        s = __builtin_amdgcn_readfirstlane(s);
        if (s < hi - lo) {
          cell = q.order[lo + s];
          break;
        }
        seg = (seg + 1) % kAXcds;
        --segs_left;
      }
      if (cell == kNone) break;
    } else {
      uint32_t slot = 0;
      if (lane == 0) slot = atomicAdd(q.work, 1u);
      slot = __builtin_amdgcn_readfirstlane(slot);
      if (slot >= ncells) break;
      cell = q.in_list != nullptr ? q.in_list[slot] : slot;
    }
    if (cell >= n) {  // a locality order that does not hold cell ids
      flags |= kFlagBadIndex;
      continue;
    }
    wave_lds_sync();
    const uint32_t q0 = k2b_ptr[cell], q1 = k2b_ptr[cell + 1];
    const uint32_t s0 = ap_ptr[cell], s1 = ap_ptr[cell + 1];
    bool deferred = !sched_ok || q1 > k2b_nnz || q0 > q1 || s1 > ap_nnz || s0 > s1 ||
                    s1 - s0 > cap;
    const bool too_long = !deferred && q1 - q0 > hc_cap;
    deferred = deferred || too_long;
    const uint32_t nq = deferred ? 0u : q1 - q0;

    uint32_t t2c[TR];
    float t2v[TR];
    const uint32_t nchq = (nq + kWave - 1) / kWave;
    const uint32_t nchr = nchq < TR ? nchq : TR;
    if (!deferred) {
      // -- clear the words and the state
      for (uint32_t w = lane; w <= nwords; w += kWave) {
        rec[w] = make_uint2(0u, 0u);
        cov[w] = (w == nwords - 1u) ? pad_bits : 0u;
      }
      for (uint32_t p = lane; p < nq; p += kWave) hc[p] = 0.0f;
      *hdummy = 0.0f;
      wave_lds_sync();
      // -- supp(t2) bits and first positions; the first chunks also go to registers
      bool bad = false;
      auto add_entry = [&](uint32_t p, uint32_t &c, float &v) {
        c = kNone;
        v = 0.0f;
        if (p < nq) {
          c = k2b_idx[q0 + p];
          v = k2b_val[q0 + p];
          const uint32_t prev = p > 0u ? k2b_idx[q0 + p - 1u] : kNone;
          if (c >= k || (p > 0u && prev >= c)) {
            bad = true;
          } else {
            atomicOr(&rec[c >> 5].x, 1u << (c & 31u));
            if (p == 0u || (prev >> 5) != (c >> 5)) rec[c >> 5].y = p;
          }
        }
      };
#pragma unroll
      for (uint32_t r = 0; r < TR; ++r) {
        t2c[r] = kNone;
        t2v[r] = 0.0f;
        if (r < nchr) add_entry(r * kWave + lane, t2c[r], t2v[r]);
      }
      for (uint32_t i = nchr; i < nchq; ++i) {
        uint32_t c;
        float v;
        add_entry(i * kWave + lane, c, v);
      }
      deferred = __ballot(bad) != 0;
    }
    wave_lds_sync();

    // -- atoms from A_prev's column, each with the range of its t1 row
    uint32_t cnt = deferred ? 0u : s1 - s0;
    uint32_t aidx[kWaveAtomSlots], arow0[kWaveAtomSlots], arow1[kWaveAtomSlots];
    float aval[kWaveAtomSlots];
    bool bad_seed = false;
#pragma unroll
    for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
      const uint32_t s = j * kWave + lane;
      aidx[j] = kNone;
      aval[j] = 0.0f;
      arow0[j] = arow1[j] = 0u;
      if (s < cnt) {
        const uint32_t m = ap_idx[s0 + s];
        aidx[j] = m;
        aval[j] = ap_val[s0 + s];
        if (m >= k || aval[j] < 0.0f) {
          bad_seed = true;
        } else {
          // the row's chunks in the padded copy (bit 0: it holds a value < 0)
          const uint32_t w0 = pt_ptr[m];
          arow0[j] = w0 >> 1;
          arow1[j] = pt_ptr[m + 1] >> 1;
          if ((w0 & 1u) != 0u) bad_seed = true;
        }
      }
    }
    if (__ballot(bad_seed) != 0) deferred = true;
    // -- h = t1 . a_prev, seed by seed in A_prev order
    for (uint32_t s = 0; s < cnt && !deferred; ++s) {
      const uint32_t j = s / kWave, l = s % kWave;
      uint32_t p0 = 0, p1 = 0;
      float am = 0.0f;
#pragma unroll
      for (uint32_t jj = 0; jj < kWaveAtomSlots; ++jj) {
        if (jj == j) {
          p0 = readlane_u32(arow0[jj], l);
          p1 = readlane_u32(arow1[jj], l);
          am = readlane_f32(aval[jj], l);
        }
      }
      scatter_row(p0, p1, am, true, nq);
      wave_lds_sync();
    }

    // -- h -= alpha * t2, and the minimum of h over supp(t2) (lowest column)
    // the minimum over supp(t2) as its order-preserving key (-0 and +0 share
    // kZeroKey), and its value
    uint32_t mkey = kInfKey;
    float mval = inf;
    uint32_t midx = kNone;
    auto t2_pass = [&](float alpha) {
      float bv = inf;
      uint32_t bi = kNone, br = 0;
      float *tp[TR];
      float tv[TR];
#pragma unroll
      for (uint32_t r = 0; r < TR; ++r) {
        if (r < nchr) {
          const uint32_t p = r * kWave + lane;
          tp[r] = p < nq ? hc + p : hdummy;
          tv[r] = *tp[r];
        }
      }
#pragma unroll
      for (uint32_t r = 0; r < TR; ++r) {
        if (r < nchr) {
          const float hn = __builtin_fmaf(-alpha, t2v[r], tv[r]);
          *tp[r] = hn;
          const float cand = t2c[r] != kNone ? hn : inf;
          if (cand < bv) bv = cand, bi = t2c[r], br = r;
        }
      }
      // entries past the registers: values re-read from K2B (kT2Batch chunks
      // in flight), tracked by position; the column is read for the winner only
      uint32_t nr = nchr;
      for (uint32_t pb = TR * kWave; pb < nq; pb += kT2Batch * kWave, nr += kT2Batch) {
        float tv2[kT2Batch], hv2[kT2Batch];
        float *tp2[kT2Batch];
#pragma unroll
        for (uint32_t b = 0; b < kT2Batch; ++b) {
          const uint32_t p = pb + b * kWave + lane;
          tv2[b] = p < nq ? k2b_val[q0 + p] : 0.0f;
          tp2[b] = p < nq ? hc + p : hdummy;
          hv2[b] = *tp2[b];
        }
#pragma unroll
        for (uint32_t b = 0; b < kT2Batch; ++b) {
          const uint32_t p = pb + b * kWave + lane;
          const float hn = __builtin_fmaf(-alpha, tv2[b], hv2[b]);
          *tp2[b] = hn;
          const float cand = p < nq ? hn : inf;
          if (cand < bv) bv = cand, bi = kTailPos | p, br = nr + b;
        }
      }
      const uint32_t key = f32_order(bv);
      const uint32_t best = wave_min_u32(key);
      mkey = best;
      mval = f32_unorder(best);
      // the lowest column holding the minimum: the lane when only one holds
      // it, else the first chunk with a holder and its lowest lane (a lane
      // keeps the first chunk where it reached its own minimum)
      uint64_t m = __ballot(key == best);  // never empty: every lane takes part
      if (nr > 1 && __builtin_popcountll(m) > 1) {
        for (uint32_t r = 0; r < nr; ++r) {
          const uint64_t mr = m & __ballot(br == r);
          if (mr != 0) {
            m = mr;
            break;
          }
        }
      }
      midx = readlane_u32(bi, (uint32_t)__builtin_ctzll(m | (1ull << 63)));
      if (midx != kNone && (midx & kTailPos) != 0u) midx = k2b_idx[q0 + (midx & ~kTailPos)];
    };
    if (!deferred) t2_pass(1.0f);
    wave_lds_sync();

    uint32_t acov = 0;  // bit j: the row of the atom in slot j is marked in cov
    float s_cell = 1.0f;  // this cell's scale (pruning only)
    for (uint32_t t = 0; t < T && !deferred; ++t) {
      const StepSched sc = sched[t];
      float alpha = sc.alpha, s_k = 1.0f;
      if constexpr (kPrune) {
        s_k = sc.keep == 0.0f ? 1.0f : s_cell * sc.keep;
        if (sc.keep != 0.0f && s_k < 0x1p-64f) {
          deferred = true;
          break;
        }
        alpha = sc.gam / s_k;
      } else if (sc.fold > 0.0f) {
        deferred = true;
        break;
      }
      // -- argmin
      uint32_t idx = midx;
      if (mkey >= kZeroKey) {  // not negative
        uint32_t cand = kNone;
        for (uint32_t w0 = 0; w0 < nwords; w0 += kWave) {
          const uint32_t w = w0 + lane;
          if (w < nwords && cand == kNone) {
            const uint32_t z = ~(rec[w].x | cov[w]);
            if (z != 0u) cand = w * 32u + (uint32_t)__builtin_ctz(z);
          }
        }
        cand = wave_min_u32(cand);
        if (mkey == kZeroKey && midx < cand) cand = midx;
        if (cand == kNone) {  // every column positive: only a dense scan decides
          deferred = true;
          break;
        }
        idx = cand;
      }
      if (trace != nullptr && lane == 0) trace[(size_t)cell * T + t] = idx;

      // -- atoms: scale every weight, add gamma at idx or append idx
      const bool restart = sc.keep == 0.0f;
      if (restart) acov = 0;
      bool hit = false, fresh = false;
      uint32_t hp0 = 0, hp1 = 0;
#pragma unroll
      for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
        if (j > 0 && j * kWave >= cap) break;  // (uniform: one slot per lane when cap <= 64)
        const bool at = aidx[j] == idx;
        aval[j] = at ? __builtin_fmaf(aval[j], sc.keep, sc.gam) : aval[j] * sc.keep;
        if (at) {
          hit = true;
          fresh = ((acov >> j) & 1u) == 0u;
          acov |= 1u << j;
          hp0 = arow0[j];
          hp1 = arow1[j];
        }
      }
      bool cover = __ballot(fresh) != 0;
      const uint64_t hits = __ballot(hit);
      uint32_t p0, p1;
      if (hits != 0) {
        const uint32_t hl = (uint32_t)__builtin_ctzll(hits);
        p0 = readlane_u32(hp0, hl);
        p1 = readlane_u32(hp1, hl);
      } else {
        cover = true;
        const uint32_t w0 = pt_ptr[idx];
        p0 = w0 >> 1;
        p1 = pt_ptr[idx + 1] >> 1;
        if ((w0 & 1u) != 0u) {  // a row with a value < 0: the dense kernel takes the cell
          deferred = true;
          break;
        }
        if (cnt < cap) {
          const uint32_t j = cnt / kWave, l = cnt % kWave;
#pragma unroll
          for (uint32_t jj = 0; jj < kWaveAtomSlots; ++jj)
            if (jj == j && lane == l)
              aidx[jj] = idx, aval[jj] = sc.gam, arow0[jj] = p0, arow1[jj] = p1,
              acov |= 1u << jj;
          ++cnt;
        } else {
          flags |= kFlagCapOverflow;
        }
      }

      // -- state: restart when gamma == 1
      if (restart) {
        for (uint32_t p = lane; p < nq; p += kWave) hc[p] = 0.0f;
        for (uint32_t w = lane; w < nwords; w += kWave)
          cov[w] = (w == nwords - 1u) ? pad_bits : 0u;
      }
      wave_lds_sync();
      // -- h += alpha * t1[idx, :]
      scatter_row(p0, p1, alpha, cover, nq);
      wave_lds_sync();
      float beta = alpha;
      if constexpr (kPrune) {
        // a drop subtracts products from w: the dense kernel takes the cell
        bool drop = false;
#pragma unroll
        for (uint32_t j = 0; j < kWaveAtomSlots; ++j)
          drop |= j * kWave + lane < cnt && aval[j] != 0.0f &&
                  !(aval[j] > prune_thr || aval[j] < -prune_thr);
        if (__ballot(drop) != 0) {
          deferred = true;
          break;
        }
        // renormalise exactly as the dense kernel does
        float part = 0.0f;
#pragma unroll
        for (uint32_t j = 0; j < kWaveAtomSlots; ++j) part += aval[j];
        const float total = wave_sum_f32(part);
        float r = 1.0f;
        if (total > kRenormFloor) {
          r = 1.0f / total;
          beta = alpha - (1.0f - total) / s_k;
#pragma unroll
          for (uint32_t j = 0; j < kWaveAtomSlots; ++j) aval[j] *= r;
        }
        s_cell = s_k * r;
      }
      // -- h -= beta * t2
      t2_pass(beta);
      wave_lds_sync();
    }

    // -- the Frank-Wolfe duality gap of the returned column, as the dense
    // kernel computes it: min g is the minimum over supp(t2) when that is
    // negative, else 0 where some column holds 0; h of an atom is the state
    // on supp(t2), or 0 for a column no product reached. Anything else (no
    // zero column, an atom of non-zero weight on a marked column) sends the
    // cell to the dense kernel.
    float gap_out = 0.0f;
    if (fw_gap != nullptr && !deferred) {
      const float s_t = kPrune ? s_cell : __uint_as_float(lds[sched_words - 2]);
      bool unknown = false;
      if (mkey > kZeroKey) {  // positive
        bool zero = false;
        for (uint32_t w0 = 0; w0 < nwords; w0 += kWave) {
          const uint32_t w = w0 + lane;
          if (w < nwords && ~(rec[w].x | cov[w]) != 0u) zero = true;
        }
        unknown = __ballot(zero) == 0;
      }
      float part = 0.0f;
#pragma unroll
      for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
        const uint32_t m = aidx[j];
        if (j * kWave + lane < cnt && m < k && aval[j] != 0.0f) {
          const uint2 rw = rec[m >> 5];
          const uint32_t bit = 1u << (m & 31u);
          float hv = 0.0f;
          if ((rw.x & bit) != 0u)
            hv = hc[rw.y + __popc(rw.x & (bit - 1u))];
          else if ((cov[m >> 5] & bit) != 0u)
            unknown = true;
          part = __builtin_fmaf(aval[j], hv, part);
        }
      }
      if (__ballot(unknown) != 0)
        deferred = true;
      else
        gap_out = s_t * (wave_sum_f32(part) - (mval < 0.0f ? mval : 0.0f));
    }

    if (deferred) {
      // a pass with a larger capacity, or the dense kernel, redoes this cell
      // from the start (and writes all of it)
      if (lane == 0) {
        if (too_long && q.long_list != nullptr)
          q.long_list[atomicAdd(q.long_cnt, 1u)] = cell;
        else
          q.dense_list[atomicAdd(q.dense_cnt, 1u)] = cell;
      }
      continue;
    }
    // -- write the atoms
    const size_t base = (size_t)cell * cap;
#pragma unroll
    for (uint32_t j = 0; j < kWaveAtomSlots; ++j) {
      const uint32_t s = j * kWave + lane;
      if (s < cnt) {
        atom_idx[base + s] = aidx[j];
        atom_val[base + s] = aval[j];
      }
    }
    if (lane == 0) {
      atom_cnt[cell] = cnt;
      if (fw_gap != nullptr) fw_gap[cell] = gap_out;
    }
  }
  if (flags != 0) atomicOr(status, flags);
}

__global__ void fw_a_ctr_zero_kernel(uint32_t *__restrict__ p, uint32_t count) {
  if (threadIdx.x < count) p[threadIdx.x] = 0u;
}

// Support state: -1 by k, 0 never, 1 for any k (tests and experiments).
int support_mode() { return a_options().support; }

uint32_t support_waves_per_cu() {
  const uint32_t w = a_options().support_waves;
  return (w >= 4 && w <= 32) ? w : kSupDefaultWaves;
}

// LDS of one support wave when `waves` waves per CU are resident: the
// bitmaps, one dummy per lane and the largest state (t2 entries, a multiple
// of 64) that fits. False when not even kSupMinHc entries fit.
bool support_tier_size(const APlan &p, uint32_t waves, uint32_t &hc_out, uint32_t &lpw_out) {
  const size_t sched_b = (size_t)p.sched_words * 4;
  const size_t fixed = ((size_t)p.nwords + 1) * 12 + (size_t)kWave * 4;
  const uint32_t blocks = (waves + kSupWavesPerBlock - 1) / kSupWavesPerBlock;
  const size_t per_block = kLdsBytesPerCU / blocks;
  const size_t per_wave = per_block > sched_b ? (per_block - sched_b) / kSupWavesPerBlock : 0;
  if (per_wave < fixed + 4 * kSupMinHc) return false;
  size_t hc = (per_wave - fixed) / 4;
  hc = hc / 64 * 64;
  if (hc > kSupMaxHc) hc = kSupMaxHc;
  hc_out = (uint32_t)hc;
  lpw_out = (uint32_t)(align_up(((size_t)p.nwords + 1) * 3 + hc + kWave, 4) * 4);
  return true;
}

// Resident waves per CU of the first support pass: the target, lowered
// (in whole blocks) until its LDS fits.
// The first support pass keeps 512 K2B entries per cell in registers (at
// fewer resident waves) when K2B rows are long on average, else 256.
bool first_pass_wide(const Csr &k2b, uint32_t n) {
  const int o = a_options().support_wide;
  if (o >= 0) return o == 1;
  return k2b.nnz > (uint64_t)n * 192u;
}

uint32_t first_pass_waves(const APlan &p, bool wide) {
  uint32_t w = support_waves_per_cu();
  if (wide && w > kSupWideWaves) w = kSupWideWaves;  // register-limited
  uint32_t hc, lpw;
  while (w > kSupWavesPerBlock && !support_tier_size(p, w, hc, lpw)) w -= kSupWavesPerBlock;
  return w;
}

template <uint32_t G, bool kHInLds, bool kRegAtoms>
hipError_t launch_variant(const APlan &plan, const DeviceInfo &dev, Csr t1, Csr k2b, Csr ap,
                          uint32_t n, uint32_t k, uint32_t T, uint32_t cap, const float *gamma,
                          uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt,
                          uint32_t *trace, float *fw_gap, void *ws, uint32_t dense_only,
                          const uint32_t *cell_list, const uint32_t *cell_count,
                          float prune_thr, uint32_t *status, hipStream_t stream) {
  static bool configured[2] = {false, false};
  const bool prune = plan.prune;  // (the plan takes one cell per wave when pruning)
  const void *fn;
  if constexpr (G == kWave)
    fn = prune ? reinterpret_cast<const void *>(&fw_a_wave_kernel<kHInLds, kRegAtoms, true>)
               : reinterpret_cast<const void *>(&fw_a_wave_kernel<kHInLds, kRegAtoms, false>);
  else
    fn = reinterpret_cast<const void *>(&fw_a_group_kernel<G, kHInLds, kRegAtoms>);
  const uint32_t wpb = plan.waves_per_block;
  const uint32_t threads = wpb * kWave;
  const uint32_t lds_bytes = plan.sched_words * 4 + wpb * plan.lds_per_wave;
  hipError_t e;
  if (!configured[prune]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytesPerCU);
    if (e != hipSuccess) return e;
    configured[prune] = true;
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
  char *w8 = static_cast<char *>(ws);
  float *state_ws = reinterpret_cast<float *>(w8 + plan.ws_dense_off);
  if constexpr (G == kWave) {
    auto kern = prune ? &fw_a_wave_kernel<kHInLds, kRegAtoms, true>
                      : &fw_a_wave_kernel<kHInLds, kRegAtoms, false>;
    const uint32_t *pt_ptr = reinterpret_cast<const uint32_t *>(w8 + plan.ws_pt_ptr_off);
    const uint2 *pt_ent = reinterpret_cast<const uint2 *>(w8 + plan.ws_pt_ent_off);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), lds_bytes, stream, pt_ptr, pt_ent,
                       k2b.ptr, k2b.idx, k2b.val, k2b.nnz, ap.ptr, ap.idx,
                       ap.val, ap.nnz, n, k, plan.kpad, T, cap, gamma, atom_idx, atom_val,
                       atom_cnt, trace, fw_gap, state_ws, plan.sched_words,
                       plan.lds_per_wave / 4, dense_only, cell_list, cell_count, prune_thr,
                       status);
  } else {
    auto kern = &fw_a_group_kernel<G, kHInLds, kRegAtoms>;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), lds_bytes, stream, t1.ptr, t1.idx,
                       t1.val, t1.nnz, k2b.ptr, k2b.idx, k2b.val, k2b.nnz, ap.ptr, ap.idx,
                       ap.val, ap.nnz, n, k, plan.kpad, T, cap, gamma, atom_idx, atom_val,
                       atom_cnt, trace, fw_gap, state_ws, plan.sched_words,
                       plan.lds_per_wave / 4, dense_only, status);
  }
  return hipGetLastError();
}

hipError_t launch_support(const APlan &plan, const DeviceInfo &dev, uint32_t tier, Csr t1,
                          Csr k2b, Csr ap, uint32_t n, uint32_t k, uint32_t T, uint32_t cap,
                          const float *gamma, uint32_t *atom_idx, float *atom_val,
                          uint32_t *atom_cnt, uint32_t *trace, float *fw_gap,
                          const SupQueues &q, const uint32_t *pt_ptr, const uint2 *pt_ent,
                          float prune_thr, uint32_t *status, hipStream_t stream) {
  // t2 entries in registers: 256 for short K2B rows, 512 when rows are long
  // on average (the first pass) or by construction (the long-row pass)
  const bool wide = tier > 0 || first_pass_wide(k2b, n);
  const uint32_t waves = tier > 0 ? kSupLongWaves : first_pass_waves(plan, wide);
  uint32_t hc_cap = 0, lpw = 0;
  if (!support_tier_size(plan, waves, hc_cap, lpw)) return hipErrorInvalidValue;
  const bool prune = plan.prune;
  auto kern = wide ? (prune ? &fw_a_support_kernel<8, true> : &fw_a_support_kernel<8, false>)
                   : (prune ? &fw_a_support_kernel<4, true> : &fw_a_support_kernel<4, false>);
  auto fn = reinterpret_cast<const void *>(kern);
  static bool configured[4] = {false, false, false, false};
  const int which = (wide ? 2 : 0) + (prune ? 1 : 0);
  hipError_t e;
  if (!configured[which]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytesPerCU);
    if (e != hipSuccess) return e;
    configured[which] = true;
  }
  const uint32_t wpb = kSupWavesPerBlock;
  const uint32_t threads = wpb * kWave;
  const uint32_t lds_bytes = plan.sched_words * 4 + wpb * lpw;
  int bpc = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, fn, threads, lds_bytes);
  if (e != hipSuccess) return e;
  if (bpc < 1) bpc = 1;
  const uint64_t want = ((uint64_t)n + wpb - 1) / wpb;
  const uint64_t cap_blocks = (uint64_t)dev.cus * (uint64_t)bpc;
  const uint32_t blocks = (uint32_t)(want < cap_blocks ? want : cap_blocks);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), lds_bytes, stream, pt_ptr, pt_ent,
                     k2b.ptr, k2b.idx, k2b.val, k2b.nnz, ap.ptr, ap.idx,
                     ap.val, ap.nnz, n, k, T, cap, gamma, atom_idx, atom_val, atom_cnt, trace,
                     fw_gap, plan.nwords, hc_cap, plan.sched_words, lpw / 4, q, prune_thr,
                     status);
  return hipGetLastError();
}

bool dense_only_requested() { return a_options().dense_argmin; }

// Lanes per cell: an override for tests and experiments, else by k.
uint32_t group_width(uint32_t k) {
  const uint32_t g = a_options().group;
  if (g == 16 || g == 32 || g == 64) return g;
  // small k: several cells per wave amortise the per-step fixed cost; large
  // k: one cell per wave keeps the dense fallback scan short
  if (k <= 512) return 16;
  if (k <= 1024) return 32;
  return 64;
}

}  // namespace

AOptions &a_options() {
  static AOptions opt;
  return opt;
}

APlan plan_a(uint32_t n, uint32_t k, uint32_t T, uint32_t cap, bool prune, uint32_t t1_nnz) {
  APlan p{};
  p.prune = prune;
  p.group = prune ? kWave : group_width(k);  // pruning runs one cell per wave
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
  }
  const size_t dense_ws = p.h_in_lds ? 0 : (size_t)p.global_waves * p.ws_words_per_wave * 4;

  // support state for large k: picks equal to the dense kernel's (cells it
  // cannot settle are queued for the dense kernel). Pass 0 is sized for
  // many resident waves; K2B rows longer than its capacity go to pass 1,
  // which holds the longest rows with fewer waves.
  p.support = false;
  const int mode = support_mode();
  if (mode != 0 && p.group == kWave && p.reg_atoms && p.sched_words != 0 &&
      !dense_only_requested() && (mode == 1 || k >= kSupportMinK)) {
    p.nwords = (k + 31u) / 32u;
    // the narrow first pass needs the least LDS: if even it does not fit,
    // there is no support state (the sizes of every pass are set at launch)
    uint32_t hc, lpw;
    if (support_tier_size(p, kSupWavesPerBlock, hc, lpw)) p.support = true;
  }
  // workspace: [counters | long-row queue | dense queue | locality order:
  // keys, bucket offsets, order | padded t1 | dense state slices]
  size_t off = 0;
  if (p.support) {
    p.ws_list_off = 256;
    p.ws_list2_off = align_up(p.ws_list_off + (size_t)n * 4, 256);
    p.ws_keys_off = align_up(p.ws_list2_off + (size_t)n * 4, 256);
    p.ws_hist_off = align_up(p.ws_keys_off + (size_t)n * 4, 256);
    p.ws_order_off = align_up(p.ws_hist_off + ((size_t)k + 1) * 4, 256);
    off = p.ws_order_off + (size_t)n * 4;
  } else {
    p.ws_list_off = p.ws_list2_off = p.ws_keys_off = p.ws_hist_off = p.ws_order_off = 0;
  }
  // the one-cell-per-wave kernel reads t1 from a padded copy: a row of len
  // entries takes ceil(len / 64) chunks, at most nnz / 64 + k in all
  p.padded = p.group == kWave;
  if (p.padded) {
    p.pad_chunks = (uint32_t)(((uint64_t)t1_nnz + kWave - 1) / kWave + k);
    p.ws_pt_ptr_off = align_up(off, 256);
    p.ws_pt_ent_off = align_up(p.ws_pt_ptr_off + ((size_t)k + 1) * 4, 256);
    off = p.ws_pt_ent_off + (size_t)p.pad_chunks * kWave * sizeof(uint2);
  }
  p.ws_dense_off = align_up(off, 256);
  p.ws_bytes = dense_ws > 0 || off > 0 ? align_up(p.ws_dense_off + dense_ws, 256) : 0;
  return p;
}

hipError_t launch_fw_a(const APlan &plan, Csr t1, Csr k2b, Csr ap, uint32_t n, uint32_t k,
                       uint32_t T, uint32_t cap, const float *gamma, float prune_thr,
                       uint32_t *atom_idx, float *atom_val, uint32_t *atom_cnt, uint32_t *trace,
                       float *fw_gap, void *ws, uint32_t *status, hipStream_t stream) {
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return e;
  const uint32_t dense_only = dense_only_requested() ? 1u : 0u;
  const uint32_t *cell_list = nullptr, *cell_count = nullptr;
  if (plan.padded) {
    char *w8 = static_cast<char *>(ws);
    uint32_t *pt_ptr = reinterpret_cast<uint32_t *>(w8 + plan.ws_pt_ptr_off);
    uint2 *pt_ent = reinterpret_cast<uint2 *>(w8 + plan.ws_pt_ent_off);
    hipLaunchKernelGGL(pad_rows_kernel, dim3(1), dim3(1024), 0, stream, t1.ptr, t1.nnz, k,
                       plan.pad_chunks, pt_ptr, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const uint32_t rows_per_block = 256 / kWave;
    const uint32_t fill_blocks = (k + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(pad_fill_kernel, dim3(fill_blocks < 65535u ? fill_blocks : 65535u),
                       dim3(256), 0, stream, t1.ptr, t1.idx, t1.val, t1.nnz, k, pt_ptr, pt_ent,
                       status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the support kernel reads t1 from the padded copy, with 32-bit byte offsets
  if (plan.support && plan.padded && plan.pad_chunks < (1u << 23)) {
    char *w8 = static_cast<char *>(ws);
    uint32_t *ctr = reinterpret_cast<uint32_t *>(w8);  // work0, work1, long, dense
    uint32_t *long_list = reinterpret_cast<uint32_t *>(w8 + plan.ws_list_off);
    uint32_t *dense_list = reinterpret_cast<uint32_t *>(w8 + plan.ws_list2_off);
    hipLaunchKernelGGL(fw_a_ctr_zero_kernel, dim3(1), dim3(64), 0, stream, ctr, 16u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the locality order of the cells (counters 8 .. 15: one per XCD segment)
    uint32_t *keys = reinterpret_cast<uint32_t *>(w8 + plan.ws_keys_off);
    uint32_t *hist = reinterpret_cast<uint32_t *>(w8 + plan.ws_hist_off);
    uint32_t *order = reinterpret_cast<uint32_t *>(w8 + plan.ws_order_off);
    const uint32_t nb = (uint32_t)(((uint64_t)n + 255) / 256 < 4096 ? ((uint64_t)n + 255) / 256
                                                                     : 4096);
    const uint32_t hb = (uint32_t)(((uint64_t)k + 256) / 256 < 4096 ? ((uint64_t)k + 256) / 256
                                                                     : 4096);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(hb), dim3(256), 0, stream, hist, k + 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const uint32_t kb = (uint32_t)(((uint64_t)n + 3) / 4 < 16384 ? ((uint64_t)n + 3) / 4 : 16384);
    hipLaunchKernelGGL(cell_key_kernel, dim3(kb), dim3(256), 0, stream, k2b.ptr, k2b.idx, k2b.val,
                       k2b.nnz, n, k, keys, hist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(key_scan_kernel, dim3(1), dim3(1024), 0, stream, hist, k + 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(cell_scatter_kernel, dim3(nb), dim3(256), 0, stream, keys, n, hist, order);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // a second pass when it holds longer K2B rows than the first
    const bool wide0 = first_pass_wide(k2b, n);
    uint32_t hc0 = 0, hc1 = 0, lpw_unused;
    support_tier_size(plan, first_pass_waves(plan, wide0), hc0, lpw_unused);
    const bool two = support_tier_size(plan, kSupLongWaves, hc1, lpw_unused) && hc1 > hc0;
    SupQueues q0{nullptr, nullptr, ctr + 0, order, ctr + 8, two ? long_list : nullptr, ctr + 2,
                 dense_list, ctr + 3};
    const uint32_t *pt_ptr = reinterpret_cast<const uint32_t *>(w8 + plan.ws_pt_ptr_off);
    const uint2 *pt_ent = reinterpret_cast<const uint2 *>(w8 + plan.ws_pt_ent_off);
    e = launch_support(plan, dev, 0, t1, k2b, ap, n, k, T, cap, gamma, atom_idx, atom_val,
                       atom_cnt, trace, fw_gap, q0, pt_ptr, pt_ent, prune_thr, status, stream);
    if (e != hipSuccess) return e;
    if (two) {
      SupQueues q1{long_list, ctr + 2, ctr + 1, nullptr, nullptr, nullptr, nullptr, dense_list,
                   ctr + 3};
      e = launch_support(plan, dev, 1, t1, k2b, ap, n, k, T, cap, gamma, atom_idx, atom_val,
                         atom_cnt, trace, fw_gap, q1, pt_ptr, pt_ent, prune_thr, status, stream);
      if (e != hipSuccess) return e;
    }
    cell_list = dense_list;
    cell_count = ctr + 3;
  }
#define SEACELLS_A_ARGS \
  plan, dev, t1, k2b, ap, n, k, T, cap, gamma, atom_idx, atom_val, atom_cnt, trace, fw_gap, \
      ws, dense_only, cell_list, cell_count, prune_thr, status, stream
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
