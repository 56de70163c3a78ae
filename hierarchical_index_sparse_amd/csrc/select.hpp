// Exact top-`want` selection with ties broken toward the lower index.
//
// The keys live in registers, thread-major: a group of NW waves holds up to
// NW * 64 * R keys and thread x of the group owns the consecutive indices
// [x * R, x * R + R) (key[r] has index x * R + r).  Key 0 marks an empty
// slot; keys come from score_key() of finite scores.  With NW == 1 a single
// wave selects on its own (several waves of one workgroup may then run
// independent selects, each with its own SelectSmem); with NW > 1 the whole
// workgroup takes part.
//
// 1. Threshold T = the want-th largest key:
//    a. (NW * R >= 8) the scores are dropped into 255 linear bins between
//       their minimum and maximum (bin = min(floor((x - min) * 255 / (max -
//       min)), 254), a non-decreasing function of x, so a key in a higher bin
//       is strictly larger than every key in a lower one and equal keys share
//       a bin; empty slots go to bin 255, which is never scanned).  Each
//       key's bin is computed once and kept as one byte in registers.  A
//       suffix scan of the LDS histogram finds the bin holding T and the
//       count of keys above it; that bin's keys are compacted into LDS and
//       one wave finds T by a bitwise binary search over the bits below the
//       candidates' common prefix (largest x with count(key >= x) >= need,
//       one compare + ballot + popcount per key and bit);
//    b. (fewer keys, a target bin too full for the LDS buffer, or a score
//       range that is not finite) the bitwise search runs over all keys.
// 2. Every key > T is kept; of the keys equal to T, the first
//    want - count(> T) in index order are kept.  Per-thread counts and wave
//    prefix scans give every thread its output offset, so emit(pos, index)
//    receives pos = 0 .. want-1 in ascending index order.
#pragma once

#include "common.hpp"

namespace hsa {

constexpr int kBins = 256;
constexpr int kBinCap = 1024;  // keys of the target bin searched by one wave

template <int NW>
struct SelectSmem {
  int red[4 * NW];
  uint32_t kmin[NW], kmax[NW];
  int hist[kBins];
  int info[4];  // target bin, count above it, keys compacted, threshold
  uint32_t cand[kBinCap];
};

// Barrier among the threads taking part in one select.
template <int NW>
__device__ __forceinline__ void sel_sync() {
  if constexpr (NW == 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

template <int NW>
__device__ __forceinline__ int sel_wave() {
  if constexpr (NW == 1) return 0;
  else return threadIdx.x / kWave;
}

// Inverse of score_key for non-empty keys: a set top bit marks a
// non-negative score (flip it back), a clear one a negative score (flip all).
__device__ __forceinline__ float key_to_score(uint32_t k) {
  const uint32_t flip = ~(uint32_t)((int32_t)k >> 31) | 0x80000000u;
  return __uint_as_float(k ^ flip);
}

__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int incl = wave_incl_scan(v);
  total = __builtin_amdgcn_readlane(incl, kWave - 1);
  return incl - v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return group_reduce<kWave>(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return group_reduce<kWave>(v, [](uint32_t a, uint32_t b) { return min(a, b); });
}
__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v) {
  return group_reduce<kWave>(v, [](uint32_t a, uint32_t b) { return a & b; });
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  return group_reduce<kWave>(v, [](uint32_t a, uint32_t b) { return a | b; });
}

template <int NW>
__device__ __forceinline__ int group_sum(int v, int* red, int parity) {
  if constexpr (NW == 1) {
    return v;
  } else {
    const int wave = threadIdx.x / kWave;
    int* buf = red + parity * NW;
    if (lane_id() == 0) buf[wave] = v;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += buf[w];
    return s;
  }
}

// Bitwise search over all keys of the group.
template <int NW, int R>
__device__ __forceinline__ uint32_t full_threshold(const uint32_t (&key)[R], int want, int* red) {
  uint32_t T = 0;
  int parity = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += __popcll(ballot(key[r] >= cand));
    cnt = group_sum<NW>(cnt, red, parity);
    parity ^= 1;
    if (cnt >= want) T = cand;
  }
  return T;
}

// Exact search over the n compacted keys of the target bin (one wave).
// FROM_SCORES: cand holds the fp32 scores' bits, turned into keys here.
template <int R2, bool FROM_SCORES = false>
__device__ __forceinline__ uint32_t bin_threshold(const uint32_t* cand, int n, int need) {
  const int lane = lane_id();
  uint32_t ck[R2];
  uint32_t all_and = 0xFFFFFFFFu, all_or = 0u;
#pragma unroll
  for (int r = 0; r < R2; ++r) {
    const int idx = r * kWave + lane;
    ck[r] = idx < n ? (FROM_SCORES ? score_key(__uint_as_float(cand[idx])) : cand[idx]) : 0u;
    if (idx < n) {
      all_and &= ck[r];
      all_or |= ck[r];
    }
  }
  all_and = wave_and_u32(all_and);
  all_or = wave_or_u32(all_or);
  const uint32_t diff = all_and ^ all_or;
  if (diff == 0u) return all_and;  // every candidate is equal
  const int top = 31 - __builtin_clz(diff);
  uint32_t T = all_and & ~((2u << top) - 1u);  // the common prefix
  // T is one of the candidates, so the bits below the lowest bit set in any
  // candidate are 0 in T too: the search stops there (integer-valued scores
  // leave many low mantissa bits clear)
  const int low = __builtin_ctz(all_or);
  for (int b = top; b >= low; --b) {
    const uint32_t c = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R2; ++r) cnt += __popcll(ballot(ck[r] >= c));
    if (cnt >= need) T = c;
  }
  return T;
}

// The want-th largest key (1 <= want <= number of non-empty keys).
template <int NW, int R>
__device__ __forceinline__ uint32_t find_threshold(const uint32_t (&key)[R], int want, SelectSmem<NW>& sm) {
  // Few keys in a single wave: the bitwise search has no barriers and is
  // cheapest.  Otherwise (many keys, or many waves whose every bitwise pass
  // would need a workgroup barrier) the histogram path is used.
  if constexpr (R < 8 && NW * R < 8) {
    return full_threshold<NW, R>(key, want, sm.red);
  } else {
    const int wave = sel_wave<NW>();
    const int lane = lane_id();
    const int tid = wave * kWave + lane;
    constexpr int NT = NW * kWave;

    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      hi = max(hi, key[r]);
      lo = min(lo, key[r] ? key[r] : 0xFFFFFFFFu);
    }
    hi = wave_max_u32(hi);
    lo = wave_min_u32(lo);
    for (int b = tid; b < kBins; b += NT) sm.hist[b] = 0;
    if (lane == 0) {
      sm.kmin[wave] = lo;
      sm.kmax[wave] = hi;
    }
    if (tid == 0) sm.info[2] = 0;
    sel_sync<NW>();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo = min(lo, sm.kmin[w]);
      hi = max(hi, sm.kmax[w]);
    }
    if (lo == hi) return hi;  // every non-empty key is equal
    const float smin = key_to_score(lo);
    const float range = key_to_score(hi) - smin;
    if (!(range < INFINITY)) {
      sel_sync<NW>();
      return full_threshold<NW, R>(key, want, sm.red);
    }
    const float scale = (float)(kBins - 1) / range;
    // bins of all keys, one byte each (4 per register), computed once; the
    // histogram counts empty slots in the unscanned bin kBins - 1
    constexpr int RP = (R + 3) / 4;
    uint32_t binp[RP];
#pragma unroll
    for (int p = 0; p < RP; ++p) binp[p] = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // max(key, lo) keeps an empty slot's arithmetic finite; its bin is
      // then overridden (kBins - 1 has every bit of the byte set)
      const uint32_t kk = max(key[r], lo);
      int bn = min((int)((key_to_score(kk) - smin) * scale), kBins - 2);
      bn |= (int)(key[r] == 0u) * (kBins - 1);
      binp[r / 4] |= (uint32_t)bn << (8 * (r % 4));
      atomicAdd(&sm.hist[bn], 1);
    }
    auto bin_at = [&](int r) { return (int)((binp[r / 4] >> (8 * (r % 4))) & 0xFFu); };
    sel_sync<NW>();
    if (wave == 0) {
      // suffix sums over bins: lane l holds bins 4l .. 4l+3 (the last is
      // the empty-slot bin, left out)
      const int c0 = sm.hist[4 * lane], c1 = sm.hist[4 * lane + 1], c2 = sm.hist[4 * lane + 2],
                c3 = lane == kWave - 1 ? 0 : sm.hist[4 * lane + 3];
      const int mine = c0 + c1 + c2 + c3;
      const int pre = wave_incl_scan(mine);  // sum over lanes <= l
      int above = __builtin_amdgcn_readlane(pre, kWave - 1) - pre;  // keys in bins of higher lanes
      const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (above < want && want <= above + cs[e]) {
          sm.info[0] = 4 * lane + e;
          sm.info[1] = above;
        }
        above += cs[e];
      }
    }
    sel_sync<NW>();
    const int tb = sm.info[0];
    const int need = want - sm.info[1];
    if (sm.hist[tb] > kBinCap) {
      sel_sync<NW>();
      return full_threshold<NW, R>(key, want, sm.red);
    }
    // compact the target bin's keys (any order)
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += bin_at(r) == tb;
    int wtot;
    int pos = wave_excl_scan(cnt, wtot);
    int base = 0;
    if (lane == 0 && wtot) base = atomicAdd(&sm.info[2], wtot);
    pos += __builtin_amdgcn_readlane(base, 0);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (bin_at(r) == tb) sm.cand[pos++] = key[r];
    sel_sync<NW>();
    if (wave == 0) {
      const int n = sm.hist[tb];
      uint32_t T;
      if (n <= 64) T = bin_threshold<1>(sm.cand, n, need);
      else if (n <= 256) T = bin_threshold<4>(sm.cand, n, need);
      else T = bin_threshold<kBinCap / kWave>(sm.cand, n, need);
      if (lane == 0) sm.info[3] = (int)T;
    }
    sel_sync<NW>();
    return (uint32_t)sm.info[3];
  }
}

// Requires: 1 <= want < number of non-empty keys.  Every thread of the
// group must call it (it synchronises the group).  emit(pos, idx, take, key) is
// called for every key of the thread in index order; `take` says whether
// the key is kept, and then pos (0 .. want-1) is its output slot.  With
// END_SYNC the group synchronises once more after emission (for callers
// that read what emit wrote to LDS, or reuse the LDS); a caller whose
// threads only write global memory after the select passes false.
template <int NW, int R, bool END_SYNC = true, typename Emit>
__device__ __forceinline__ void select_top(const uint32_t (&key)[R], int want, SelectSmem<NW>& sm, Emit&& emit) {
  const int wave = sel_wave<NW>();
  const int lane = lane_id();
  const uint32_t T = find_threshold<NW, R>(key, want, sm);

  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    gt += key[r] > T;
    eq += key[r] == T;
  }
  int gt_w, eq_w;
  (void)wave_excl_scan(gt, gt_w);
  const int eq_ex = wave_excl_scan(eq, eq_w);
  int gt_total = gt_w, eq_before = 0, sel_before = 0;
  if constexpr (NW > 1) {
    int* g = sm.red + 2 * NW;  // the search passes use red[0 .. 2 NW)
    int* e = sm.red + 3 * NW;
    if (lane == 0) {
      g[wave] = gt_w;
      e[wave] = eq_w;
    }
    __syncthreads();
    gt_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) gt_total += g[w];
    const int need_all = want - gt_total;
    for (int w = 0; w < wave; ++w) {
      sel_before += g[w] + min(max(need_all - eq_before, 0), e[w]);
      eq_before += e[w];
    }
  }
  const int need_eq = want - gt_total;
  int ties = min(max(need_eq - (eq_before + eq_ex), 0), eq);  // ties this thread keeps
  int sel_w;
  int pos = sel_before + wave_excl_scan(gt + ties, sel_w);
  const int idx0 = (wave * kWave + lane) * R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int is_eq = key[r] == T;
    const int tk = (int)(key[r] > T) | (is_eq & (int)(ties > 0));
    ties -= is_eq & tk;
    emit(pos, idx0 + r, tk != 0, key[r]);
    pos += tk;
  }
  if constexpr (END_SYNC) sel_sync<NW>();  // LDS may be reused by the caller
}


// ---- the same select over fp32 scores held directly
//
// For callers that hold the scores: the order of score_key() on finite
// scores is the order of the scores themselves (-0 and +0 equal), so the
// scores are compared as floats and no key is formed per element.  Empty
// slots hold a quiet NaN: fminf / fmaxf pass over it and every comparison
// with it is false; it falls into histogram bin 0, whose count starts at
// minus the number of empty slots.  Same result as select_top on the keys.

// Bitwise search over all scores of the group (keys formed on the fly).
template <int NW, int R>
__device__ __forceinline__ uint32_t full_threshold_f(const float (&v)[R], int want, int* red) {
  uint32_t T = 0;
  int parity = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += __popcll(ballot(v[r] == v[r] && score_key(v[r]) >= cand));
    cnt = group_sum<NW>(cnt, red, parity);
    parity ^= 1;
    if (cnt >= want) T = cand;
  }
  return T;
}

// The want-th largest key over the group's scores (1 <= want <= number of
// non-empty slots; n_empty = number of empty slots in the whole group).
template <int NW, int R>
__device__ __forceinline__ bool hist_threshold_f(const float (&v)[R], int want, int n_empty, SelectSmem<NW>& sm,
                                                 uint32_t& T_out) {
  const int wave = sel_wave<NW>();
  const int lane = lane_id();
  const int tid = wave * kWave + lane;
  constexpr int NT = NW * kWave;

  float flo = INFINITY, fhi = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    flo = fminf(flo, v[r]);
    fhi = fmaxf(fhi, v[r]);
  }
  uint32_t lo = wave_min_u32(score_key(flo)), hi = wave_max_u32(score_key(fhi));
  for (int b = tid; b < kBins; b += NT) sm.hist[b] = b == 0 ? -n_empty : 0;
  if (lane == 0) {
    sm.kmin[wave] = lo;
    sm.kmax[wave] = hi;
  }
  if (tid == 0) sm.info[2] = 0;
  sel_sync<NW>();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, sm.kmin[w]);
    hi = max(hi, sm.kmax[w]);
  }
  if (lo == hi) {  // every non-empty score is equal
    T_out = hi;
    return true;
  }
  const float smin = key_to_score(lo);
  const float range = key_to_score(hi) - smin;
  if (!(range < INFINITY)) return false;
  const float scale = (float)(kBins - 1) / range;
  constexpr int RP = (R + 3) / 4;
  uint32_t binp[RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) binp[p] = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // fmaxf sends an empty slot (NaN) to 0, i.e. to bin 0
    const int bn = min((int)fmaxf((v[r] - smin) * scale, 0.f), kBins - 2);
    binp[r / 4] |= (uint32_t)bn << (8 * (r % 4));
    atomicAdd(&sm.hist[bn], 1);
  }
  auto bin_at = [&](int r) { return (int)((binp[r / 4] >> (8 * (r % 4))) & 0xFFu); };
  sel_sync<NW>();
  if (wave == 0) {
    const int c0 = sm.hist[4 * lane], c1 = sm.hist[4 * lane + 1], c2 = sm.hist[4 * lane + 2],
              c3 = lane == kWave - 1 ? 0 : sm.hist[4 * lane + 3];
    const int mine = c0 + c1 + c2 + c3;
    const int pre = wave_incl_scan(mine);
    int above = __builtin_amdgcn_readlane(pre, kWave - 1) - pre;
    const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (above < want && want <= above + cs[e]) {
        sm.info[0] = 4 * lane + e;
        sm.info[1] = above;
      }
      above += cs[e];
    }
  }
  sel_sync<NW>();
  const int tb = sm.info[0];
  const int need = want - sm.info[1];
  if (sm.hist[tb] > kBinCap) return false;
  // compact the target bin's scores (any order); in bin 0 the empty slots
  // are passed over
  const bool bin0 = tb == 0;
  auto in_bin = [&](int r) { return bin_at(r) == tb && (!bin0 || v[r] == v[r]); };
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) cnt += in_bin(r);
  int wtot;
  int pos = wave_excl_scan(cnt, wtot);
  int base = 0;
  if (lane == 0 && wtot) base = atomicAdd(&sm.info[2], wtot);
  pos += __builtin_amdgcn_readlane(base, 0);
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (in_bin(r)) sm.cand[pos++] = __float_as_uint(v[r]);
  sel_sync<NW>();
  if (wave == 0) {
    const int n = sm.hist[tb];
    uint32_t T;
    if (n <= 64) T = bin_threshold<1, true>(sm.cand, n, need);
    else if (n <= 256) T = bin_threshold<4, true>(sm.cand, n, need);
    else T = bin_threshold<kBinCap / kWave, true>(sm.cand, n, need);
    if (lane == 0) sm.info[3] = (int)T;
  }
  sel_sync<NW>();
  T_out = (uint32_t)sm.info[3];
  return true;
}

template <int NW, int R>
__device__ __forceinline__ uint32_t find_threshold_f(const float (&v)[R], int want, int n_empty, SelectSmem<NW>& sm) {
  uint32_t T;
  if (hist_threshold_f<NW, R>(v, want, n_empty, sm, T)) return T;
  sel_sync<NW>();  // (uniform) the histogram's LDS is read no more
  return full_threshold_f<NW, R>(v, want, sm.red);
}

// select_top over fp32 scores (empty slots: quiet NaN, n_empty of them in
// the group).  emit(pos, idx, take) as in select_top.
template <int NW, int R, bool END_SYNC = true, typename Emit>
__device__ __forceinline__ void select_top_f(const float (&v)[R], int want, int n_empty, SelectSmem<NW>& sm,
                                             Emit&& emit) {
  const int wave = sel_wave<NW>();
  const int lane = lane_id();
  const float Tf = key_to_score(find_threshold_f<NW, R>(v, want, n_empty, sm));

  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    gt += v[r] > Tf;
    eq += v[r] == Tf;
  }
  int gt_w, eq_w;
  (void)wave_excl_scan(gt, gt_w);
  const int eq_ex = wave_excl_scan(eq, eq_w);
  int gt_total = gt_w, eq_before = 0, sel_before = 0;
  if constexpr (NW > 1) {
    int* g = sm.red + 2 * NW;
    int* e = sm.red + 3 * NW;
    if (lane == 0) {
      g[wave] = gt_w;
      e[wave] = eq_w;
    }
    __syncthreads();
    gt_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) gt_total += g[w];
    const int need_all = want - gt_total;
    for (int w = 0; w < wave; ++w) {
      sel_before += g[w] + min(max(need_all - eq_before, 0), e[w]);
      eq_before += e[w];
    }
  }
  const int need_eq = want - gt_total;
  int ties = min(max(need_eq - (eq_before + eq_ex), 0), eq);
  int sel_w;
  int pos = sel_before + wave_excl_scan(gt + ties, sel_w);
  const int idx0 = (wave * kWave + lane) * R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int is_eq = v[r] == Tf;
    const int tk = (int)(v[r] > Tf) | (is_eq & (int)(ties > 0));
    ties -= is_eq & tk;
    emit(pos, idx0 + r, tk != 0);
    pos += tk;
  }
  if constexpr (END_SYNC) sel_sync<NW>();
}

}  // namespace hsa
