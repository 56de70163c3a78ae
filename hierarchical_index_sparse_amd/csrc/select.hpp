// Exact top-`want` selection with ties broken toward the lower index.
//
// The keys live in registers.  A workgroup of NW waves holds up to
// NW * 64 * R keys; wave w owns the contiguous index range
// [w * 64 * R, (w + 1) * 64 * R) and key[r] of lane l has index
// w * 64 * R + r * 64 + l.  Key 0 marks an empty slot; keys come from
// score_key() of finite scores.
//
// 1. Threshold T = the want-th largest key, found in two phases:
//    a. the scores are dropped into 256 linear bins between their minimum
//       and maximum (bin = floor((x - min) * 256 / (max - min)), a
//       non-decreasing function of x, so a key in a higher bin is strictly
//       larger than every key in a lower one and equal keys share a bin);
//       a suffix scan of the LDS histogram finds the bin holding T and the
//       count of keys above it;
//    b. that bin's keys are compacted into LDS and one wave finds T exactly
//       by a bitwise binary search (largest x with count(key >= x) >= need;
//       one compare + ballot + popcount per key and bit).
//    When the bin is too full for the LDS buffer, or the score range is not
//    finite, the bitwise search runs over all keys instead.
// 2. Every key > T is kept; of the keys equal to T, the first
//    want - count(> T) in index order are kept.  The kept indices are
//    compacted in ascending index order with ballot/mbcnt, so emit(pos,
//    index) receives pos = 0 .. want-1 in index order.
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

__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

template <int NW>
__device__ __forceinline__ int wg_sum(int v, int* red, int parity) {
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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = max(v, (uint32_t)shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = min(v, (uint32_t)shfl_xor((int)v, o));
  return v;
}

// Bitwise search over all registers of all waves: T and count(key > T).
template <int NW, int R>
__device__ __forceinline__ uint32_t full_threshold(const uint32_t (&key)[R], int want, int* red) {
  uint32_t T = 0;
  int parity = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += __popcll(ballot(key[r] >= cand));
    cnt = wg_sum<NW>(cnt, red, parity);
    parity ^= 1;
    if (cnt >= want) T = cand;
  }
  return T;
}

// The want-th largest key (1 <= want <= number of non-empty keys).
// Exact search over the n compacted keys of the target bin by wave 0.
template <int R2>
__device__ __forceinline__ uint32_t bin_threshold(const uint32_t* cand, int n, int need) {
  const int lane = lane_id();
  uint32_t ck[R2];
#pragma unroll
  for (int r = 0; r < R2; ++r) {
    const int idx = r * kWave + lane;
    ck[r] = idx < n ? cand[idx] : 0u;
  }
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R2; ++r) cnt += __popcll(ballot(ck[r] >= c));
    if (cnt >= need) T = c;
  }
  return T;
}

template <int NW, int R>
__device__ __forceinline__ uint32_t find_threshold(const uint32_t (&key)[R], int want, SelectSmem<NW>& sm) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  constexpr int NT = NW * kWave;
  // few keys per lane: the plain bitwise search is cheaper than the histogram
  if constexpr (R < 8) return full_threshold<NW, R>(key, want, sm.red);

  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    hi = max(hi, key[r]);
    lo = min(lo, key[r] ? key[r] : 0xFFFFFFFFu);
  }
  hi = wave_max_u32(hi);
  lo = wave_min_u32(lo);
  for (int b = threadIdx.x; b < kBins; b += NT) sm.hist[b] = 0;
  if (lane == 0) {
    sm.kmin[wave] = lo;
    sm.kmax[wave] = hi;
  }
  if (threadIdx.x == 0) sm.info[2] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, sm.kmin[w]);
    hi = max(hi, sm.kmax[w]);
  }
  if (lo == hi) return hi;  // every non-empty key is equal
  const float smin = key_to_score(lo);
  const float range = key_to_score(hi) - smin;
  if (!(range < INFINITY)) {
    __syncthreads();
    return full_threshold<NW, R>(key, want, sm.red);
  }
  const float scale = (float)kBins / range;
  auto bin_of = [&](uint32_t k) { return min((int)((key_to_score(k) - smin) * scale), kBins - 1); };
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (key[r]) atomicAdd(&sm.hist[bin_of(key[r])], 1);
  __syncthreads();
  if (wave == 0) {
    // suffix sums over bins: lane l holds bins 4l .. 4l+3
    const int c0 = sm.hist[4 * lane], c1 = sm.hist[4 * lane + 1], c2 = sm.hist[4 * lane + 2],
              c3 = sm.hist[4 * lane + 3];
    const int mine = c0 + c1 + c2 + c3;
    int incl = mine;  // sum over lanes >= l
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_down(incl, o, kWave);
      if (lane + o < kWave) incl += v;
    }
    int above = incl - mine;  // keys in bins of higher lanes
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
  __syncthreads();
  const int tb = sm.info[0];
  const int above = sm.info[1];
  const int need = want - above;
  if (sm.hist[tb] > kBinCap) {
    __syncthreads();
    return full_threshold<NW, R>(key, want, sm.red);
  }
  // compact the target bin's keys (any order)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool in = key[r] != 0u && bin_of(key[r]) == tb;
    const uint64_t m = ballot(in);
    if (m) {
      const int first = __builtin_ctzll(m);
      int base = 0;
      if (lane == first) base = atomicAdd(&sm.info[2], __popcll(m));
      base = __shfl(base, first, kWave);
      if (in) sm.cand[base + lanes_below(m)] = key[r];
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int n = sm.info[2];
    uint32_t T;
    if (n <= 64) T = bin_threshold<1>(sm.cand, n, need);
    else if (n <= 256) T = bin_threshold<4>(sm.cand, n, need);
    else T = bin_threshold<kBinCap / kWave>(sm.cand, n, need);
    if (lane == 0) sm.info[3] = (int)T;
  }
  __syncthreads();
  return (uint32_t)sm.info[3];
}

// Requires: 1 <= want < number of non-empty keys.  Must be called by every
// thread of the workgroup (it contains barriers).
template <int NW, int R, typename Emit>
__device__ __forceinline__ void select_top(const uint32_t (&key)[R], int want, SelectSmem<NW>& sm, Emit&& emit) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const uint32_t T = find_threshold<NW, R>(key, want, sm);

  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    gt += __popcll(ballot(key[r] > T));
    eq += __popcll(ballot(key[r] == T));
  }
  int* g = sm.red + 2 * NW;  // the search passes use red[0 .. 2 NW)
  int* e = sm.red + 3 * NW;
  if (lane == 0) {
    g[wave] = gt;
    e[wave] = eq;
  }
  __syncthreads();
  int gt_total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) gt_total += g[w];
  const int need_eq = want - gt_total;
  int eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) {
    const int take = min(max(need_eq - eq_before, 0), e[w]);
    sel_before += g[w] + take;
    eq_before += e[w];
  }

  int e_run = eq_before, o_run = sel_before;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool is_eq = key[r] == T;
    const uint64_t eqm = ballot(is_eq);
    const bool take = key[r] > T || (is_eq && e_run + (int)lanes_below(eqm) < need_eq);
    const uint64_t selm = ballot(take);
    if (take) emit(o_run + (int)lanes_below(selm), wave * kWave * R + r * kWave + lane);
    o_run += __popcll(selm);
    e_run += __popcll(eqm);
  }
  __syncthreads();  // LDS may be reused by the caller
}

}  // namespace hsa
