// Exact top-`want` selection with ties broken toward the lower index.
//
// The keys live in registers.  A workgroup of NW waves holds up to
// NW * 64 * R keys; wave w owns the contiguous index range
// [w * 64 * R, (w + 1) * 64 * R) and key[r] of lane l has index
// w * 64 * R + r * 64 + l.  Key 0 marks an empty slot.
//
// Method: a bitwise binary search finds the threshold T, the largest key x
// with count(key >= x) >= want (32 rounds; each round counts with one
// compare + ballot + popcount per register, the waves' counts meet in LDS).
// Every key > T is kept; of the keys equal to T, the first want - count(> T)
// in index order are kept.  The kept indices are then compacted in
// ascending index order with ballot/mbcnt, so emit(pos, index) receives
// pos = 0 .. want-1 in index order.
#pragma once

#include "common.hpp"

namespace hsa {

template <int NW>
__device__ __forceinline__ int wg_sum(int v, int* lds, int parity) {
  if constexpr (NW == 1) {
    return v;
  } else {
    const int wave = threadIdx.x / kWave;
    int* buf = lds + parity * NW;
    if (lane_id() == 0) buf[wave] = v;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += buf[w];
    return s;
  }
}

// LDS words needed by select_top<NW>.
template <int NW>
constexpr int select_lds_words() { return 4 * NW; }

// Requires: 1 <= want < number of non-empty keys.  Must be called by every
// thread of the workgroup (it contains barriers when NW > 1).
template <int NW, int R, typename Emit>
__device__ __forceinline__ void select_top(const uint32_t (&key)[R], int want, int* lds, Emit&& emit) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();

  uint32_t T = 0;
  int parity = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += __popcll(ballot(key[r] >= cand));
    cnt = wg_sum<NW>(cnt, lds, parity);
    parity ^= 1;
    if (cnt >= want) T = cand;
  }

  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    gt += __popcll(ballot(key[r] > T));
    eq += __popcll(ballot(key[r] == T));
  }

  int gt_total, eq_before, sel_before;
  if constexpr (NW == 1) {
    gt_total = gt;
    eq_before = 0;
    sel_before = 0;
  } else {
    int* g = lds + 2 * NW;
    int* e = lds + 3 * NW;
    if (lane == 0) {
      g[wave] = gt;
      e[wave] = eq;
    }
    __syncthreads();
    gt_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) gt_total += g[w];
    const int need = want - gt_total;
    eq_before = 0;
    sel_before = 0;
    for (int w = 0; w < wave; ++w) {
      const int take = min(max(need - eq_before, 0), e[w]);
      sel_before += g[w] + take;
      eq_before += e[w];
    }
  }
  const int need_eq = want - gt_total;

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
  if constexpr (NW > 1) __syncthreads();  // LDS may be reused by the caller
}

}  // namespace hsa
