// Step 3's exact top-k of one query over its candidate slots, shared by the
// token select kernel and the decode kernel that runs the select and the
// attention in one launch.
//
// HISA page, second stage: only the tokens of the kept blocks are scored,
// and the k best of them are the query's token list.  A query with no more
// causal candidates than k keeps all of them.
#pragma once

#include "common.hpp"
#include "select.hpp"

namespace hsa {

// Candidates of the query at position t: its own block c, the number of
// kept blocks n_sel = min(c + 1, m) and of causal slots n_valid (upper
// bounds: a block list may be shorter, see select_query_tokens).
__device__ __forceinline__ void candidate_count(int t, int B, int m, int& c, int& n_sel, int& n_valid) {
  c = t / B;
  n_sel = (c + 1 <= m) ? c + 1 : m;
  n_valid = (n_sel - 1) * B + (t - c * B + 1);
}

// The token list of query q (row q of blk / scores) by the NW * 64 threads
// of the workgroup.  Slot s of the query is token (bl[s / B] * B + s % B);
// its score is scores[q * m * B + s].  `bl` is LDS for the block list (m
// entries, padded to a multiple of 4).
//
// When the query keeps all of its candidates, keep(slot, token) is called
// for every slot in [keep_lo, keep_hi) (token -1 past the causal ones), each
// slot by one thread, and the function returns false (no barrier at its
// end).  Otherwise the select runs and emit(pos, token, take) is called as
// select_top_f calls its emitter (every k positions taken once, take = false
// for a thread's other calls); the function returns true, and with END_SYNC
// the workgroup has passed a barrier after the last emit.
//
// ONEBLK: R <= B (both powers of two), so a thread's R slots lie in one
// kept block and its tokens are one base plus the slot offset.
template <int NW, int R, bool ONEBLK, bool END_SYNC, typename Keep, typename Emit>
__device__ __forceinline__ bool select_query_tokens(const float* __restrict__ scores, const int32_t* __restrict__ blk,
                                                    int q, int L, int nq, int B, int log2B, int m, int k,
                                                    const int32_t* __restrict__ lens, int keep_lo, int keep_hi,
                                                    SelectSmem<NW>& lds, int* bl, Keep&& keep, Emit&& emit) {
  constexpr int NT = NW * 64;
  const int i = q % nq;
  const int t = query_pos(seq_len_of(lens, L, q / nq), nq, i);
  int c, n_sel, n_valid;
  candidate_count(t, B, m, c, n_sel, n_valid);  // upper bounds: the list may be shorter
  const int32_t* blq = blk + (size_t)q * m;
  if (n_valid <= k) {
    // keep all: a slot is a token iff its entry is a block and the token is
    // causal; the invalid slots all follow the valid ones
    for (int slot = keep_lo + (int)threadIdx.x; slot < keep_hi; slot += NT) {
      const int j = slot < n_valid ? blq[slot >> log2B] : -1;
      const int tk = (j << log2B) + (slot & (B - 1));
      keep(slot, (j >= 0 && slot < n_valid && tk <= t) ? tk : -1);
    }
    return false;
  }
  // the slot scores do not depend on the block list: both loads in flight
  // together, one round trip before the barrier (slots past the list's
  // real length are read but masked below)
  const float* sc = scores + (size_t)q * m * B;  // 32-byte aligned: m * B is a multiple of 8
  const int idx0 = threadIdx.x * R;
  const float empty = __uint_as_float(0x7FC00000u);  // quiet NaN: an empty slot of select_top_f
  float v[R];
  if constexpr (R >= 4) {
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      if (idx0 + r + 3 < n_valid) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(sc + idx0 + r);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[r + e] = x[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = idx0 + r + e;
          v[r + e] = idx < n_valid ? sc[idx] : empty;
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = idx0 + r;
      v[r] = idx < n_valid ? sc[idx] : empty;
    }
  }
  for (int p = threadIdx.x; p < n_sel; p += NT) bl[p] = blq[p];
  __syncthreads();
  // the list's length: its entries are a valid prefix, then -1
  if (bl[n_sel - 1] < 0) {  // (uniform) shorter than min(c + 1, m)
    int lo = 0, hi = n_sel - 1;  // bl[lo] is valid, bl[hi] is not
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (bl[mid] >= 0) lo = mid;
      else hi = mid;
    }
    n_sel = lo + 1;
    n_valid = (n_sel - 1) * B + (t - c * B + 1);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (idx0 + r >= n_valid) v[r] = empty;
    if (n_valid <= k) {
      for (int slot = keep_lo + (int)threadIdx.x; slot < keep_hi; slot += NT) {
        const int j = slot < n_valid ? bl[slot >> log2B] : -1;
        keep(slot, slot < n_valid ? (j << log2B) + (slot & (B - 1)) : -1);
      }
      return false;
    }
  }
  const int bmask = B - 1;
  const int tbase = ONEBLK ? (bl[min(idx0 >> log2B, n_sel - 1)] << log2B) | (idx0 & bmask) : 0;
  select_top_f<NW, R, END_SYNC>(v, k, NT * R - n_valid, lds, [&](int pos, int idx, bool take) {
    emit(pos, ONEBLK ? tbase + (idx - idx0) : (bl[idx >> log2B] << log2B) | (idx & bmask), take);
  });
  return true;
}

}  // namespace hsa
