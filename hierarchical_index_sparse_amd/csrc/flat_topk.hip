// The flat indexer: for every query, score every causal token s <= t with
// the indexer's dot product and keep the top-k.
//
// HISA page (the problem and the original method): the indexer scores each
// query against all previous tokens and keeps the most relevant ones; the
// hierarchical method replaces exactly this step, and degrades to it when
// every block is kept.  Built here as the baseline the hierarchical path is
// measured against, with the same output form (ascending token lists,
// padded with -1; ties to the lower index).
//
// Kernel 1 (k_flat_scores): S^T = kI qI^T on v_mfma_f32_16x16x32_bf16 for
// 64 queries x 512 tokens per workgroup (A = 16 key rows, B = 16 queries);
// each wave keeps the 64 queries in registers over its 128 tokens, and each
// lane holds 4 consecutive tokens of one query and writes them with one
// 16-byte store.  Tiles after the tile's last query are skipped.  Bound by
// the score writes (4 bytes per causal pair).
//
// Kernel 2, contexts of at most 65536 tokens (k_flat_row_select): one
// 16-wave workgroup per query selects from its whole score row held in
// registers (up to 64 keys per thread), in one pass over the row.
// Longer contexts (k_flat_chunk_select): the t+1 candidates of a query are cut into
// chunks of kFlatChunk tokens (what one 4-wave select holds in registers);
// each chunk keeps its own top-min(k, n) with the exact select of
// select.hpp.  A query with a single chunk writes its list directly.
// Kernel 3 (k_flat_merge): groups of up to 8192 / k (k <= 2048, 4 waves) or
// 32768 / k (16 waves) chunk winners are
// merged by the same select until one list per query remains.  The global
// top-k under (score desc, index asc) is contained in the union of the
// chunks' top-k under the same order, and every level keeps the lists in
// ascending index order, so ties resolve exactly as in one select.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace hsa {

constexpr int kFlatChunk = 4 * 64 * 32;   // 8192 keys per chunk select: 4 waves x 64 lanes x 32
// merge selects: 4 waves (8192 keys) while that holds four lists of k, else 16 waves (32768 keys)
constexpr int kFlatMergeSmall = 4 * 64 * 32;
constexpr int kFlatMergeLarge = 16 * 64 * 32;
constexpr int kFlatStageMax = 8192;
constexpr int kFlatKeysPerWG = 512;  // score tile: 64 queries x 512 tokens (128 per wave)

template <int DI, bool STREAM>
__global__ __launch_bounds__(256) void k_flat_scores(const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI,
                                                     float* __restrict__ scores, int L, int nq, int Lp,
                                                     int qtiles_per_seq) {
  constexpr int KS = DI / 32;
  const int b = blockIdx.y / qtiles_per_seq;
  const int i0 = (blockIdx.y % qtiles_per_seq) * 64;
  const int t_last = query_pos(L, nq, min(nq, i0 + 64) - 1);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int jl = lane & 15, gq = lane >> 4;
  const int wkey0 = blockIdx.x * kFlatKeysPerWG + wave * (kFlatKeysPerWG / 4);  // this wave's first token
  if (wkey0 > t_last) return;

  // B operands: the 64 queries (4 tiles of 16), kept for all of the wave's keys
  u32x4 qb[4][KS];
  int tq[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int i = min(i0 + 16 * mt + jl, nq - 1);
    const uint16_t* qsrc = qI + ((size_t)b * nq + i) * DI + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[mt][ks] = *reinterpret_cast<const u32x4*>(qsrc + 32 * ks);
    tq[mt] = i0 + 16 * mt + jl < nq ? query_pos(L, nq, i) : -1;  // -1: no such query
  }
  for (int key0 = wkey0; key0 < wkey0 + kFlatKeysPerWG / 4 && key0 <= t_last; key0 += 32) {
    // A operands: 2 tiles of 16 key rows
    u32x4 ka[2][KS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int row = min(key0 + 16 * kt + jl, L - 1);
      const uint16_t* src = kI + ((size_t)b * L + row) * DI + 8 * gq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[kt][ks] = *reinterpret_cast<const u32x4*>(src + 32 * ks);
    }
    // the 8 (query tile, key tile) accumulators advance together over ks:
    // eight independent MFMA chains in flight
    f32x4 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[mt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          acc[mt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kt][ks]),
                                                                __builtin_bit_cast(bf16x8, qb[mt][ks]), acc[mt][kt],
                                                                0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float* dst = scores + ((size_t)b * nq + i0 + 16 * mt + jl) * Lp;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // lane: tokens s0 .. s0+3 of query i0 + 16mt + jl
        const int s0 = key0 + 16 * kt + 4 * gq;
        if (s0 <= tq[mt]) {
          if constexpr (STREAM) __builtin_nontemporal_store(acc[mt][kt], reinterpret_cast<f32x4*>(dst + s0));
          else *reinterpret_cast<f32x4*>(dst + s0) = acc[mt][kt];
        }
      }
    }
  }
}

// Rows of at most kFlatRowMax candidates (contexts up to 64K tokens): one
// 16-wave workgroup per query holds the whole score row in registers
// (R scores per thread) and runs the exact select of select.hpp once, with
// the kept tokens staged in LDS and written in coalesced stores.  The row
// is read from memory once and nothing is merged.  Queries are launched in
// groups of similar row length (R = the smallest power of two with
// 1024 R >= t + 1), so short rows do not pay for the longest.
constexpr int kFlatRowMax = 16 * 64 * 64;

template <int R>
__global__ __launch_bounds__(1024) void k_flat_row_select(const float* __restrict__ scores, int32_t* __restrict__ tok,
                                                          int L, int nq, int Lp, int k, int i_lo) {
  constexpr int NT = 1024;
  __shared__ SelectSmem<16> lds;
  extern __shared__ int stage[];  // k + 64 ints
  const int i = i_lo + (int)blockIdx.x;
  const size_t q = (size_t)blockIdx.y * nq + i;
  const int n = query_pos(L, nq, i) + 1;  // candidates: tokens 0 .. t
  int32_t* out = tok + q * k;
  if (n <= k) {  // every causal token is kept
    for (int s = threadIdx.x; s < k; s += NT) out[s] = s < n ? s : -1;
    return;
  }
  const float* sc = scores + q * Lp;
  const int idx0 = threadIdx.x * R;
  const float empty = __uint_as_float(0x7FC00000u);  // quiet NaN: an empty slot of select_top_f
  float v[R];
  if constexpr (R >= 4) {
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      if (idx0 + r + 3 < n) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(sc + idx0 + r);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[r + e] = x[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[r + e] = idx0 + r + e < n ? sc[idx0 + r + e] : empty;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = idx0 + r < n ? sc[idx0 + r] : empty;
  }
  const int dummy = k + lane_id();
  if constexpr (R <= 32) {
    select_top_f<16, R>(v, k, NT * R - n, lds, [&](int pos, int idx, bool take) { stage[take ? pos : dummy] = idx; });
  } else {
    // (64 per thread: the key form, which spills fewer of the 128 registers
    // a 1024-thread workgroup allows)
    uint32_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) key[r] = v[r] == v[r] ? score_key(v[r]) : 0u;
    select_top<16, R>(key, k, lds, [&](int pos, int idx, bool take, uint32_t) { stage[take ? pos : dummy] = idx; });
  }
  if ((k & 3) == 0) {
    for (int p = threadIdx.x * 4; p < k; p += NT * 4)
      *reinterpret_cast<i32x4*>(out + p) = *reinterpret_cast<const i32x4*>(stage + p);
  } else {
    for (int p = threadIdx.x; p < k; p += NT) out[p] = stage[p];
  }
}

// Rows of more than kFlatStreamMin candidates: one 4-wave workgroup per
// query selects straight from the score row in memory, in passes (after the
// first, the row, at most 256 KB, comes from L2).  Wave w owns a contiguous
// segment of the row and reads it with coalesced 16-byte loads, so index
// order is segment, then load, then lane, then element.
//   1. the row's minimum and maximum;
//   2. a 255-bin linear histogram between them and a suffix scan for the bin
//      that holds the want-th largest score; a bin of more than kBinCap
//      scores is narrowed to its own minimum and maximum and histogrammed
//      again (a few levels at most; a bitwise search over all keys if that
//      does not end it);
//   3. the bin's scores compacted into LDS and the threshold found exactly
//      among them (bitwise search over their keys, one wave);
//   4. counts of scores above and equal to the threshold per wave: the
//      ties kept are the first ones in index order;
//   5. the kept indices written in ascending order, each at the slot wave
//      scans give it.
// Few registers and 5 KB of LDS per workgroup: many workgroups share a CU,
// where the register-resident select of one 1024-thread workgroup per
// query left each CU one select at a time.
constexpr int kFlatStreamMin = 16384;

__global__ __launch_bounds__(256) void k_flat_stream_select(const float* __restrict__ scores,
                                                            int32_t* __restrict__ tok, int L, int nq, int Lp, int k,
                                                            int i_lo) {
  constexpr int NW = 4;
  constexpr int NT = NW * kWave;
  __shared__ int hist[kBins];
  __shared__ uint32_t cand[kBinCap];
  __shared__ uint32_t wlo[NW], whi[NW];
  __shared__ int wcnt[2][NW];
  __shared__ int info[4];  // target bin, count above it, compaction slot, threshold key
  const int i = i_lo + (int)blockIdx.x;
  const size_t q = (size_t)blockIdx.y * nq + i;
  const int n = query_pos(L, nq, i) + 1;  // candidates: tokens 0 .. t
  int32_t* out = tok + q * k;
  const int tid = threadIdx.x;
  if (n <= k) {  // every causal token is kept
    for (int x = tid; x < k; x += NT) out[x] = x < n ? x : -1;
    return;
  }
  const float* row = scores + q * Lp;
  const int wave = tid / kWave, lane = lane_id();
  const int segw = (n + NW * 256 - 1) / (NW * 256) * 256;  // 64 lanes x 4 per load
  const int s0 = min(n, wave * segw), s1 = min(n, s0 + segw);
  const int want = k;
  auto load4 = [&](int b, float (&v)[4], bool (&ok)[4]) {
    const int idx = b + 4 * lane;
    if (idx + 3 < s1) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(row + idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = x[e];
        ok[e] = true;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok[e] = idx + e < s1;
        v[e] = ok[e] ? row[idx + e] : 0.f;
      }
    }
  };
  // minimum and maximum over the group, as keys (order-preserving)
  auto group_minmax = [&](uint32_t lo, uint32_t hi, uint32_t& glo, uint32_t& ghi) {
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
      wlo[wave] = lo;
      whi[wave] = hi;
    }
    __syncthreads();
    glo = wlo[0];
    ghi = whi[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      glo = min(glo, wlo[w]);
      ghi = max(ghi, whi[w]);
    }
  };
  auto group_count = [&](int c, int slot) {
    c = wave_incl_scan(c);
    c = __builtin_amdgcn_readlane(c, kWave - 1);
    if (lane == 0) wcnt[slot][wave] = c;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) total += wcnt[slot][w];
    return total;
  };

  // 1. extremes of the row
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;
  for (int b = s0; b < s1; b += 256) {
    float v[4];
    bool ok[4];
    load4(b, v, ok);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[e]) {
        const uint32_t kk = score_key(v[e]);
        klo = min(klo, kk);
        khi = max(khi, kk);
      }
  }
  for (int x = tid; x < kBins; x += NT) hist[x] = 0;
  if (tid == 0) info[2] = 0;
  uint32_t glo, ghi;
  group_minmax(klo, khi, glo, ghi);

  // 2.-3. the threshold key T
  uint32_t T = 0;
  bool found = false;
  int above = 0;  // scores above the interval [glo, ghi] (all kept)
  for (int level = 0; level < 6; ++level) {
    if (glo == ghi) {  // every score left in the interval is equal
      T = ghi;
      found = true;
      break;
    }
    const float flo = key_to_score(glo), fhi = key_to_score(ghi);
    const float range = fhi - flo;
    if (!(range < INFINITY)) break;
    const float scale = (float)(kBins - 1) / range;
    auto bin_of = [&](float x) { return min((int)((x - flo) * scale), kBins - 2); };
    for (int b = s0; b < s1; b += 256) {
      float v[4];
      bool ok[4];
      load4(b, v, ok);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok[e] && v[e] >= flo && v[e] <= fhi) atomicAdd(&hist[bin_of(v[e])], 1);
    }
    __syncthreads();
    const int need = want - above;
    if (wave == 0) {
      const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                c3 = lane == kWave - 1 ? 0 : hist[4 * lane + 3];
      const int pre = wave_incl_scan(c0 + c1 + c2 + c3);
      int abv = __builtin_amdgcn_readlane(pre, kWave - 1) - pre;
      const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (abv < need && need <= abv + cs[e]) {
          info[0] = 4 * lane + e;
          info[1] = abv;
        }
        abv += cs[e];
      }
    }
    __syncthreads();
    const int tb = info[0];
    const int cnt = hist[tb];
    above += info[1];
    if (cnt <= kBinCap) {
      // compact the bin's scores (any order) and search among them
      for (int b = s0; b < s1; b += 256) {
        float v[4];
        bool ok[4];
        load4(b, v, ok);
        int c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c += ok[e] && v[e] >= flo && v[e] <= fhi && bin_of(v[e]) == tb;
        int wtot;
        int pos = wave_excl_scan(c, wtot);
        int base = 0;
        if (lane == 0 && wtot) base = atomicAdd(&info[2], wtot);
        pos += __builtin_amdgcn_readlane(base, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ok[e] && v[e] >= flo && v[e] <= fhi && bin_of(v[e]) == tb) cand[pos++] = __float_as_uint(v[e]);
      }
      __syncthreads();
      if (wave == 0) {
        const int nc = info[2];
        const int need_bin = want - above;
        uint32_t Tb;
        if (nc <= 64) Tb = bin_threshold<1, true>(cand, nc, need_bin);
        else if (nc <= 256) Tb = bin_threshold<4, true>(cand, nc, need_bin);
        else Tb = bin_threshold<kBinCap / kWave, true>(cand, nc, need_bin);
        if (lane == 0) info[3] = (int)Tb;
      }
      __syncthreads();
      T = (uint32_t)info[3];
      found = true;
      break;
    }
    // narrow the interval to the bin's own extremes and histogram again
    uint32_t blo = 0xFFFFFFFFu, bhi = 0u;
    for (int b = s0; b < s1; b += 256) {
      float v[4];
      bool ok[4];
      load4(b, v, ok);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok[e] && v[e] >= flo && v[e] <= fhi && bin_of(v[e]) == tb) {
          const uint32_t kk = score_key(v[e]);
          blo = min(blo, kk);
          bhi = max(bhi, kk);
        }
    }
    __syncthreads();  // every thread has read hist[tb] and info
    for (int x = tid; x < kBins; x += NT) hist[x] = 0;
    group_minmax(blo, bhi, glo, ghi);
  }
  if (!found) {
    // bitwise search over the keys of the whole row: the largest T with
    // at least `want` keys >= T
    T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c_t = T | (1u << bit);
      int c = 0;
      for (int b = s0; b < s1; b += 256) {
        float v[4];
        bool ok[4];
        load4(b, v, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) c += ok[e] && score_key(v[e]) >= c_t;
      }
      if (group_count(c, bit & 1) >= want) T = c_t;
      __syncthreads();  // wcnt[bit & 1] is rewritten two bits later
    }
  }
  const float Tf = key_to_score(T);

  // 4. scores above / equal to T per wave; ties to the lowest indices
  int gt = 0, eq = 0;
  for (int b = s0; b < s1; b += 256) {
    float v[4];
    bool ok[4];
    load4(b, v, ok);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt += ok[e] && v[e] > Tf;
      eq += ok[e] && v[e] == Tf;
    }
  }
  __syncthreads();  // wcnt may still be read by the bitwise search
  gt = __builtin_amdgcn_readlane(wave_incl_scan(gt), kWave - 1);
  eq = __builtin_amdgcn_readlane(wave_incl_scan(eq), kWave - 1);
  if (lane == 0) {
    wcnt[0][wave] = gt;
    wcnt[1][wave] = eq;
  }
  __syncthreads();
  int gt_total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) gt_total += wcnt[0][w];
  const int need_eq = want - gt_total;
  int pos = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    pos += wcnt[0][w] + min(max(need_eq - eq_before, 0), wcnt[1][w]);
    eq_before += wcnt[1][w];
  }
  const int ties = min(max(need_eq - eq_before, 0), wcnt[1][wave]);  // this wave's kept ties

  // 5. write the kept indices in order
  int ties_used = 0;
  for (int b = s0; b < s1; b += 256) {
    float v[4];
    bool ok[4];
    load4(b, v, ok);
    int te = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) te += ok[e] && v[e] == Tf;
    int tw;
    int tr = ties_used + wave_excl_scan(te, tw);  // ties before this lane's first, in index order
    bool keep[4];
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool is_eq = ok[e] && v[e] == Tf;
      keep[e] = (ok[e] && v[e] > Tf) || (is_eq && tr < ties);
      tr += is_eq;
      c += keep[e];
    }
    ties_used += tw;
    int cw;
    int p = pos + wave_excl_scan(c, cw);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (keep[e]) out[p++] = b + 4 * lane + e;
    pos += cw;
  }
}

// One (query, chunk).  Lists of chunk winners are (key, token) pairs in
// ascending token order with their count.
template <int NW, int R>
__global__ __launch_bounds__(NW * 64) void k_flat_chunk_select(const float* __restrict__ scores,
                                                               uint2* __restrict__ lists, int* __restrict__ counts,
                                                               int32_t* __restrict__ tok, int L, int nq, int Lp,
                                                               int k, int nchunk) {
  constexpr int NT = NW * 64;
  static_assert(NT * R <= kFlatChunk, "a chunk must fit the group");
  __shared__ SelectSmem<NW> lds;
  extern __shared__ int stage[];  // k + 64 ints (final lists are staged)
  const int q = blockIdx.x;
  const int c = blockIdx.y;
  const int t = query_pos(L, nq, q % nq);
  const int n_all = t + 1;
  int32_t* out = tok + (size_t)q * k;
  if (n_all <= k) {  // every causal token is kept
    if (c == 0)
      for (int s = threadIdx.x; s < k; s += NT) out[s] = s < n_all ? s : -1;
    return;
  }
  const int lo = c * kFlatChunk;
  if (lo >= n_all) return;
  const int n = min(kFlatChunk, n_all - lo);
  const bool single = n_all <= kFlatChunk;  // then c == 0 and the list is final
  const float* sc = scores + (size_t)q * Lp + lo;
  const int idx0 = threadIdx.x * R;
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; r += 4) {
    if (idx0 + r + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sc + idx0 + r);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[r + e] = score_key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) key[r + e] = idx0 + r + e < n ? score_key(sc[idx0 + r + e]) : 0u;
    }
  }
  uint2* lst = lists + ((size_t)q * nchunk + c) * k;
  if (n <= k) {  // a short last chunk: all of it goes to the merge
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (idx0 + r < n) lst[idx0 + r] = make_uint2(key[r], (unsigned)(lo + idx0 + r));
    if (threadIdx.x == 0) counts[(size_t)q * nchunk + c] = n;
    return;
  }
  if (single) {  // k <= kFlatStageMax (checked at the API): the list is staged in LDS
    const int dummy = k + lane_id();
    select_top<NW, R>(key, k, lds, [&](int pos, int idx, bool take, uint32_t) { stage[take ? pos : dummy] = lo + idx; });
    for (int p = threadIdx.x; p < k; p += NT) out[p] = stage[p];
    return;
  }
  select_top<NW, R>(key, k, lds, [&](int pos, int idx, bool take, uint32_t kv) {
    if (take) lst[pos] = make_uint2(kv, (unsigned)(lo + idx));
  });
  if (threadIdx.x == 0) counts[(size_t)q * nchunk + c] = k;
}

// One (query, group of up to G lists) of a merge level: n_in lists per query
// at this level (fewer for early queries), n_in = ceil(n_chunks_of_query /
// G^level).  Writes list `grp` of the next level, or the final tokens when
// this group is the query's only one.
template <int NW, int R>
__global__ __launch_bounds__(NW * 64) void k_flat_merge(const uint2* __restrict__ lin, const int* __restrict__ cin,
                                                        uint2* __restrict__ lout, int* __restrict__ cout,
                                                        int32_t* __restrict__ tok, int L, int nq, int k, int nchunk,
                                                        int G, int level) {
  constexpr int NT = NW * 64;
  __shared__ SelectSmem<NW> lds;
  extern __shared__ int stage[];  // k + 64 ints
  const int q = blockIdx.x;
  const int grp = blockIdx.y;
  const int t = query_pos(L, nq, q % nq);
  const int n_all = t + 1;
  if (n_all <= k || n_all <= kFlatChunk) return;  // finished by the chunk select
  int n_in = (n_all + kFlatChunk - 1) / kFlatChunk;
  for (int l = 0; l < level; ++l) n_in = (n_in + G - 1) / G;
  if (n_in <= 1) return;  // finished at an earlier level
  const int first = grp * G;
  if (first >= n_in) return;
  const int nl = min(G, n_in - first);
  const bool final_list = n_in <= G;
  // candidates: lists first .. first+nl-1; every list but the last holds k
  const int cnt_last = cin[(size_t)q * nchunk + first + nl - 1];
  const int n = (nl - 1) * k + cnt_last;
  const uint2* src = lin + ((size_t)q * nchunk + first) * k;  // list j of the group starts at j * k
  const int idx0 = threadIdx.x * R;
  // only the keys stay in registers (R of them, up to 32 with 16 waves);
  // a kept key's token is read back from the list when it is emitted
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = idx0 + r;
    key[r] = s < n ? src[s].x : 0u;
  }
  if (final_list) {
    int32_t* out = tok + (size_t)q * k;
    if (n <= k) {  // every candidate is kept (in index order)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (idx0 + r < k) out[idx0 + r] = idx0 + r < n ? (int)src[idx0 + r].y : -1;
      for (int p = NT * R + threadIdx.x; p < k; p += NT) out[p] = -1;
      return;
    }
    const int dummy = k + lane_id();
    select_top<NW, R>(key, k, lds, [&](int pos, int idx, bool take, uint32_t) {
      stage[take ? pos : dummy] = take ? (int)src[idx].y : 0;
    });
    for (int p = threadIdx.x; p < k; p += NT) out[p] = stage[p];
    return;
  }
  uint2* dst = lout + ((size_t)q * nchunk + grp) * k;
  if (n <= k) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (idx0 + r < n) dst[idx0 + r] = src[idx0 + r];
    if (threadIdx.x == 0) cout[(size_t)q * nchunk + grp] = n;
    return;
  }
  select_top<NW, R>(key, k, lds, [&](int pos, int idx, bool take, uint32_t kv) {
    if (take) dst[pos] = make_uint2(kv, src[idx].y);
  });
  if (threadIdx.x == 0) cout[(size_t)q * nchunk + grp] = k;
}

// ----------------------------------------------------------------- host side

// seq_len <= 2^30 (checked by the caller), so both fit in an int
static int flat_nchunk(const Dims& s) { return (int)(((long long)s.L + kFlatChunk - 1) / kFlatChunk); }
static int flat_lp(const Dims& s) { return (int)(((long long)s.L + 3) & ~3ll); }
static bool flat_row_select(const Dims& s) { return s.k < s.L && s.L <= kFlatRowMax; }
static bool flat_needs_lists(const Dims& s) { return s.k < s.L && !flat_row_select(s) && flat_nchunk(s) > 1; }

bool flat_topk_supported(const Dims& s) {
  if (s.k >= s.L) return true;  // everything is kept: no select
  // final lists are staged in LDS; a merge group holds at least two lists
  return s.k <= kFlatStageMax;  // a merge group then holds at least 32768 / 8192 = 4 lists
}

size_t flat_topk_ws_bytes(const Dims& s) {
  const size_t nqt = (size_t)s.b * s.nq;
  if (s.k >= s.L) return 0;
  size_t bytes = align_up(nqt * flat_lp(s) * sizeof(float));
  if (flat_needs_lists(s)) {
    const size_t lists = nqt * flat_nchunk(s) * s.k;
    bytes += 2 * align_up(lists * sizeof(uint2)) + 2 * align_up(nqt * flat_nchunk(s) * sizeof(int));
  }
  return bytes;
}

template <int NW, int R>
static void launch_merge(dim3 grid, size_t dyn, const uint2* lin, const int* cin, uint2* lout, int* cout,
                         int32_t* tok, const Dims& s, int nchunk, int G, int level, hipStream_t st) {
  HSA_LAUNCH((k_flat_merge<NW, R>), grid, dim3(NW * 64), dyn, st, lin, cin, lout, cout, tok, s.L, s.nq, s.k,
                     nchunk, G, level);
}

hipError_t launch_flat_topk(const Dims& s, const uint16_t* qI, const uint16_t* kI, int32_t* tok, void* ws,
                            hipStream_t st) {
  const int nq_total = s.b * s.nq;
  if (nq_total == 0) return hipSuccess;
  const int nchunk = flat_nchunk(s);
  const int Lp = flat_lp(s);
  unsigned char* p = static_cast<unsigned char*>(ws);
  float* scores = reinterpret_cast<float*>(p);
  if (s.k < s.L) {
    const int qtiles = (s.nq + 63) / 64;
    dim3 grid((s.L + kFlatKeysPerWG - 1) / kFlatKeysPerWG, qtiles * s.b);
    const bool nt = (size_t)nq_total * Lp * sizeof(float) > kStreamStoreBytes;
    if (s.dI == 64 && nt)
      HSA_LAUNCH((k_flat_scores<64, true>), grid, dim3(256), 0, st, qI, kI, scores, s.L, s.nq, Lp, qtiles);
    else if (s.dI == 64)
      HSA_LAUNCH((k_flat_scores<64, false>), grid, dim3(256), 0, st, qI, kI, scores, s.L, s.nq, Lp, qtiles);
    else if (nt)
      HSA_LAUNCH((k_flat_scores<128, true>), grid, dim3(256), 0, st, qI, kI, scores, s.L, s.nq, Lp, qtiles);
    else
      HSA_LAUNCH((k_flat_scores<128, false>), grid, dim3(256), 0, st, qI, kI, scores, s.L, s.nq, Lp, qtiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p += align_up((size_t)nq_total * Lp * sizeof(float));
  }
  uint2* lists[2] = {nullptr, nullptr};
  int* counts[2] = {nullptr, nullptr};
  if (flat_needs_lists(s)) {
    const size_t nl = (size_t)nq_total * nchunk;
    for (int i = 0; i < 2; ++i) {
      lists[i] = reinterpret_cast<uint2*>(p);
      p += align_up(nl * s.k * sizeof(uint2));
      counts[i] = reinterpret_cast<int*>(p);
      p += align_up(nl * sizeof(int));
    }
  }
  // staged final lists: k + 64 ints (k <= kFlatStageMax when a select runs)
  const size_t dyn = s.k < s.L ? sizeof(int) * ((size_t)s.k + kWave) : 0;
  if (flat_row_select(s)) {
    // one launch per row-length group: queries i with 512 R < t + 1 <= 1024 R
    const int base = s.L - s.nq;  // t = base + i
    for (int R = 1; R <= 64; R <<= 1) {
      const int i_lo = R == 1 ? 0 : std::max(0, 512 * R - base);
      const int i_hi = std::min(s.nq, 1024 * R - base);
      if (i_lo >= i_hi) continue;
      const dim3 grid(i_hi - i_lo, s.b);
      if (512 * R >= kFlatStreamMin) {  // rows of more than 16384 candidates
        HSA_LAUNCH(k_flat_stream_select, grid, dim3(256), 0, st, scores, tok, s.L, s.nq, Lp, s.k, i_lo);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        continue;
      }
#define HSA_FR(RR)                                                                                         \
  case RR:                                                                                                 \
    HSA_LAUNCH((k_flat_row_select<RR>), grid, dim3(1024), dyn, st, scores, tok, s.L, s.nq, Lp, s.k, i_lo); \
    break;
      switch (R) {
        HSA_FR(1) HSA_FR(2) HSA_FR(4) HSA_FR(8) HSA_FR(16)
      }
#undef HSA_FR
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  HSA_LAUNCH((k_flat_chunk_select<4, 32>), dim3(nq_total, s.k < s.L ? nchunk : 1), dim3(256), dyn, st,
                     scores, lists[0], counts[0], tok, s.L, s.nq, Lp, s.k, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !flat_needs_lists(s)) return e;
  // merge levels until one list per query remains
  const bool small = 4 * s.k <= kFlatMergeSmall;  // 4-wave merges only when a group holds 4+ lists
  const int G = (small ? kFlatMergeSmall : kFlatMergeLarge) / s.k;  // >= 2
  int n_lists = nchunk, level = 0, cur = 0;
  while (n_lists > 1) {
    const int groups = (n_lists + G - 1) / G;
    const int n_max = min(G, n_lists) * s.k;  // candidates of the fullest group
    dim3 grid(nq_total, groups);
    const uint2* lin = lists[cur];
    const int* cin = counts[cur];
    uint2* lout = lists[cur ^ 1];
    int* cout = counts[cur ^ 1];
    int r = 1;
    while (r * (small ? 256 : 1024) < n_max) r <<= 1;
#define HSA_MG(NW, RR) \
  case RR: launch_merge<NW, RR>(grid, dyn, lin, cin, lout, cout, tok, s, nchunk, G, level, st); break;
    if (small) {
      switch (r) {
        HSA_MG(4, 1) HSA_MG(4, 2) HSA_MG(4, 4) HSA_MG(4, 8) HSA_MG(4, 16) HSA_MG(4, 32)
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (r) {
        HSA_MG(16, 1) HSA_MG(16, 2) HSA_MG(16, 4) HSA_MG(16, 8) HSA_MG(16, 16) HSA_MG(16, 32)
        default: return hipErrorInvalidValue;
      }
    }
#undef HSA_MG
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    n_lists = groups;
    cur ^= 1;
    ++level;
  }
  return hipSuccess;
}

}  // namespace hsa
