// Step 3: token scores inside the kept blocks and the top-k token selection.
//
// HISA page (two-step method, step two): only the tokens of the m kept
// blocks are scored, with the original indexer rule, and the best k are
// kept.  Candidates are the tokens s <= t of the kept blocks.
//
// Candidate slots: slot p * B + r stands for token blk[p] * B + r.  Kept
// blocks other than the query's own block c are full and precede c, and c
// is the last valid list entry, so the valid slots are exactly the prefix
// [0, n_valid) with n_valid = (n_sel - 1) * B + (t - c * B + 1), and slot
// order is token order.  A list holds n_sel = min(c + 1, m) blocks when it
// comes from the two-level selection; the three-level one can keep fewer
// (its candidates are the blocks of the kept super-blocks), padded with -1.
// The scorers skip -1 entries and the select and the enumeration take n_sel
// from the list itself; min(c + 1, m) is only an upper bound.
//
// Kernel 1 (k_token_scores): one workgroup per (query, list entry) streams
// that block's kI rows (d_index/8 lanes per row, 16-byte loads) and writes
// the fp32 scores of its slots to the workspace.
// Kernel 2 (k_token_select): one workgroup per query; when n_valid <= k all
// candidates are written, otherwise the exact select of select.hpp runs over
// the slot scores.
// When no query can have more than k candidates (k >= m * B, or a context
// of at most k tokens), every list is its candidate enumeration and
// k_token_enum writes it alone: 4 slots per thread, one 16-byte store,
// workgroups spread over the list so that long lists of few queries do not
// wait on one workgroup's chain of block-list loads.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"
#include "token_select.hpp"

namespace hsa {

// Largest m with m * B <= 32768 candidates at the smallest block size.

// Workgroup (q, y) writes the 1024-slot chunks y, y + gridDim.y, ... of
// query q's list.  B >= 8, so 4 consecutive slots from a multiple of 4 lie
// in one block.
__global__ __launch_bounds__(256) void k_token_enum(const int32_t* __restrict__ blk, int32_t* __restrict__ tok,
                                                    int L, int nq, int B, int log2B, int m, int k,
                                                    const int32_t* __restrict__ lens) {
  const int q = blockIdx.x;
  const int t = query_pos(seq_len_of(lens, L, q / nq), nq, q % nq);
  int c, n_sel, n_valid;
  candidate_count(t, B, m, c, n_sel, n_valid);
  int32_t* out = tok + (size_t)q * k;
  for (long long s0l = ((long long)blockIdx.y * 256 + threadIdx.x) * 4; s0l < k; s0l += (long long)gridDim.y * 1024) {
    const int s0 = (int)s0l;
    // a slot is a token iff its list entry is a block and the token is causal
    // (only the last kept block, c, is cut by t); -1 entries and what follows
    // them come after every valid slot
    const int j = s0 < n_valid ? blk[(size_t)q * m + (s0 >> log2B)] : -1;
    int v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tk = (j << log2B) + ((s0 + e) & (B - 1));
      v[e] = (j >= 0 && s0 + e < n_valid && tk <= t) ? tk : -1;
    }
    if ((k & 3) == 0) {
      *reinterpret_cast<i32x4*>(out + s0) = i32x4{v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (s0 + e < k) out[s0 + e] = v[e];
    }
  }
}

template <int DI>
__global__ __launch_bounds__(256) void k_token_scores(const uint16_t* __restrict__ qI,
                                                      const uint16_t* __restrict__ kI,
                                                      const int32_t* __restrict__ blk, float* __restrict__ scores,
                                                      int L, int nq, int B, int m, int k,
                                                      const int32_t* __restrict__ lens) {
  constexpr int LPR = DI / 8;
  constexpr int RPI = 256 / LPR;  // rows per workgroup iteration
  constexpr int NIT = 128 / RPI;  // iterations for the largest block (B = 128)
  const int p = blockIdx.x;
  const int q = blockIdx.y;
  const int b = q / nq, i = q % nq;
  const int t = query_pos(seq_len_of(lens, L, b), nq, i);
  int c, n_sel, n_valid;
  candidate_count(t, B, m, c, n_sel, n_valid);
  if (n_valid <= k || p >= n_sel) return;
  const int j = blk[(size_t)q * m + p];
  if (j < 0) return;  // a shorter (three-level) list

  const int tid = threadIdx.x;
  const int col8 = tid % LPR;
  float qv[8];
  {
    const u32x4 v = *reinterpret_cast<const u32x4*>(qI + (size_t)q * DI + col8 * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(v[e]);
      qv[2 * e + 1] = bf16_hi(v[e]);
    }
  }
  const uint16_t* kb = kI + ((size_t)b * L + (size_t)j * B) * DI;
  float* out = scores + (size_t)q * m * B + (size_t)p * B;
  const int rows = min(B, t - j * B + 1);
  // every row load in flight at once, then the dot products
  u32x4 v[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (it * RPI < B) {
      const int r = min(it * RPI + tid / LPR, rows - 1);
      v[it] = *reinterpret_cast<const u32x4*>(kb + (size_t)r * DI + col8 * 8);
    }
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (it * RPI < B) {
      const int r = it * RPI + tid / LPR;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += qv[2 * e] * bf16_lo(v[it][e]);
        dot += qv[2 * e + 1] * bf16_hi(v[it][e]);
      }
      dot = group_sum_f<LPR>(dot);
      if (r < rows && col8 == 0) out[r] = dot;
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled scoring for prefill: one workgroup per tile of QT = 64 * QW
// consecutive queries of one sequence.  The tile's kept blocks are merged
// into a union (LDS bitmaps: one QT-bit mask of queries per block); every
// union block is then read once and scored against just the queries whose
// mask bit is set, 16 at a time, with v_mfma_f32_16x16x32_bf16
// (A = 16 kI rows of the block, B = the 16 queries' indexer vectors, so the
// accumulator holds 4 consecutive tokens of one query per lane and is
// stored with one 16-byte write).  kI traffic per tile is the union size
// times B rows instead of m blocks per query.
// ---------------------------------------------------------------------------

constexpr int kTiledWaves = 8;

// Exclusive scan of two counters over the threads of the workgroup.
__device__ __forceinline__ void wg_scan2(int a, int b, int* lds, int& a_ex, int& b_ex, int& a_tot, int& b_tot) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int ai = a, bi = b;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int va = __shfl_up(ai, o, kWave), vb = __shfl_up(bi, o, kWave);
    if (lane >= o) {
      ai += va;
      bi += vb;
    }
  }
  if (lane == kWave - 1) {
    lds[wave] = ai;
    lds[kTiledWaves + wave] = bi;
  }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < kTiledWaves; ++w) {
    const int xa = lds[w], xb = lds[kTiledWaves + w];
    if (w < wave) {
      pa += xa;
      pb += xb;
    }
    ta += xa;
    tb += xb;
  }
  a_ex = pa + ai - a;
  b_ex = pb + bi - b;
  a_tot = ta;
  b_tot = tb;
  __syncthreads();
}

struct TiledLayout {
  size_t bitmap, uidx, ulist, uoff, posbuf, qtile, scan, wscratch, total;
};

__host__ __device__ inline TiledLayout tiled_layout(int nJ, int QW, int m, int DI) {
  TiledLayout t;
  const int QT = 64 * QW;
  size_t o = 0;
  t.bitmap = o;
  o += (size_t)nJ * QW * 8;
  t.uidx = o;
  o += (size_t)nJ * 4;
  t.ulist = o;
  o += (size_t)nJ * 4;
  t.uoff = o;
  o += (size_t)(nJ + 1) * 4;
  t.posbuf = o;
  o += ((size_t)QT * m * 2 + 15) / 16 * 16;
  t.qtile = o;
  o += (size_t)QT * DI * 2;
  t.scan = o;
  o += 2 * kTiledWaves * 4 + 16;
  t.wscratch = o;  // per wave: query slot and list position of each mask rank
  o += (size_t)kTiledWaves * QT * 4;
  t.total = o;
  return t;
}

template <int DI, int QW, bool STREAM>
__global__ __launch_bounds__(kTiledWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_token_scores_tiled(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI, const int32_t* __restrict__ blk,
    float* __restrict__ scores, int L, int nq, int B, int m, int k, int tiles_per_seq, int n_tiles, int nJ_max,
    int parts) {
  constexpr int QT = 64 * QW;
  constexpr int KS = DI / 32;
  constexpr int NT = kTiledWaves * 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const TiledLayout lay = tiled_layout(nJ_max, QW, m, DI);
  uint64_t* bitmap = reinterpret_cast<uint64_t*>(smem + lay.bitmap);
  int* uidx = reinterpret_cast<int*>(smem + lay.uidx);
  int* ulist = reinterpret_cast<int*>(smem + lay.ulist);
  int* uoff = reinterpret_cast<int*>(smem + lay.uoff);
  uint16_t* posbuf = reinterpret_cast<uint16_t*>(smem + lay.posbuf);
  uint16_t* qtile = reinterpret_cast<uint16_t*>(smem + lay.qtile);
  int* scan = reinterpret_cast<int*>(smem + lay.scan);

  // `parts` workgroups share a tile, each scoring every parts-th union block
  // (the union grows with the tile's position; late tiles hold every block)
  const int tile = n_tiles - 1 - (int)blockIdx.x / parts;  // longest tiles first
  const int part = (int)blockIdx.x % parts;
  const int b = tile / tiles_per_seq;
  const int i0 = (tile % tiles_per_seq) * QT;
  const int nqt = min(nq - i0, QT);
  const int nJ = query_pos(L, nq, i0 + nqt - 1) / B + 1;
  const int tid = threadIdx.x;
  const size_t qrow0 = (size_t)b * nq + i0;

  for (int x = tid; x < nJ * QW; x += NT) bitmap[x] = 0ull;
  for (int x = tid; x < QT * (DI / 8); x += NT) {
    const int qq = x / (DI / 8), c8 = x % (DI / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qq < nqt) v = *reinterpret_cast<const u32x4*>(qI + (qrow0 + qq) * DI + c8 * 8);
    *reinterpret_cast<u32x4*>(qtile + qq * DI + c8 * 8) = v;
  }
  __syncthreads();

  // 1. bitmaps of (block -> queries of the tile that kept it and need scoring)
  for (int x = tid; x < nqt * m; x += NT) {
    const int qq = x / m, p = x % m;
    int c, n_sel, n_valid;
    candidate_count(query_pos(L, nq, i0 + qq), B, m, c, n_sel, n_valid);
    if (n_valid > k && p < n_sel) {
      const int j = blk[(qrow0 + qq) * m + p];
      if (j >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&bitmap[j * QW + qq / 64]), 1ull << (qq % 64));
    }
  }
  __syncthreads();

  // 2. union list in ascending block order, with each entry's offset into posbuf
  const int per = (nJ + NT - 1) / NT;
  const int j_lo = min(nJ, tid * per), j_hi = min(nJ, j_lo + per);
  int cu = 0, cp = 0;
  for (int j = j_lo; j < j_hi; ++j) {
    int pc = 0;
#pragma unroll
    for (int w = 0; w < QW; ++w) pc += __popcll(bitmap[j * QW + w]);
    cu += pc > 0;
    cp += pc;
  }
  int u_ex, p_ex, nU, n_pairs;
  wg_scan2(cu, cp, scan, u_ex, p_ex, nU, n_pairs);
  for (int j = j_lo; j < j_hi; ++j) {
    int pc = 0;
#pragma unroll
    for (int w = 0; w < QW; ++w) pc += __popcll(bitmap[j * QW + w]);
    if (pc > 0) {
      ulist[u_ex] = j;
      uoff[u_ex] = p_ex;
      uidx[j] = u_ex;
      ++u_ex;
      p_ex += pc;
    } else {
      uidx[j] = -1;
    }
  }
  __syncthreads();

  // 3. list position of every (query, kept block) pair, in mask-rank order
  for (int x = tid; x < nqt * m; x += NT) {
    const int qq = x / m, p = x % m;
    int c, n_sel, n_valid;
    candidate_count(query_pos(L, nq, i0 + qq), B, m, c, n_sel, n_valid);
    const int j = (n_valid > k && p < n_sel) ? blk[(qrow0 + qq) * m + p] : -1;
    if (j >= 0) {
      int rank = 0;
#pragma unroll
      for (int w = 0; w < QW; ++w) {
        const uint64_t word = bitmap[j * QW + w];
        if (w < qq / 64) rank += __popcll(word);
        else if (w == qq / 64) rank += __popcll(word & ((1ull << (qq % 64)) - 1ull));
      }
      posbuf[uoff[uidx[j]] + rank] = (uint16_t)p;
    }
  }
  __syncthreads();

  // 4. score every union block against the queries that kept it.  A wave
  // loads all of a block's kI rows at once (one memory latency per block),
  // then, per group of 16 queries, loads the group's indexer vectors from
  // LDS once and runs the block's m-tiles back to back.
  constexpr int kMaxMT = 8;  // B <= 128
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int slot = lane & 15;
  const int kgrp = lane >> 4;
  const size_t kseq = (size_t)b * L;
  uint16_t* sq = reinterpret_cast<uint16_t*>(smem + lay.wscratch) + (size_t)wave * 2 * QT;
  uint16_t* sp = sq + QT;
  const int n_mt = B / 16;
  for (int u = part * kTiledWaves + wave; u < nU; u += parts * kTiledWaves) {
    const int j = ulist[u];
    const int off = uoff[u];
    int pc = 0;
#pragma unroll
    for (int w = 0; w < QW; ++w) {
      const uint64_t word = bitmap[j * QW + w];
      if ((word >> lane) & 1ull) {
        const int rank = pc + (int)lanes_below(word);
        sq[rank] = (uint16_t)(w * 64 + lane);
        sp[rank] = posbuf[off + rank];
      }
      pc += __popcll(word);
    }
    const uint16_t* blk_rows = kI + (kseq + (size_t)j * B) * DI + 8 * kgrp;
    const int max_row = L - 1 - j * B;  // rows past the sequence end are clamped (their scores are unused)
    u32x4 a[kMaxMT][KS];
#pragma unroll
    for (int mt = 0; mt < kMaxMT; ++mt) {
      if (mt < n_mt) {
        const int r = min(16 * mt + slot, max_row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[mt][ks] = *reinterpret_cast<const u32x4*>(blk_rows + (size_t)r * DI + 32 * ks);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    for (int g = 0; g * 16 < pc; ++g) {
      const int rank = g * 16 + slot;
      const bool valid = rank < pc;
      const int qq = valid ? sq[rank] : 0;
      const int pos = valid ? sp[rank] : 0;
      bf16x8 bq[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(qtile + qq * DI + 8 * kgrp + 32 * ks);
        bq[ks] = __builtin_bit_cast(bf16x8, v);
      }
      const int t = query_pos(L, nq, i0 + qq);
      float* dst = scores + (qrow0 + qq) * (size_t)m * B + (size_t)pos * B + 4 * kgrp;
#pragma unroll
      for (int mt = 0; mt < kMaxMT; ++mt) {
        if (mt < n_mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt][ks]), bq[ks], acc, 0, 0, 0);
          // acc[e]: token j*B + 16 mt + 4 kgrp + e of query qq
          if (valid) {
            const int s0 = j * B + 16 * mt + 4 * kgrp;
            if (s0 + 3 <= t) {
              if constexpr (STREAM) __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(dst + 16 * mt));
              else *reinterpret_cast<f32x4*>(dst + 16 * mt) = acc;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (s0 + e <= t) dst[16 * mt + e] = acc[e];
            }
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------------------
// Block-major scoring (many queries per kept block, e.g. a chunk of new
// queries against a long context).  The kept (query, slot) pairs are
// inverted into one list per (sequence, block): counted with atomics,
// offsets by a one-workgroup scan, lists filled through per-block cursors
// (their order varies, but every score goes to its fixed slot, so results
// are deterministic).  Then each workgroup loads one block's kI rows and
// scores up to kBmChunk of its queries with MFMA, so each block's keys are
// read once per kBmChunk queries instead of once per query.
constexpr int kBmChunk = 64;

__device__ __forceinline__ bool bm_entry(const int32_t* __restrict__ blk, long long e, int L, int nq, int B, int m,
                                         int k, int nb, int& bj) {
  const int q = (int)(e / m), p = (int)(e % m);
  int c, n_sel, n_valid;
  candidate_count(query_pos(L, nq, q % nq), B, m, c, n_sel, n_valid);
  if (n_valid <= k || p >= n_sel) return false;
  const int j = blk[e];
  if (j < 0) return false;  // a shorter (three-level) list
  bj = (q / nq) * nb + j;
  return true;
}

__global__ __launch_bounds__(256) void k_bm_zero(int* __restrict__ counts, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) counts[i] = 0;
}

__global__ __launch_bounds__(256) void k_bm_count(const int32_t* __restrict__ blk, int* __restrict__ counts, int L,
                                                  int nq, int B, int m, int k, int nb, long long total) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    int bj;
    if (bm_entry(blk, e, L, nq, B, m, k, nb, bj)) atomicAdd(&counts[bj], 1);
  }
}

// One workgroup: offsets[i] = sum of counts before i, chunk_off[i] = sum of
// ceil(count / kBmChunk) before i (both with a final total), cursor = offsets.
__global__ __launch_bounds__(1024) void k_bm_scan(const int* __restrict__ counts, int* __restrict__ offsets,
                                                  int* __restrict__ chunk_off, int* __restrict__ cursor, int n) {
  __shared__ int s_cnt[16], s_chk[16];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int a = 0, ch = 0;
  for (int i = lo; i < hi; ++i) {
    a += counts[i];
    ch += (counts[i] + kBmChunk - 1) / kBmChunk;
  }
  const int ia = wave_incl_scan(a), ic = wave_incl_scan(ch);
  const int wave = tid / kWave;
  if (lane_id() == kWave - 1) {
    s_cnt[wave] = ia;
    s_chk[wave] = ic;
  }
  __syncthreads();
  int ba = 0, bc = 0;
  for (int w = 0; w < wave; ++w) {
    ba += s_cnt[w];
    bc += s_chk[w];
  }
  int ra = ba + ia - a, rc = bc + ic - ch;  // exclusive prefix at lo
  for (int i = lo; i < hi; ++i) {
    offsets[i] = ra;
    cursor[i] = ra;
    chunk_off[i] = rc;
    ra += counts[i];
    rc += (counts[i] + kBmChunk - 1) / kBmChunk;
  }
  if (tid == 1023) {
    offsets[n] = ra;
    chunk_off[n] = rc;
  }
}

__global__ __launch_bounds__(256) void k_bm_fill(const int32_t* __restrict__ blk, int* __restrict__ cursor,
                                                 int2* __restrict__ entries, int L, int nq, int B, int m, int k,
                                                 int nb, long long total) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    int bj;
    if (bm_entry(blk, e, L, nq, B, m, k, nb, bj))
      entries[atomicAdd(&cursor[bj], 1)] = make_int2((int)(e / m), (int)(e % m));
  }
}

// One workgroup = one chunk of up to kBmChunk entries of one (sequence,
// block) list; wave w takes entries 16w .. 16w+15.  S^T = kI_block qI^T per
// 16-token tile (A = 16 key rows, B = 16 queries): each lane holds 4
// consecutive tokens of one query and writes them with one 16-byte store to
// that query's slots p*B + r.  Rows past L are clamped (their slots lie past
// the query's candidates and are never read).
template <int DI>
__global__ __launch_bounds__(256) void k_bm_scores(const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI,
                                                   const int2* __restrict__ entries, const int* __restrict__ offsets,
                                                   const int* __restrict__ chunk_off, float* __restrict__ scores,
                                                   int L, int nq, int B, int m, int nb, int nlist) {
  constexpr int KS = DI / 32;
  const int wg = blockIdx.x;
  if (wg >= chunk_off[nlist]) return;
  int lo = 0, hi = nlist;  // the list whose chunk range holds wg
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= wg) lo = mid; else hi = mid;
  }
  const int bj = lo;
  const int e0 = offsets[bj] + (wg - chunk_off[bj]) * kBmChunk;
  const int e1 = min(e0 + kBmChunk, offsets[bj + 1]);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int jl = lane & 15, gq = lane >> 4;
  const int w0 = e0 + 16 * wave;
  if (w0 >= e1) return;
  const int b = bj / nb, j = bj % nb;
  const int2 ent = entries[min(w0 + jl, e1 - 1)];  // this lane's query and slot (column jl)
  const bool live = w0 + jl < e1;
  u32x4 qb[KS];
  {
    const uint16_t* src = qI + (size_t)ent.x * DI + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const u32x4*>(src + 32 * ks);
  }
  float* dst = scores + (size_t)ent.x * m * B + (size_t)ent.y * B + 4 * gq;
  const uint16_t* kb = kI + (size_t)b * L * DI;
  // two 16-row tiles at a time (B >= 16 here, a multiple of 16): their
  // accumulators advance together over ks, two independent MFMA chains
  for (int r0 = 0; r0 < B; r0 += 32) {
    const bool two = r0 + 16 < B;  // uniform
    u32x4 a[2][KS];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = min(j * B + r0 + 16 * h + jl, L - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a[h][ks] = *reinterpret_cast<const u32x4*>(kb + (size_t)row * DI + 8 * gq + 32 * ks);
    }
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[h][ks]),
                                                         __builtin_bit_cast(bf16x8, qb[ks]), acc[h], 0, 0, 0);
    if (live) {
      *reinterpret_cast<f32x4*>(dst + r0) = acc[0];
      if (two) *reinterpret_cast<f32x4*>(dst + r0 + 16) = acc[1];
    }
  }
}

// Dynamic LDS of the select: the query's block list (m entries, padded to a
// multiple of 4) and, when k <= kStageMax (STAGED), the output list plus one
// dummy slot per lane, so that the list leaves in coalesced 16-byte stores
// instead of one 4-byte store per kept token and emission needs no branch.
constexpr int kStageMax = 8192;
static inline size_t tsel_lds_bytes(int m, int k) {
  return sizeof(int) * ((size_t)((m + 3) & ~3) + (k <= kStageMax ? (size_t)k + kWave : 0));
}

// ONEBLK: R <= B (both powers of two), so a thread's R slots lie in one
// kept block and its tokens are one base plus the slot offset.
template <int NW, int R, bool STAGED, bool ONEBLK>
__global__ __launch_bounds__(NW * 64) void k_token_select(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ blk, int32_t* __restrict__ tok,
                                                          int L, int nq, int B, int log2B, int m, int k,
                                                          const int32_t* __restrict__ lens) {
  constexpr int NT = NW * 64;
  __shared__ SelectSmem<NW> lds;
  extern __shared__ int dyn_lds[];
  int* bl = dyn_lds;
  int* stage = dyn_lds + ((m + 3) & ~3);
  const int q = blockIdx.x;
  int32_t* out = tok + (size_t)q * k;
  const int dummy = k + lane_id();
  const bool selected = select_query_tokens<NW, R, ONEBLK, STAGED>(
      scores, blk, q, L, nq, B, log2B, m, k, lens, 0, k, lds, bl, [&](int slot, int v) { out[slot] = v; },
      [&](int pos, int v, bool take) {
        if constexpr (STAGED) stage[take ? pos : dummy] = v;
        else if (take) out[pos] = v;
      });
  if constexpr (STAGED) {
    if (!selected) return;
    // select_top ends with a barrier: the staged list is complete
    if ((k & 3) == 0) {
      for (int p = threadIdx.x * 4; p < k; p += NT * 4)
        *reinterpret_cast<u32x4*>(out + p) = *reinterpret_cast<const u32x4*>(stage + p);
    } else {
      for (int p = threadIdx.x; p < k; p += NT) out[p] = stage[p];
    }
  }
}

// Workspace: the slot-ordered scores, then (block-major scoring) the list
// counts, offsets, chunk offsets, cursors and the (query, slot) entries.
struct BmLayout {
  size_t counts, offsets, chunk_off, cursor, entries, total;
};
static BmLayout bm_layout(const Dims& s, size_t base) {
  const size_t nl = (size_t)s.b * s.nb;
  BmLayout t;
  size_t o = base;
  t.counts = o;
  o += align_up(nl * 4);
  t.offsets = o;
  o += align_up((nl + 1) * 4);
  t.chunk_off = o;
  o += align_up((nl + 1) * 4);
  t.cursor = o;
  o += align_up(nl * 4);
  t.entries = o;
  o += align_up((size_t)s.b * s.nq * s.m * sizeof(int2));
  t.total = o;
  return t;
}

static int tiled_qw(const Dims& s);

// Block-major scoring pays off when a query tile of the tiled scorer would
// keep each block only a few times (a chunk of queries against a long
// context: 64 queries x 128 kept blocks out of 4096), so that every block's
// keys would be streamed for very few queries; when tiles amortise well
// (prefill, where consecutive queries keep 32 of a tile's blocks on average)
// the tiled scorer stays.  Decode keeps the per-query scorer.
static bool use_block_major(const Dims& s) {
  if (s.B < 16 || s.nq < 64 || (long long)s.b * s.nq * s.m >= (1ll << 30) || (long long)s.b * s.nb >= (1ll << 24))
    return false;
  const int qw = tiled_qw(s);
  return qw == 0 || 64ll * qw * s.m < 8ll * s.nb;
}

size_t token_topk_ws_bytes(const Dims& s) {
  if ((long long)s.k >= (long long)s.m * s.B) return 0;
  const size_t scores = align_up((size_t)s.b * s.nq * s.m * s.B * sizeof(float));
  return use_block_major(s) ? bm_layout(s, scores).total : scores;
}

template <int NW, int R, bool STAGED, bool ONEBLK>
static void launch_tsel_k(const Dims& s, size_t dyn, int log2B, const float* sc, const int32_t* blk, int32_t* tok,
                          hipStream_t st) {
  HSA_LAUNCH((k_token_select<NW, R, STAGED, ONEBLK>), dim3(s.b * s.nq), dim3(NW * 64), dyn, st, sc, blk, tok,
                     s.L, s.nq, s.B, log2B, s.m, s.k, s.lens);
}

// Variants: a thread's slots span several blocks only when R > B (R > 8,
// since B >= 8); the list exceeds the staging limit only when the group
// can hold more than kStageMax candidates.
template <int NW, int R>
static hipError_t launch_tsel_r(bool scoring, const Dims& s, const float* sc, const int32_t* blk, int32_t* tok,
                                hipStream_t st) {
  const int log2B = __builtin_ctz((unsigned)s.B);  // B is a power of two
  const bool staged = s.k <= kStageMax;
  const bool oneblk = R <= s.B;
  // without scoring every query takes the keep-all path, which uses no LDS;
  // with scoring m * B <= 32768 (checked at the API), so m <= 4096
  const size_t dyn = scoring ? tsel_lds_bytes(s.m, s.k) : 0;
  constexpr bool kMulti = R > 8;
  constexpr bool kLong = NW * 64 * R > kStageMax;
  if constexpr (NW == 16) {
    // few queries, latency-bound: kept entries go straight to memory, so the
    // select needs no closing barrier and no staged copy
    if (scoring && oneblk) {
      launch_tsel_k<16, R, false, true>(s, dyn, log2B, sc, blk, tok, st);
      return hipGetLastError();
    }
  }
  if (!scoring || (staged && oneblk)) {
    // (without scoring the variant does not matter: the keep-all path)
    launch_tsel_k<NW, R, true, true>(s, dyn, log2B, sc, blk, tok, st);
  } else if (staged) {
    if constexpr (kMulti) launch_tsel_k<NW, R, true, false>(s, dyn, log2B, sc, blk, tok, st);
    else return hipErrorInvalidValue;
  } else if (oneblk) {
    if constexpr (kLong) launch_tsel_k<NW, R, false, true>(s, dyn, log2B, sc, blk, tok, st);
    else return hipErrorInvalidValue;
  } else {
    if constexpr (kLong && kMulti) launch_tsel_k<NW, R, false, false>(s, dyn, log2B, sc, blk, tok, st);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_tsel(int R, bool scoring, const Dims& s, const float* sc, const int32_t* blk, int32_t* tok,
                              hipStream_t st) {
  switch (R) {
    case 1: return launch_tsel_r<NW, 1>(scoring, s, sc, blk, tok, st);
    case 2: return launch_tsel_r<NW, 2>(scoring, s, sc, blk, tok, st);
    case 4: return launch_tsel_r<NW, 4>(scoring, s, sc, blk, tok, st);
    case 8: return launch_tsel_r<NW, 8>(scoring, s, sc, blk, tok, st);
    case 16: return launch_tsel_r<NW, 16>(scoring, s, sc, blk, tok, st);
    case 32: return launch_tsel_r<NW, 32>(scoring, s, sc, blk, tok, st);
    case 64:
      if constexpr (NW <= 4) return launch_tsel_r<NW, 64>(scoring, s, sc, blk, tok, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

constexpr size_t kMaxLds = 160 * 1024;

// Queries per tile of the tiled scorer (64 * QW), or 0 when the per-query
// scorer is used (few queries per sequence, small blocks, or no LDS room).
static int tiled_qw(const Dims& s) {
  if (s.B < 16 || s.nq < 64) return 0;
  for (int qw = 4; qw >= 1; qw >>= 1) {
    if (qw > 1 && s.nq < 64 * qw) continue;
    if (tiled_layout(s.nb, qw, s.m, s.dI).total <= kMaxLds) return qw;
  }
  return 0;
}

template <int DI, int QW, bool NT>
static hipError_t launch_tiled_nt(const Dims& s, const uint16_t* qI, const uint16_t* kI, const int32_t* blk,
                                  float* scores, hipStream_t st) {
  const int QT = 64 * QW;
  const int tiles_per_seq = (s.nq + QT - 1) / QT;
  const int n_tiles = tiles_per_seq * s.b;
  const size_t lds = tiled_layout(s.nb, QW, s.m, DI).total;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_token_scores_tiled<DI, QW, NT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  if (e != hipSuccess) return e;
  // about two workgroups per CU in total, at most 4 per tile
  const int parts = std::max(1, std::min(4, (512 + n_tiles - 1) / n_tiles));
  HSA_LAUNCH((k_token_scores_tiled<DI, QW, NT>), dim3(n_tiles * parts), dim3(kTiledWaves * 64), lds, st, qI, kI,
                     blk, scores, s.L, s.nq, s.B, s.m, s.k, tiles_per_seq, n_tiles, s.nb, parts);
  return hipGetLastError();
}

template <int DI, int QW>
static hipError_t launch_tiled_t(const Dims& s, const uint16_t* qI, const uint16_t* kI, const int32_t* blk,
                                 float* scores, hipStream_t st) {
  if ((size_t)s.b * s.nq * s.m * s.B * sizeof(float) > kStreamStoreBytes)
    return launch_tiled_nt<DI, QW, true>(s, qI, kI, blk, scores, st);
  return launch_tiled_nt<DI, QW, false>(s, qI, kI, blk, scores, st);
}

static hipError_t launch_tiled(const Dims& s, int qw, const uint16_t* qI, const uint16_t* kI, const int32_t* blk,
                               float* scores, hipStream_t st) {
  if (s.dI == 64) {
    if (qw == 4) return launch_tiled_t<64, 4>(s, qI, kI, blk, scores, st);
    if (qw == 2) return launch_tiled_t<64, 2>(s, qI, kI, blk, scores, st);
    return launch_tiled_t<64, 1>(s, qI, kI, blk, scores, st);
  }
  if (qw == 4) return launch_tiled_t<128, 4>(s, qI, kI, blk, scores, st);
  if (qw == 2) return launch_tiled_t<128, 2>(s, qI, kI, blk, scores, st);
  return launch_tiled_t<128, 1>(s, qI, kI, blk, scores, st);
}

hipError_t launch_token_scores(const Dims& s, const uint16_t* qI, const uint16_t* kI, const int32_t* blk,
                               void* ws, hipStream_t st) {
  const int nq_total = s.b * s.nq;
  if (nq_total == 0 || !((long long)s.k < (long long)s.m * s.B && s.L > s.k)) return hipSuccess;
  float* scores = static_cast<float*>(ws);
  const int qw = tiled_qw(s);
  if (use_block_major(s)) {
    unsigned char* base = static_cast<unsigned char*>(ws);
    const BmLayout lay = bm_layout(s, align_up((size_t)nq_total * s.m * s.B * sizeof(float)));
    int* counts = reinterpret_cast<int*>(base + lay.counts);
    int* offsets = reinterpret_cast<int*>(base + lay.offsets);
    int* chunk_off = reinterpret_cast<int*>(base + lay.chunk_off);
    int* cursor = reinterpret_cast<int*>(base + lay.cursor);
    int2* entries = reinterpret_cast<int2*>(base + lay.entries);
    const int nl = s.b * s.nb;
    const long long total = (long long)nq_total * s.m;
    const int g1 = (int)std::min<long long>((total + 255) / 256, 8192);
    HSA_LAUNCH(k_bm_zero, dim3(std::min((nl + 255) / 256, 1024)), dim3(256), 0, st, counts, nl);
    HSA_LAUNCH(k_bm_count, dim3(g1), dim3(256), 0, st, blk, counts, s.L, s.nq, s.B, s.m, s.k, s.nb, total);
    HSA_LAUNCH(k_bm_scan, dim3(1), dim3(1024), 0, st, counts, offsets, chunk_off, cursor, nl);
    HSA_LAUNCH(k_bm_fill, dim3(g1), dim3(256), 0, st, blk, cursor, entries, s.L, s.nq, s.B, s.m, s.k, s.nb,
                       total);
    const int gs = (int)((total + kBmChunk - 1) / kBmChunk + nl);
    if (s.dI == 64)
      HSA_LAUNCH((k_bm_scores<64>), dim3(gs), dim3(256), 0, st, qI, kI, entries, offsets, chunk_off, scores,
                         s.L, s.nq, s.B, s.m, s.nb, nl);
    else
      HSA_LAUNCH((k_bm_scores<128>), dim3(gs), dim3(256), 0, st, qI, kI, entries, offsets, chunk_off,
                         scores, s.L, s.nq, s.B, s.m, s.nb, nl);
    return hipGetLastError();
  }
  if (qw > 0) return launch_tiled(s, qw, qI, kI, blk, scores, st);
  dim3 grid(s.m, nq_total);
  if (s.dI == 64)
    HSA_LAUNCH((k_token_scores<64>), grid, dim3(256), 0, st, qI, kI, blk, scores, s.L, s.nq, s.B, s.m, s.k,
                       s.lens);
  else
    HSA_LAUNCH((k_token_scores<128>), grid, dim3(256), 0, st, qI, kI, blk, scores, s.L, s.nq, s.B, s.m, s.k,
                       s.lens);
  return hipGetLastError();
}

hipError_t launch_token_topk(const Dims& s, const uint16_t* qI, const uint16_t* kI, const int32_t* blk, int32_t* tok,
                             void* ws, hipStream_t st) {
  const int nq_total = s.b * s.nq;
  if (nq_total == 0) return hipSuccess;
  float* scores = static_cast<float*>(ws);
  const bool any_scoring = (long long)s.k < (long long)s.m * s.B && s.L > s.k;
  int n_max = s.m * s.B;
  if (any_scoring) {
    const hipError_t e = launch_token_scores(s, qI, kI, blk, ws, st);
    if (e != hipSuccess) return e;
  } else {  // every query keeps all of its candidates
    const dim3 grid((unsigned)nq_total, (unsigned)std::min<long long>((s.k + 1023ll) / 1024, 4096));
    HSA_LAUNCH(k_token_enum, grid, dim3(256), 0, st, blk, tok, s.L, s.nq, s.B, __builtin_ctz((unsigned)s.B), s.m,
               s.k, s.lens);
    return hipGetLastError();
  }
  if (nq_total >= 512 && n_max <= 4 * 64 * 64) {  // many queries: a 4-wave workgroup per query
    int r = 1;
    while (r * 256 < n_max) r <<= 1;
    return launch_tsel<4>(r, any_scoring, s, scores, blk, tok, st);
  }
  int r = 1;
  while (r * 1024 < n_max) r <<= 1;
  if (r > 32) return hipErrorInvalidValue;
  return launch_tsel<16>(r, any_scoring, s, scores, blk, tok, st);
}

}  // namespace hsa
