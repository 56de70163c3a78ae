// Step 2: block scores and the top-m block selection.
//
// HISA page (two-step method, step one): the block summaries are scored with
// the indexer's own rule (dot product with the query's indexer vector) and
// the best m blocks are kept; the first block and the last block (the one
// holding the query) are always kept.  HiLS page (section 2.2): a chunk's
// coarse score comes from its landmark vectors; here the maximum over them.
//
// Kernel 1 (k_block_scores_mfma for >= 64 queries per sequence, else the
// GEMV k_block_scores): score_j = max_l qI . S[j, l] for the causal
// blocks 1..c-1 of every query that needs scoring (c + 1 > m), written as
// fp32 to the workspace.  Each wave streams summary rows with 16-byte loads
// (d_index/8 lanes per row), multiplies by the query chunk it holds in
// registers and reduces across the row's lanes with xor shuffles.
// Kernel 2 (k_block_select): one workgroup per query runs the exact
// register-resident select of select.hpp over those scores.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"
#include "summary.hpp"
#include "token_select.hpp"

namespace hsa {

constexpr int kScoreBlocksPerWG = 64;

// GEMV block scores for few queries per sequence (decode).  Each workgroup
// takes 64 blocks of one query; its 4 waves issue every summary-row load
// first (16-byte loads, d_index/8 lanes per row) and then reduce.  With
// blockIdx.z == 1 the workgroup instead summarises block sum_start +
// blockIdx.x of sequence blockIdx.y: the host folds the newest blocks'
// summaries in here only when no query scores them (they are its own,
// always-kept block), which saves a dependent launch per decode step.
template <int DI, int NL>
__global__ __launch_bounds__(256) void k_block_scores(const uint16_t* __restrict__ qI,
                                                      const uint16_t* __restrict__ S, float* __restrict__ scores,
                                                      int L, int nq, int B, int nb, int m,
                                                      const uint16_t* __restrict__ kI, const int8_t* __restrict__ W,
                                                      uint16_t* __restrict__ S_out, int sum_start, int batch,
                                                      const int32_t* __restrict__ lens) {
  constexpr int LPR = DI / 8;     // lanes per summary row
  constexpr int RPL = kWave / LPR;  // rows per wave load
  constexpr int ITER = kScoreBlocksPerWG * NL / (4 * RPL);
  static_assert(RPL % NL == 0, "a block's landmarks must share one wave load");

  if (blockIdx.z == 1) {
    __shared__ float red[NL][256 / LPR][DI];
    if ((int)blockIdx.y >= batch) return;  // uniform
    const int Lb = seq_len_of(lens, L, blockIdx.y);
    // per-sequence lengths (n_q == 1): the block of the sequence's query
    const int jb = (lens ? (Lb - 1) / B : sum_start) + (int)blockIdx.x;
    if (jb >= nb || jb * B >= Lb) return;  // uniform
    summarise_block<DI, NL>(kI, W, S_out, L, Lb, B, nb, jb, blockIdx.y, red);
    return;
  }
  const int q = blockIdx.y;  // b * nq + i
  if (q >= batch * nq) return;
  const int b = q / nq, i = q % nq;
  const int t = query_pos(seq_len_of(lens, L, b), nq, i);
  const int c = t / B;
  if (c + 1 <= m) return;
  const int j0 = max(1, (int)blockIdx.x * kScoreBlocksPerWG);
  const int j1 = min(c, (int)(blockIdx.x + 1) * kScoreBlocksPerWG);  // exclusive
  if (j0 >= j1) return;

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col8 = lane % LPR;
  float qv[8];
  {
    const u32x4 v = *reinterpret_cast<const u32x4*>(qI + (size_t)q * DI + col8 * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(v[e]);
      qv[2 * e + 1] = bf16_hi(v[e]);
    }
  }
  const uint16_t* Sb = S + (size_t)b * nb * NL * DI;
  const int row_begin = j0 * NL + wave * RPL + lane / LPR;
  const int row_end = j1 * NL;
  u32x4 v[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int row = min(row_begin + it * 4 * RPL, row_end - 1);
    v[it] = *reinterpret_cast<const u32x4*>(Sb + (size_t)row * DI + col8 * 8);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int row = row_begin + it * 4 * RPL;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot += qv[2 * e] * bf16_lo(v[it][e]);
      dot += qv[2 * e + 1] * bf16_hi(v[it][e]);
    }
    dot = group_sum_f<LPR>(dot);
    if constexpr (NL > 1) dot = group_max_f<LPR * NL>(dot);  // a block's landmark rows are adjacent
    if (row < row_end && (lane % (LPR * NL)) == 0) scores[(size_t)q * nb + row / NL] = dot;
  }
}

// MFMA block scores for many queries: one workgroup scores 64 consecutive
// queries of one sequence against 128 summary rows (128 / NL blocks); wave w
// takes rows 32w .. 32w+31 for all 64 queries.  C = qI S^T with
// v_mfma_f32_16x16x32_bf16: A = 16 queries' indexer vectors, B = 16 summary
// rows; the accumulator holds 4 queries x 1 row per lane, the max over a
// block's NL landmark rows is an xor shuffle across adjacent lanes.  Tiles
// above the causal diagonal are skipped and only the scores the select reads
// (blocks 1 .. c-1 of queries with c + 1 > m) are written.
template <int DI, int NL>
__global__ __launch_bounds__(256) void k_block_scores_mfma(const uint16_t* __restrict__ qI,
                                                           const uint16_t* __restrict__ S,
                                                           float* __restrict__ scores, int L, int nq, int B,
                                                           int nb, int m, int qtiles_per_seq) {
  constexpr int KS = DI / 32;
  const int b = blockIdx.y / qtiles_per_seq;
  const int i0 = (blockIdx.y % qtiles_per_seq) * 64;
  const int i_last = min(nq, i0 + 64) - 1;
  const int c_last = query_pos(L, nq, i_last) / B;
  if (c_last + 1 <= m) return;  // no query of the tile needs scores
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int jl = lane & 15, gq = lane >> 4;
  const int row0 = blockIdx.x * 128 + wave * 32;  // first summary row of this wave
  if (row0 / NL >= c_last) return;                // every block is non-causal or forced
  const int nrows = nb * NL;

  // B operands: 2 tiles of 16 summary rows
  u32x4 bs[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = min(row0 + 16 * nt + jl, nrows - 1);
    const uint16_t* src = S + ((size_t)b * nrows + row) * DI + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bs[nt][ks] = *reinterpret_cast<const u32x4*>(src + 32 * ks);
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    // A operand: 16 queries
    const int qa = min(i0 + 16 * mt + jl, nq - 1);
    const uint16_t* qsrc = qI + ((size_t)b * nq + qa) * DI + 8 * gq;
    u32x4 a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = *reinterpret_cast<const u32x4*>(qsrc + 32 * ks);
    // both row tiles' accumulators advance together over ks (two
    // independent MFMA chains in flight)
    f32x4 accs[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        accs[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[ks]),
                                                           __builtin_bit_cast(bf16x8, bs[nt][ks]), accs[nt], 0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = accs[nt];
      // lane: queries 16mt + 4gq + e, summary row row0 + 16nt + jl
      if constexpr (NL > 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = group_max_f<NL>(acc[e]);
      }
      const int row = row0 + 16 * nt + jl;
      const int j = row / NL;
      if (row % NL == 0 && row < nrows) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + 16 * mt + 4 * gq + e;
          if (i >= nq) continue;
          const int c = query_pos(L, nq, i) / B;
          if (c + 1 > m && j >= 1 && j < c) scores[((size_t)b * nq + i) * nb + j] = acc[e];
        }
      }
    }
  }
}

// Prefill block top-m in one launch (contexts of at most kTileMaxBlocks
// blocks): one workgroup takes kTileQ (16, or 8 when that leaves too few
// workgroups to fill the chip) consecutive queries of one sequence and
// computes their block scores on the matrix cores straight into LDS (A =
// the queries' indexer vectors, held in registers (16 rows, the last query
// repeated past kTileQ); wave w takes summary
// rows 32w .. 32w+31 of every 128-row tile up to the last query's causal
// block, two MFMA chains at a time; the landmark maximum is an xor shuffle
// across adjacent lanes).  Each wave then runs the one-wave select for a
// quarter of the queries on their LDS rows, so the scores never leave the
// chip.  Row
// slot j of a query holds block j; only blocks 1 .. c-1 are candidates.
constexpr int kTileMaxBlocks = 2048;

template <int DI, int NL, int R, int kTileQ>
__global__ __launch_bounds__(256) void k_block_topm_tile(const uint16_t* __restrict__ qI,
                                                         const uint16_t* __restrict__ S, int32_t* __restrict__ blk,
                                                         int L, int nq, int B, int nb, int m, int qtiles_per_seq,
                                                         int ldsw) {
  constexpr int KS = DI / 32;
  extern __shared__ __attribute__((aligned(16))) float sc[];  // [kTileQ][ldsw]
  __shared__ SelectSmem<1> sms[4];
  const int b = blockIdx.x / qtiles_per_seq;
  const int i0 = (blockIdx.x % qtiles_per_seq) * kTileQ;
  const int nqt = min(kTileQ, nq - i0);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int jl = lane & 15, gq = lane >> 4;
  const int c_last = query_pos(L, nq, i0 + nqt - 1) / B;
  const int nrows = nb * NL;
  if (c_last + 1 > m) {  // (uniform) some query of the tile scores blocks
    u32x4 a[KS];
    {
      const uint16_t* qsrc = qI + ((size_t)b * nq + i0 + min(jl, nqt - 1)) * DI + 8 * gq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ks] = *reinterpret_cast<const u32x4*>(qsrc + 32 * ks);
    }
    const int row_end = c_last * NL;  // rows of blocks 0 .. c_last - 1
    for (int r0 = 32 * wave; r0 < row_end; r0 += 128) {
      u32x4 bs[2][KS];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = min(r0 + 16 * nt + jl, nrows - 1);
        const uint16_t* src = S + ((size_t)b * nrows + row) * DI + 8 * gq;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bs[nt][ks] = *reinterpret_cast<const u32x4*>(src + 32 * ks);
      }
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[ks]),
                                                            __builtin_bit_cast(bf16x8, bs[nt][ks]), acc[nt], 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // lane: queries 4gq + e, summary row r0 + 16nt + jl
        if constexpr (NL > 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[nt][e] = group_max_f<NL>(acc[nt][e]);
        }
        const int row = r0 + 16 * nt + jl;
        if (row % NL == 0 && row < row_end) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * gq + e < kTileQ) sc[(4 * gq + e) * ldsw + row / NL] = acc[nt][e];
        }
      }
    }
  }
  __syncthreads();
  for (int qq = wave; qq < nqt; qq += 4) {
    const int i = i0 + qq;
    const int c = query_pos(L, nq, i) / B;
    int32_t* out = blk + ((size_t)b * nq + i) * m;
    if (c + 1 <= m) {
      for (int j = lane; j < m; j += kWave) out[j] = j <= c ? j : -1;
      continue;
    }
    const int want = m - 2;
    const int n = c - 1;  // candidates: blocks 1 .. c-1, in slots 1 .. c-1
    if (lane == 0) {
      out[0] = 0;
      out[m - 1] = c;
    }
    if (want == 0) continue;
    const float empty = __uint_as_float(0x7FC00000u);
    const float* row = sc + qq * ldsw;
    float v[R];
#pragma unroll
    for (int r = 0; r < R; r += (R >= 4 ? 4 : 1)) {
      const int j0 = lane * R + r;
      if constexpr (R >= 4) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (j0 < ldsw) x = *reinterpret_cast<const f32x4*>(row + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[r + e] = (j0 + e >= 1 && j0 + e <= n) ? x[e] : empty;
      } else {
        v[r] = (j0 >= 1 && j0 <= n) ? row[j0] : empty;
      }
    }
    select_top_f<1, R, false>(v, want, kWave * R - n, sms[wave], [&](int pos, int idx, bool take) {
      if (take) out[1 + pos] = idx;
    });
  }
}

// Score-only build of the block-score contraction (a measurement aid: the
// scores of k_block_scores_mfma without the selection), tiled for the
// matrix cores.  One workgroup of 8 waves takes 256 consecutive queries:
// waves w and w + 4 hold queries 64 (w % 4) .. 64 (w % 4) + 63 as MFMA A
// operands in registers and share the 16-row groups of every 128-row
// summary tile between them (even groups to w, odd groups to w + 4), so
// two waves per SIMD keep the matrix cores fed.  Each tile is loaded once
// per workgroup into LDS (padded rows, double-buffered: the next tile's
// rows are in flight in registers while the current one is multiplied) and
// read by all eight waves as B operands, so every summary row fetched from
// L2 feeds 256 queries.  Instead of writing every score it keeps, per
// query, the maximum over the scored blocks 1 .. c-1 (all landmark rows of
// a block count, so the landmark maximum is part of it), reduced over lanes
// and over the wave pair on chip: one float per (query, chunk) leaves the
// chip.  -inf marks a query with no scored block in the chunk.  A row group
// that every query of the wave scores in full takes the maximum without
// per-element bounds; groups past every query's causal rows are skipped.
constexpr int kMaxQT = 256;   // queries per workgroup
constexpr int kMaxRT = 128;   // summary rows per tile
constexpr int kMaxWaves = 8;  // waves per workgroup

template <int DI>
__global__ __launch_bounds__(kMaxWaves * 64) void k_block_scores_max(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ S, float* __restrict__ out, int L, int nq,
    int log2B, int nb, int NL, int m, int qtiles_per_seq, int tiles_per_chunk, int nchunks) {
  constexpr int KS = DI / 32;
  constexpr int NT = kMaxWaves * 64;
  constexpr int LPR = DI / 8;              // 16-byte lanes per summary row
  constexpr int RPP = NT / LPR;            // rows per load pass of the workgroup
  constexpr int NP = kMaxRT / RPP;         // load passes per tile
  constexpr int PITCH = DI + 8;            // LDS row pitch (bf16): 16-byte reads conflict-free
  __shared__ __attribute__((aligned(16))) uint16_t bt[2][kMaxRT * PITCH];
  __shared__ float pair_mx[4][64];
  const int b = blockIdx.y / qtiles_per_seq;
  // the latest query tiles (the most causal tiles) are dispatched first
  const int i0 = (qtiles_per_seq - 1 - (int)(blockIdx.y % qtiles_per_seq)) * kMaxQT;
  const int chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int qgrp = wave & 3, half = wave >> 2;  // query group, row-group parity
  const int lane = lane_id();
  const int jl = lane & 15, gq = lane >> 4;
  const int nrows = nb * NL;
  const int i_last = min(nq, i0 + kMaxQT) - 1;
  const int c_last = query_pos(L, nq, i_last) >> log2B;
  // rows any query of the tile scores: blocks 1 .. c_last - 1
  const int tile_lo = chunk * tiles_per_chunk;
  const int tile_hi = min((c_last * NL + kMaxRT - 1) / kMaxRT, (chunk + 1) * tiles_per_chunk);  // exclusive
  // scored rows of query i: NL <= row < hi(i) (none when c + 1 <= m)
  auto rows_hi = [&](int i) {
    const int c = query_pos(L, nq, i) >> log2B;
    return c + 1 > m ? c * NL : 0;
  };
  // the lane's accumulator entries hold queries qw + 16 mt + 4 gq + e
  const int qw = i0 + 64 * qgrp;
  const bool wave_live = qw < nq;  // uniform over the wave
  const int hi_first = wave_live ? rows_hi(qw) : 0;                 // every live query scores rows below this
  const int hi_last = wave_live ? rows_hi(min(nq, qw + 64) - 1) : 0;  // no query scores rows from here on

  float mx[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx[mt][e] = -INFINITY;

  if (c_last + 1 > m && tile_lo < tile_hi) {  // uniform over the workgroup
    u32x4 a[4][KS];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int qa = min(qw + 16 * mt + jl, nq - 1);
      const uint16_t* qsrc = qI + ((size_t)b * nq + qa) * DI + 8 * gq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[mt][ks] = *reinterpret_cast<const u32x4*>(qsrc + 32 * ks);
    }
    const uint16_t* Sb = S + (size_t)b * nrows * DI;
    const int lr = tid / LPR, lc = 8 * (tid % LPR);  // this thread's row in a pass, first column
    u32x4 st[NP];
    auto load_tile = [&](int tile) {  // global -> registers
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int row = min(tile * kMaxRT + p * RPP + lr, nrows - 1);
        st[p] = *reinterpret_cast<const u32x4*>(Sb + (size_t)row * DI + lc);
      }
    };
    auto stage_tile = [&](int buf) {  // registers -> LDS
#pragma unroll
      for (int p = 0; p < NP; ++p)
        *reinterpret_cast<u32x4*>(&bt[buf][(p * RPP + lr) * PITCH + lc]) = st[p];
    };
    load_tile(tile_lo);
    stage_tile(0);
    __syncthreads();
    int buf = 0;
    for (int tile = tile_lo; tile < tile_hi; ++tile) {
      const bool more = tile + 1 < tile_hi;  // uniform
      if (more) load_tile(tile + 1);
      const uint16_t* bb = bt[buf];
#pragma unroll
      for (int g = 0; g < kMaxRT / 32; ++g) {
        const int nt = 2 * g + half;
        const int row0 = tile * kMaxRT + 16 * nt;  // the group's first row (uniform)
        if (row0 >= hi_last) break;                 // no query of the wave scores these rows or later ones
        u32x4 bs[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          bs[ks] = *reinterpret_cast<const u32x4*>(bb + (16 * nt + jl) * PITCH + 8 * gq + 32 * ks);
        // the 4 query tiles' accumulators advance together over ks: four
        // independent MFMA chains in flight instead of one at a time
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt][ks]),
                                                              __builtin_bit_cast(bf16x8, bs[ks]), acc[mt], 0, 0, 0);
        if (row0 >= NL && row0 + 16 <= hi_first) {  // every query of the wave scores all 16 rows
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx[mt][e] = fmaxf(mx[mt][e], acc[mt][e]);
        } else {
          const int row = row0 + jl;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = qw + 16 * mt + 4 * gq + e;
              if (row >= NL && row < rows_hi(i)) mx[mt][e] = fmaxf(mx[mt][e], acc[mt][e]);
            }
        }
      }
      if (more) {
        stage_tile(buf ^ 1);  // the other buffer: last read two tiles ago, before the barrier below
        __syncthreads();
        buf ^= 1;
      }
    }
  }
  // max over the 16 rows (lanes jl) of each accumulator entry, then over
  // the wave pair: the odd-group wave hands its maxima to the even one
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx[mt][e] = group_max_f<16>(mx[mt][e]);
  if (half == 1 && jl == 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) pair_mx[qgrp][16 * mt + 4 * gq + e] = mx[mt][e];
  }
  __syncthreads();
  if (half == 0 && jl == 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mt + 4 * gq + e;
        const int i = qw + r;
        if (i < nq) out[((size_t)b * nq + i) * nchunks + chunk] = fmaxf(mx[mt][e], pair_mx[qgrp][r]);
      }
  }
}

// The per-chunk maxima of k_block_scores_max reduced to one per query.
__global__ __launch_bounds__(256) void k_block_max_reduce(const float* __restrict__ part, float* __restrict__ out,
                                                          int nq_total, int nchunks) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= nq_total) return;
  float v = -INFINITY;
  for (int c = 0; c < nchunks; ++c) v = fmaxf(v, part[(size_t)q * nchunks + c]);
  out[q] = v;
}

template <int NW, int R>
__global__ __launch_bounds__(NW == 1 ? 256 : NW * 64) void k_block_select(const float* __restrict__ scores,
                                                                          int32_t* __restrict__ blk, int L, int nq,
                                                                          int B, int nb, int m, int nq_total,
                                                                          const int32_t* __restrict__ lens,
                                                                          bool vec) {
  constexpr int QPB = NW == 1 ? 4 : 1;  // queries per workgroup
  constexpr int GT = NW * kWave;        // threads per select group
  __shared__ SelectSmem<NW> lds[QPB];
  const int wave = threadIdx.x / kWave;
  const int q = NW == 1 ? (int)blockIdx.x * 4 + wave : (int)blockIdx.x;
  if (q >= nq_total) return;  // wave-uniform (NW == 1 only)
  SelectSmem<NW>& sm = lds[NW == 1 ? wave : 0];
  const int gtid = NW == 1 ? lane_id() : (int)threadIdx.x;
  const int i = q % nq;
  const int t = query_pos(seq_len_of(lens, L, q / nq), nq, i);
  const int c = t / B;
  int32_t* out = blk + (size_t)q * m;
  if (c + 1 <= m) {
    for (int j = gtid; j < m; j += GT) out[j] = j <= c ? j : -1;
    return;
  }
  const int want = m - 2;
  const int n = c - 1;  // candidates: blocks 1 .. c-1 (index = block - 1)
  if (gtid == 0) {
    out[0] = 0;
    out[m - 1] = c;
  }
  if (want == 0) return;
  uint32_t key[R];
  if constexpr (R >= 4) {
    if (vec) {
      // (uniform) 16-byte-aligned score rows: slot = block number, thread
      // x loads blocks x*R .. x*R+R-1 with R/4 aligned 16-byte loads and
      // keeps blocks 1 .. c-1 (scalar loads at a stride of R floats were
      // the select's longest phase)
      const float* sc = scores + (size_t)q * nb;
#pragma unroll
      for (int r = 0; r < R; r += 4) {
        const int j0 = gtid * R + r;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (j0 < nb) v = *reinterpret_cast<const f32x4*>(sc + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[r + e] = (j0 + e >= 1 && j0 + e <= n) ? score_key(v[e]) : 0u;
      }
      select_top<NW, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
        if (take) out[1 + pos] = idx;
      });
      return;
    }
  }
  const float* sc = scores + (size_t)q * nb + 1;  // slot = block number - 1
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = gtid * R + r;
    const float v = sc[idx < n ? idx : 0];  // branch-free: all loads in flight together
    key[r] = idx < n ? score_key(v) : 0u;
  }
  select_top<NW, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
    if (take) out[1 + pos] = 1 + idx;
  });
}

// Decode block top-m in one launch (few queries, at most kFusedMaxBlocks
// scored blocks, one summary vector per block): one 1024-thread workgroup
// per query scores its causal blocks 1..c-1 into LDS (16-byte summary-row
// loads, d_index/8 lanes per row, 8 rounds of loads in flight, dot products
// reduced by xor shuffles) and runs the 16-wave select on them, so the
// scores never leave the chip.  Workgroups past the queries summarise the
// newest blocks when the host folds that in (as for k_block_scores).
constexpr int kFusedMaxBlocks = 2048;

template <int DI, int R, int NWS>
__global__ __launch_bounds__(1024) void k_block_topm_decode(const uint16_t* __restrict__ qI,
                                                            const uint16_t* __restrict__ S, int32_t* __restrict__ blk,
                                                            int L, int nq, int B, int nb, int m, int nq_total,
                                                            const uint16_t* __restrict__ kI,
                                                            uint16_t* __restrict__ S_out, int sum_start, int nsum,
                                                            const int32_t* __restrict__ lens) {
  constexpr int LPR = DI / 8;      // lanes per summary row
  constexpr int RPI = 1024 / LPR;  // rows per round of the workgroup
  constexpr int U = 8;             // rounds of loads in flight
  __shared__ __attribute__((aligned(16))) float sc[kFusedMaxBlocks];
  __shared__ SelectSmem<NWS> sm;
  __shared__ float red[1][1024 / LPR][DI];
  if ((int)blockIdx.x >= nq_total) {  // folded summary of a newest block (uniform)
    const int w = (int)blockIdx.x - nq_total;
    const int bs = w / nsum;
    const int Lb = seq_len_of(lens, L, bs);
    // per-sequence lengths (n_q == 1): the block of the sequence's query
    const int jb = (lens ? (Lb - 1) / B : sum_start) + w % nsum;
    if (jb >= nb || jb * B >= Lb) return;
    summarise_block<DI, 1, 1024>(kI, nullptr, S_out, L, Lb, B, nb, jb, bs, red);
    return;
  }
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = q / nq;
  const int t = query_pos(seq_len_of(lens, L, b), nq, q % nq);
  const int c = t / B;
  int32_t* out = blk + (size_t)q * m;
  if (c + 1 <= m) {
    for (int j = tid; j < m; j += 1024) out[j] = j <= c ? j : -1;
    return;
  }
  const int want = m - 2;
  const int n = c - 1;  // candidates: blocks 1 .. c-1 (index = block - 1)
  if (tid == 0) {
    out[0] = 0;
    out[m - 1] = c;
  }
  if (want == 0) return;

  const int col8 = tid % LPR, r0 = tid / LPR;
  float qv[8];
  {
    const u32x4 v = *reinterpret_cast<const u32x4*>(qI + (size_t)q * DI + col8 * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(v[e]);
      qv[2 * e + 1] = bf16_hi(v[e]);
    }
  }
  const uint16_t* Sb = S + ((size_t)b * nb + 1) * DI;  // row j-1 = block j
  for (int base = 0; base < n; base += U * RPI) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(base + u * RPI + r0, n - 1);
      v[u] = *reinterpret_cast<const u32x4*>(Sb + (size_t)row * DI + col8 * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += qv[2 * e] * bf16_lo(v[u][e]);
        dot += qv[2 * e + 1] * bf16_hi(v[u][e]);
      }
      dot = group_sum_f<LPR>(dot);
      const int row = base + u * RPI + r0;
      if (col8 == 0 && row < n) sc[row] = dot;
    }
  }
  __syncthreads();
  // the select: 16 waves (R keys per thread) or one wave (R keys per lane,
  // no workgroup barriers)
  if (NWS == 1 && tid >= kWave) return;
  uint32_t key[R];
  if constexpr (R >= 4) {
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sc + tid * R + r);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[r + e] = tid * R + r + e < n ? score_key(v[e]) : 0u;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid * R + r;
      key[r] = idx < n ? score_key(sc[idx]) : 0u;
    }
  }
  select_top<NWS, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
    if (take) out[1 + pos] = 1 + idx;
  });
}

// Decode, the block top-m and step 3's token scores in one launch (few
// queries, one summary vector per block, at most kFusedMaxBlocks scored
// blocks).  P workgroups per query each repeat the query's block selection
// (as k_block_topm_decode: the causal blocks' scores into LDS, the one-wave
// select), keep the list in LDS, and then score the tokens of every P-th
// kept block (list positions p, p + P, ...) into the slot-ordered scores,
// as k_token_scores does; workgroup p = 0 writes the list.  The repeats
// read the query's block summaries again (from L2: the P workgroups of a
// query get workgroup ids congruent mod 8, which the hardware deals to one
// XCD), and the launch saves a launch gap and the list's trip through
// memory.  Workgroups past the queries summarise the newest blocks when the
// host folds that in.
constexpr int kBtMaxM = 1024;

template <int DI, int R>
__global__ __launch_bounds__(1024) void k_block_token_decode(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ S, const uint16_t* __restrict__ kI,
    int32_t* __restrict__ blk, float* __restrict__ scores, int L, int nq, int B, int log2B, int nb, int m, int k,
    int nq_total, int P, int n_query_wg, uint16_t* __restrict__ S_out, int sum_start, int nsum,
    const int32_t* __restrict__ lens) {
  constexpr int LPR = DI / 8;      // lanes per row
  constexpr int RPI = 1024 / LPR;  // rows per round of the workgroup
  constexpr int U = 8;             // rounds of loads in flight
  __shared__ __attribute__((aligned(16))) float sc[kFusedMaxBlocks];
  __shared__ SelectSmem<1> sm;
  __shared__ float red[1][1024 / LPR][DI];
  __shared__ int lst[kBtMaxM];
  if ((int)blockIdx.x >= n_query_wg) {  // folded summary of a newest block (uniform)
    const int w = (int)blockIdx.x - n_query_wg;
    const int bs = w / nsum;
    const int Lb = seq_len_of(lens, L, bs);
    const int jb = (lens ? (Lb - 1) / B : sum_start) + w % nsum;
    if (jb >= nb || jb * B >= Lb) return;
    summarise_block<DI, 1, 1024>(kI, nullptr, S_out, L, Lb, B, nb, jb, bs, red);
    return;
  }
  // workgroup x: XCD x % 8; queries 8 g + x % 8 of group g = x / (8 P)
  const int x = blockIdx.x;
  const int slot = x >> 3;
  const int q = (slot / P) * 8 + (x & 7);
  const int p = slot % P;
  if (q >= nq_total) return;
  const int tid = threadIdx.x;
  const int b = q / nq;
  const int t = query_pos(seq_len_of(lens, L, b), nq, q % nq);
  const int c = t / B;
  const int col8 = tid % LPR, r0 = tid / LPR;
  float qv[8];
  {
    const u32x4 v = *reinterpret_cast<const u32x4*>(qI + (size_t)q * DI + col8 * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(v[e]);
      qv[2 * e + 1] = bf16_hi(v[e]);
    }
  }
  // ---- the block list, in LDS
  if (c + 1 <= m) {
    for (int j = tid; j < m; j += 1024) lst[j] = j <= c ? j : -1;
  } else {
    const int want = m - 2;
    const int n = c - 1;  // candidates: blocks 1 .. c-1 (index = block - 1)
    if (tid == 0) {
      lst[0] = 0;
      lst[m - 1] = c;
    }
    if (want > 0) {
      const uint16_t* Sb = S + ((size_t)b * nb + 1) * DI;  // row j-1 = block j
      for (int base = 0; base < n; base += U * RPI) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int row = min(base + u * RPI + r0, n - 1);
          v[u] = *reinterpret_cast<const u32x4*>(Sb + (size_t)row * DI + col8 * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dot += qv[2 * e] * bf16_lo(v[u][e]);
            dot += qv[2 * e + 1] * bf16_hi(v[u][e]);
          }
          dot = group_sum_f<LPR>(dot);
          const int row = base + u * RPI + r0;
          if (col8 == 0 && row < n) sc[row] = dot;
        }
      }
      __syncthreads();
      if (tid < kWave) {  // one-wave select, R keys per lane
        uint32_t key[R];
#pragma unroll
        for (int r = 0; r < R; r += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sc + tid * R + r);
#pragma unroll
          for (int e = 0; e < 4; ++e) key[r + e] = tid * R + r + e < n ? score_key(v[e]) : 0u;
        }
        select_top<1, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
          if (take) lst[1 + pos] = 1 + idx;
        });
      }
    }
  }
  __syncthreads();
  if (p == 0)
    for (int j = tid; j < m; j += 1024) blk[(size_t)q * m + j] = lst[j];

  // ---- token scores of list positions p, p + P, ... (slot i * B + r)
  int cq, n_sel, n_valid;
  candidate_count(t, B, m, cq, n_sel, n_valid);
  if (n_valid <= k) return;  // the query keeps all of its candidates
  const int mine = (n_sel - p + P - 1) / P;
  if (mine <= 0) return;
  const int total = mine * B;  // rows of this workgroup's blocks
  const uint16_t* kseq = kI + (size_t)b * L * DI;
  float* outq = scores + (size_t)q * m * B;
  for (int base = 0; base < total; base += U * RPI) {
    u32x4 v[U];
    int slot_of[U], rows_of[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = min(base + u * RPI + r0, total - 1);
      const int i = p + (g >> log2B) * P;
      const int j = max(lst[i], 0);
      const int r = g & (B - 1);
      const int rows = min(B, t - j * B + 1);
      slot_of[u] = i * B + r;
      rows_of[u] = lst[i] >= 0 ? rows - r : 0;  // > 0: a causal row of a kept block
      v[u] = *reinterpret_cast<const u32x4*>(kseq + ((size_t)j * B + min(r, rows - 1)) * DI + col8 * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += qv[2 * e] * bf16_lo(v[u][e]);
        dot += qv[2 * e + 1] * bf16_hi(v[u][e]);
      }
      dot = group_sum_f<LPR>(dot);
      if (col8 == 0 && base + u * RPI + r0 < total && rows_of[u] > 0) outq[slot_of[u]] = dot;
    }
  }
}

// Workgroups per query of k_block_token_decode (0: not used): the query
// workgroups should fill the chip in one round (one 1024-thread workgroup
// per CU), with at least 4 per query to share out its token rows.  The few
// summary workgroups of a fold run on the CUs the first query workgroups
// free (decode_128k: 8 per query and 32 summaries, 41.0 µs per step,
// against 7 per query sharing the first round with them, 41.5 µs).
static int block_token_parts(const Dims& s) {
  const int groups = (s.b * s.nq + 7) / 8;
  return std::min(8, 256 / (8 * groups));
}

static int block_token_fold_wgs(const Dims& s, const SummaryFold* fold) {
  if (!fold) return 0;
  return s.b * (s.lens ? 1 : s.nb - fold->start_block);
}

bool block_token_fusable(const Dims& s, const SummaryFold* /*fold*/) {
  const int nq_total = s.b * s.nq;
  const int c_max = (s.L - 1) / s.B;
  if (nq_total == 0 || s.nq >= 64 || s.nL != 1 || c_max + 1 <= s.m || c_max - 1 > kFusedMaxBlocks) return false;
  if (!((long long)s.k < (long long)s.m * s.B && s.L > s.k) || s.m > kBtMaxM) return false;
  return block_token_parts(s) >= 4;
}

hipError_t launch_block_token_decode(const Dims& s, const uint16_t* qI, const uint16_t* S, const uint16_t* kI,
                                     int32_t* blk, float* scores, hipStream_t st, const SummaryFold* fold) {
  if (!block_token_fusable(s, fold)) return hipErrorInvalidValue;
  const int nq_total = s.b * s.nq;
  const int n_fold = block_token_fold_wgs(s, fold);
  const int P = block_token_parts(s);
  const int n_query_wg = ((nq_total + 7) / 8) * 8 * P;
  const int nsum = fold ? (s.lens ? 1 : s.nb - fold->start_block) : 1;
  uint16_t* S_out = fold ? fold->S : nullptr;
  const int start = fold ? fold->start_block : s.nb;
  const int n_max = (s.L - 1) / s.B - 1;
  const dim3 grid(n_query_wg + n_fold);
  const int log2B = __builtin_ctz((unsigned)s.B);
#define HSA_BT(DI, RR)                                                                                              \
  HSA_LAUNCH((k_block_token_decode<DI, RR>), grid, dim3(1024), 0, st, qI, S, kI, blk, scores, s.L, s.nq, s.B, log2B, \
             s.nb, s.m, s.k, nq_total, P, n_query_wg, S_out, start, nsum, s.lens)
  if (s.dI == 64) {
    if (n_max <= 1024) HSA_BT(64, 16); else HSA_BT(64, 32);
  } else {
    if (n_max <= 1024) HSA_BT(128, 16); else HSA_BT(128, 32);
  }
#undef HSA_BT
  return hipGetLastError();
}

template <int NW, int R>
static hipError_t launch_select_r(int nq_total, const float* scores, int32_t* blk, const Dims& s, hipStream_t st) {
  dim3 grid(NW == 1 ? (nq_total + 3) / 4 : nq_total), block(NW == 1 ? 256 : NW * 64);
  // block-number slots need nb % 4 == 0 (aligned rows) and slots for blocks
  // 0 .. c_max - 1 of the latest query
  const int c_max = (s.L - 1) / s.B;
  const bool vec = R >= 4 && s.nb % 4 == 0 && (long long)NW * kWave * R >= c_max;
  HSA_LAUNCH((k_block_select<NW, R>), grid, block, 0, st, scores, blk, s.L, s.nq, s.B, s.nb, s.m, nq_total,
                     s.lens, vec);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_select(int R, int nq_total, const float* scores, int32_t* blk, const Dims& s,
                                hipStream_t st) {
  switch (R) {
    case 1: return launch_select_r<NW, 1>(nq_total, scores, blk, s, st);
    case 2: return launch_select_r<NW, 2>(nq_total, scores, blk, s, st);
    case 4: return launch_select_r<NW, 4>(nq_total, scores, blk, s, st);
    case 8: return launch_select_r<NW, 8>(nq_total, scores, blk, s, st);
    case 16: return launch_select_r<NW, 16>(nq_total, scores, blk, s, st);
    case 32:
      if constexpr (NW > 1) return launch_select_r<NW, 32>(nq_total, scores, blk, s, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

size_t block_topm_ws_bytes(const Dims& s) { return align_up((size_t)s.b * s.nq * s.nb * sizeof(float)); }

// Chunks of 128-row summary tiles per 256-query tile of k_block_scores_max.
// A workgroup loads its queries' indexer vectors (64 KB) once for all the
// tiles of its chunk, so the tiles are split into chunks only as far as
// needed to give about two workgroups per CU (512), the most the LDS holds,
// so that causal tiles of very different lengths still spread over the chip.
constexpr int kScoreMaxWgs = 256;

static void score_max_plan(const Dims& s, int& tiles_per_chunk, int& nchunks) {
  const int qtiles = std::max(1, s.b * ((s.nq + kMaxQT - 1) / kMaxQT));
  const int ntiles = std::max(1, (s.nb * s.nL + kMaxRT - 1) / kMaxRT);
  // about one 8-wave workgroup per CU; row chunks only when the query
  // tiles alone would leave CUs idle
  const int want = std::max(1, std::min(ntiles, (kScoreMaxWgs + qtiles - 1) / qtiles));
  tiles_per_chunk = (ntiles + want - 1) / want;
  nchunks = (ntiles + tiles_per_chunk - 1) / tiles_per_chunk;
}

size_t block_score_max_ws_bytes(const Dims& s) {
  int tpc, nchunks;
  score_max_plan(s, tpc, nchunks);
  return nchunks > 1 ? align_up((size_t)s.b * s.nq * nchunks * sizeof(float)) : 0;
}

hipError_t launch_block_score_max(const Dims& s, const uint16_t* qI, const uint16_t* S, float* out, void* ws,
                                  hipStream_t st) {
  const int nq_total = s.b * s.nq;
  if (nq_total == 0) return hipSuccess;
  int tpc, nchunks;
  score_max_plan(s, tpc, nchunks);
  const int qtiles = (s.nq + kMaxQT - 1) / kMaxQT;
  float* dst = nchunks > 1 ? static_cast<float*>(ws) : out;
  const dim3 grid(nchunks, qtiles * s.b);
  const int log2B = __builtin_ctz((unsigned)s.B);
  const dim3 block(kMaxWaves * 64);
  if (s.dI == 64)
    HSA_LAUNCH((k_block_scores_max<64>), grid, block, 0, st, qI, S, dst, s.L, s.nq, log2B, s.nb, s.nL, s.m, qtiles,
               tpc, nchunks);
  else
    HSA_LAUNCH((k_block_scores_max<128>), grid, block, 0, st, qI, S, dst, s.L, s.nq, log2B, s.nb, s.nL, s.m,
               qtiles, tpc, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 1) return e;
  HSA_LAUNCH(k_block_max_reduce, dim3((nq_total + 255) / 256), dim3(256), 0, st, dst, out, nq_total, nchunks);
  return hipGetLastError();
}

static int pick_r(int n, int nw) {
  int r = 1;
  while (r * 64 * nw < n) r <<= 1;
  return r;
}

bool block_topm_can_fold(const Dims& s, int start_block) {
  const int c_max = (s.L - 1) / s.B;
  // the GEMV kernel runs (few queries, some query scores blocks) and no
  // query scores a block >= start_block (the highest scored is c_max - 1);
  // with per-sequence lengths (one query each) the re-summarised block is
  // always the query's own, never scored
  if (s.lens) return s.nq == 1 && c_max + 1 > s.m;
  return s.nq < 64 && c_max + 1 > s.m && start_block >= c_max && start_block < s.nb;
}

hipError_t launch_block_topm(const Dims& s, const uint16_t* qI, const uint16_t* S, int32_t* blk, void* ws,
                             hipStream_t st, const SummaryFold* fold) {
  const int nq_total = s.b * s.nq;
  if (nq_total == 0) return hipSuccess;
  float* scores = static_cast<float*>(ws);
  // the last query has the most causal blocks
  const int c_max = (s.L - 1) / s.B;
  const int n_max = c_max - 1;
  if (c_max + 1 > s.m && s.nq >= 64 && s.nb <= kTileMaxBlocks && !s.lens) {
    // scores and select in one launch, the scores in LDS; 8 queries per
    // workgroup when 16 would leave fewer than 1024 workgroups
    const int tq = (long long)s.b * ((s.nq + 15) / 16) >= 1024 ? 16 : 8;
    const int qtiles = (s.nq + tq - 1) / tq;
    const int ldsw = (s.nb + 3) & ~3;
    const size_t lds = (size_t)tq * ldsw * sizeof(float);
    const int r = pick_r(n_max, 1);
#define HSA_TT(DI, NL, RR, TQ)                                                                                     \
  do {                                                                                                             \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_topm_tile<DI, NL, RR, TQ>),          \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                      \
    if (e != hipSuccess) return e;                                                                                 \
    HSA_LAUNCH((k_block_topm_tile<DI, NL, RR, TQ>), dim3(qtiles * s.b), dim3(256), lds, st, qI, S, blk, s.L, s.nq, \
               s.B, s.nb, s.m, qtiles, ldsw);                                                                      \
  } while (0)
#define HSA_TQ(DI, NL, RR)             \
  if (tq == 16) HSA_TT(DI, NL, RR, 16); \
  else HSA_TT(DI, NL, RR, 8);
#define HSA_TR(DI, NL)                    \
  switch (r) {                            \
    case 1: HSA_TQ(DI, NL, 1) break;      \
    case 2: HSA_TQ(DI, NL, 2) break;      \
    case 4: HSA_TQ(DI, NL, 4) break;      \
    case 8: HSA_TQ(DI, NL, 8) break;      \
    case 16: HSA_TQ(DI, NL, 16) break;    \
    default: HSA_TQ(DI, NL, 32) break;    \
  }
    if (s.dI == 64) {
      if (s.nL == 1) { HSA_TR(64, 1) } else if (s.nL == 2) { HSA_TR(64, 2) } else { HSA_TR(64, 4) }
    } else {
      if (s.nL == 1) { HSA_TR(128, 1) } else if (s.nL == 2) { HSA_TR(128, 2) } else { HSA_TR(128, 4) }
    }
#undef HSA_TQ
#undef HSA_TR
#undef HSA_TT
    return hipGetLastError();
  }
  if (c_max + 1 > s.m && s.nq >= 64) {
    const int qtiles = (s.nq + 63) / 64;
    dim3 grid((s.nb * s.nL + 127) / 128, qtiles * s.b);
#define HSA_SM(DI, NL)                                                                                      \
  HSA_LAUNCH((k_block_scores_mfma<DI, NL>), grid, dim3(256), 0, st, qI, S, scores, s.L, s.nq, s.B, \
                     s.nb, s.m, qtiles)
    if (s.dI == 64) {
      if (s.nL == 1) HSA_SM(64, 1); else if (s.nL == 2) HSA_SM(64, 2); else HSA_SM(64, 4);
    } else {
      if (s.nL == 1) HSA_SM(128, 1); else if (s.nL == 2) HSA_SM(128, 2); else HSA_SM(128, 4);
    }
#undef HSA_SM
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (c_max + 1 > s.m && s.nL == 1 && n_max <= kFusedMaxBlocks && nq_total < 512) {
    const int nsum = fold ? (s.lens ? 1 : s.nb - fold->start_block) : 0;
    dim3 grid(nq_total + (fold ? s.b * nsum : 0));
    const uint16_t* kI = fold ? fold->kI : nullptr;
    uint16_t* S_out = fold ? fold->S : nullptr;
    const int start = fold ? fold->start_block : s.nb;
    const int ns = max(nsum, 1);
#define HSA_FD(DI, RR)                                                                                             \
  HSA_LAUNCH((k_block_topm_decode<DI, RR, 1>), grid, dim3(1024), 0, st, qI, S, blk, s.L, s.nq, s.B, s.nb, s.m, \
                     nq_total, kI, S_out, start, ns, s.lens)
    if (s.dI == 64) {
      if (n_max <= 1024) HSA_FD(64, 16); else HSA_FD(64, 32);
    } else {
      if (n_max <= 1024) HSA_FD(128, 16); else HSA_FD(128, 32);
    }
#undef HSA_FD
    return hipGetLastError();
  } else if (c_max + 1 > s.m) {
    const int xs = (c_max + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG;
    const int nsum = fold ? (s.lens ? 1 : s.nb - fold->start_block) : 0;
    dim3 grid(max(xs, nsum), max(nq_total, fold ? s.b : 0), fold ? 2 : 1);
    const uint16_t* kI = fold ? fold->kI : nullptr;
    const int8_t* W = fold ? fold->W : nullptr;
    uint16_t* S_out = fold ? fold->S : nullptr;
    const int start = fold ? fold->start_block : s.nb;
#define HSA_SC(DI, NL)                                                                                          \
  HSA_LAUNCH((k_block_scores<DI, NL>), grid, dim3(256), 0, st, qI, S, scores, s.L, s.nq, s.B, s.nb, s.m, \
                     kI, W, S_out, start, s.b, s.lens)
    if (s.dI == 64) {
      if (s.nL == 1) HSA_SC(64, 1); else if (s.nL == 2) HSA_SC(64, 2); else HSA_SC(64, 4);
    } else {
      if (s.nL == 1) HSA_SC(128, 1); else if (s.nL == 2) HSA_SC(128, 2); else HSA_SC(128, 4);
    }
#undef HSA_SC
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // many queries: one wave per query (<= 512 candidates) or a 4-wave
  // workgroup per query; few queries: 16 waves per query (shortest latency)
  if (nq_total >= 512 && n_max <= 64 * 8) return launch_select<1>(pick_r(n_max, 1), nq_total, scores, blk, s, st);
  if (nq_total >= 512 && n_max <= 4 * 64 * 32) return launch_select<4>(pick_r(n_max, 4), nq_total, scores, blk, s, st);
  return launch_select<16>(pick_r(n_max, 16), nq_total, scores, blk, s, st);
}

}  // namespace hsa
