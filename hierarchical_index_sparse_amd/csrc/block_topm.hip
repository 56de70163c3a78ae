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
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"
#include "summary.hpp"

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
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[ks]),
                                                      __builtin_bit_cast(bf16x8, bs[nt][ks]), acc, 0, 0, 0);
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

template <int DI, int R>
__global__ __launch_bounds__(1024) void k_block_topm_decode(const uint16_t* __restrict__ qI,
                                                            const uint16_t* __restrict__ S, int32_t* __restrict__ blk,
                                                            int L, int nq, int B, int nb, int m, int nq_total,
                                                            const uint16_t* __restrict__ kI,
                                                            uint16_t* __restrict__ S_out, int sum_start, int nsum,
                                                            const int32_t* __restrict__ lens) {
  constexpr int LPR = DI / 8;      // lanes per summary row
  constexpr int RPI = 1024 / LPR;  // rows per round of the workgroup
  constexpr int U = 8;             // rounds of loads in flight
  __shared__ float sc[kFusedMaxBlocks];
  __shared__ SelectSmem<16> sm;
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
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = tid * R + r;
    key[r] = idx < n ? score_key(sc[idx]) : 0u;
  }
  select_top<16, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
    if (take) out[1 + pos] = 1 + idx;
  });
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
  HSA_LAUNCH((k_block_topm_decode<DI, RR>), grid, dim3(1024), 0, st, qI, S, blk, s.L, s.nq, s.B, s.nb, s.m, \
                     nq_total, kI, S_out, start, ns, s.lens)
    if (s.dI == 64) {
      if (n_max <= 1024) HSA_FD(64, 1); else HSA_FD(64, 2);
    } else {
      if (n_max <= 1024) HSA_FD(128, 1); else HSA_FD(128, 2);
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
