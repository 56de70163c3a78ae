// A third, coarser level above the blocks: super-blocks of G consecutive
// blocks (G a power of two).
//
// LSA page (latent space and hierarchical clustering): keys are organised as
// a tree and a query descends from the root, scoring only a few nodes at
// every level instead of every leaf.  Here the tree is fixed: level 1 holds
// super-blocks of G blocks, level 2 the blocks, level 3 the tokens.  A
// super-block is summarised by the mean of its blocks' summaries and
// selected exactly like a block (HISA page, step one: indexer-rule scores,
// the first and the query's own super-block always kept); the blocks are
// then selected among the blocks of the kept super-blocks only.
//
// k_super_summary: S2[J, l] = bf16_rne(sum_g S[J*G + g, l] / G), one thread
// per 8 output elements, fp32 sums scaled by the exact power of two 1/G;
// blocks past the sequence's last block count as zero.  With per-sequence
// lengths only the super-block holding each sequence's last block is
// rebuilt.
// Level 1 reuses the block top-m launcher with block size B*G, nsb
// super-blocks and m2 kept.
// k_block_topm_l2: one workgroup per query gathers the summary rows of its
// candidate blocks (the blocks j <= c of its kept super-blocks, at most
// m2*G), scores them into LDS and runs the exact select for m - 2 blocks
// besides block 0 and block c.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"
#include "summary.hpp"

namespace hsa {

template <int DI>
__global__ __launch_bounds__(256) void k_super_summary(const uint16_t* __restrict__ S, uint16_t* __restrict__ S2,
                                                       int nb, int nsb, int NL, int lgG, int start_super,
                                                       int n_items, const int32_t* __restrict__ lens, int L,
                                                       int B) {
  constexpr int C8 = DI / 8;  // 16-byte chunks per summary row
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= n_items) return;
  const int per_super = NL * C8;
  const int nJ = lens ? 1 : nsb - start_super;
  const int rest = item % per_super;      // l * C8 + e8
  const int b = item / (per_super * nJ);
  int J, nb_b;  // super-block, blocks of the sequence
  if (lens) {
    const int Lb = seq_len_of(lens, L, b);
    J = ((Lb - 1) / B) >> lgG;
    nb_b = (Lb + B - 1) / B;
  } else {
    J = start_super + (item / per_super) % nJ;
    nb_b = nb;
  }
  const int G = 1 << lgG;
  const int g_end = min(G, nb_b - (J << lgG));
  const uint16_t* src = S + (((size_t)b * nb + ((size_t)J << lgG)) * NL * C8 + rest) * 8;
  const size_t stride = (size_t)NL * DI;  // one block's summary rows
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int g = 0;
  for (; g + 4 <= g_end; g += 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const u32x4*>(src + (size_t)(g + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(v[u][e]);
        acc[2 * e + 1] += bf16_hi(v[u][e]);
      }
    }
  }
  for (; g < g_end; ++g) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)g * stride);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(v[e]);
      acc[2 * e + 1] += bf16_hi(v[e]);
    }
  }
  const float inv_g = __builtin_ldexpf(1.f, -lgG);  // exact
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f32_to_bf16_rne(acc[2 * e] * inv_g) | (f32_to_bf16_rne(acc[2 * e + 1] * inv_g) << 16);
  *reinterpret_cast<u32x4*>(S2 + (((size_t)b * nsb + J) * NL * C8 + rest) * 8) = o;
}

// Candidate slot s of a query (0 <= s < n) is block sup[s / G] * G + s % G:
// the kept super-blocks are ascending and only the last one (the query's
// own) can be cut short by c, so the slots enumerate the candidate blocks
// in ascending order without gaps.
template <int DI, int NL, int NW, int R>
__global__ __launch_bounds__(NW * 64) void k_block_topm_l2(const uint16_t* __restrict__ qI,
                                                           const uint16_t* __restrict__ S,
                                                           const int32_t* __restrict__ sup,
                                                           int32_t* __restrict__ blk, int L, int nq, int B, int lgG,
                                                           int nb, int m2, int m, const int32_t* __restrict__ lens) {
  constexpr int NT = NW * kWave;
  constexpr int LPR = DI / 8;     // lanes per summary row
  constexpr int RPI = NT / LPR;   // rows per round of the workgroup
  constexpr int U = 4;            // rounds of loads in flight
  static_assert((kWave / LPR) % NL == 0, "a block's landmarks must share one wave load");
  __shared__ float sc[NT * R];
  __shared__ SelectSmem<NW> sm;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = q / nq;
  const int t = query_pos(seq_len_of(lens, L, b), nq, q % nq);
  const int c = t / B;
  const int gmask = (1 << lgG) - 1;
  const int C = c >> lgG;
  const int n_sup = min(C + 1, m2);
  const int n = ((n_sup - 1) << lgG) + (c & gmask) + 1;  // candidate blocks
  const int32_t* sq = sup + (size_t)q * m2;
  int32_t* out = blk + (size_t)q * m;
  if (n <= m) {
    for (int s = tid; s < m; s += NT) out[s] = s < n ? (sq[s >> lgG] << lgG) + (s & gmask) : -1;
    return;
  }
  if (tid == 0) {
    out[0] = 0;
    out[m - 1] = c;
  }
  const int want = m - 2;
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
  const uint16_t* Sb = S + (size_t)b * nb * NL * DI;
  const int nrows = n * NL;
  for (int base = 0; base < nrows; base += U * RPI) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(base + u * RPI + r0, nrows - 1);
      const int slot = row / NL;
      const int j = (sq[slot >> lgG] << lgG) + (slot & gmask);
      v[u] = *reinterpret_cast<const u32x4*>(Sb + ((size_t)j * NL + row % NL) * DI + col8 * 8);
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
      if constexpr (NL > 1) dot = group_max_f<LPR * NL>(dot);  // a block's landmark rows are adjacent
      const int row = base + u * RPI + r0;
      if (row < nrows && tid % (LPR * NL) == 0) sc[row / NL] = dot;
    }
  }
  __syncthreads();
  // slot 0 is block 0 and slot n - 1 is block c: both forced, not candidates
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = tid * R + r;
    key[r] = (idx >= 1 && idx <= n - 2) ? score_key(sc[idx]) : 0u;
  }
  select_top<NW, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
    if (take) out[1 + pos] = (sq[idx >> lgG] << lgG) + (idx & gmask);
  });
}

// Decode (few queries, one summary vector per block): both levels in one
// launch.  One 1024-thread workgroup per query scores its causal
// super-blocks 1..C-1 into LDS (16-byte summary-row loads, d_index/8 lanes
// per row, 8 rounds of loads in flight), selects m2 - 2 of them, keeps the
// list in LDS, then scores the candidate blocks of the kept super-blocks
// into the same LDS and selects m - 2 of those.  Workgroups past the
// queries re-summarise the newest block and its super-block when the host
// folds that in: every query's own block and super-block are always kept,
// so neither summary is read here.
constexpr int kFused3MaxSuper = 2048;  // level-1 scores held in LDS
constexpr int kFused3MaxM2 = 1024;     // level-1 list held in LDS

template <int DI, int R1, int R2>
__global__ __launch_bounds__(1024) void k_block_topm_3level_decode(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ S, const uint16_t* __restrict__ S2,
    int32_t* __restrict__ sup, int32_t* __restrict__ blk, int L, int nq, int B, int lgG, int nb, int nsb, int m2,
    int m, int nq_total, const uint16_t* __restrict__ kI, uint16_t* __restrict__ S_out,
    uint16_t* __restrict__ S2_out, int sum_start, int nsum, const int32_t* __restrict__ lens) {
  constexpr int LPR = DI / 8;      // lanes per summary row
  constexpr int RPI = 1024 / LPR;  // rows per round of the workgroup
  constexpr int U = 8;             // rounds of loads in flight
  constexpr int NSC = 1024 * R2 > kFused3MaxSuper ? 1024 * R2 : kFused3MaxSuper;
  static_assert(1024 * R1 <= kFused3MaxSuper, "level-1 keys exceed the LDS scores");
  __shared__ union {
    struct {
      float sc[NSC];
      int32_t sl[kFused3MaxM2];
    } q;
    float red[1][1024 / LPR][DI];
  } u;
  __shared__ SelectSmem<16> sm;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= nq_total) {  // folded summaries of a newest block (uniform)
    const int w = (int)blockIdx.x - nq_total;
    const int bs = w / nsum;
    const int Lb = seq_len_of(lens, L, bs);
    const int jb = (lens ? (Lb - 1) / B : sum_start) + w % nsum;
    if (jb >= nb) return;
    summarise_block<DI, 1, 1024>(kI, nullptr, S_out, L, Lb, B, nb, jb, bs, u.red, S2_out, lgG);
    return;
  }
  const int q = blockIdx.x;
  const int b = q / nq;
  const int t = query_pos(seq_len_of(lens, L, b), nq, q % nq);
  const int c = t / B;
  const int C = c >> lgG;
  const int gmask = (1 << lgG) - 1;
  int32_t* sup_out = sup + (size_t)q * m2;
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
  // rows [row0, row0 + n) of a summary array, row r's index given by
  // idx_of(r); dot products into u.q.sc[r - row0]
  auto score_rows = [&](const uint16_t* base, int n, auto idx_of) {
    for (int r = 0; r < n; r += U * RPI) {
      u32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int row = min(r + k * RPI + r0, n - 1);
        v[k] = *reinterpret_cast<const u32x4*>(base + (size_t)idx_of(row) * DI + col8 * 8);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dot += qv[2 * e] * bf16_lo(v[k][e]);
          dot += qv[2 * e + 1] * bf16_hi(v[k][e]);
        }
        dot = group_sum_f<LPR>(dot);
        const int row = r + k * RPI + r0;
        if (col8 == 0 && row < n) u.q.sc[row] = dot;
      }
    }
  };

  // level 1: super-blocks
  int n_sup;
  if (C + 1 <= m2) {
    n_sup = C + 1;
    for (int j = tid; j < m2; j += 1024) {
      const int v = j <= C ? j : -1;
      sup_out[j] = v;
      u.q.sl[j] = v;
    }
  } else {
    n_sup = m2;
    if (tid == 0) {
      sup_out[0] = u.q.sl[0] = 0;
      sup_out[m2 - 1] = u.q.sl[m2 - 1] = C;
    }
    const int want1 = m2 - 2;
    if (want1 > 0) {
      const int n1 = C - 1;  // candidates: super-blocks 1 .. C-1 (index = super-block - 1)
      score_rows(S2 + ((size_t)b * nsb + 1) * DI, n1, [](int row) { return row; });
      __syncthreads();
      uint32_t key[R1];
#pragma unroll
      for (int r = 0; r < R1; ++r) {
        const int idx = tid * R1 + r;
        key[r] = idx < n1 ? score_key(u.q.sc[idx]) : 0u;
      }
      select_top<16, R1>(key, want1, sm, [&](int pos, int idx, bool take, uint32_t) {
        if (take) sup_out[1 + pos] = u.q.sl[1 + pos] = 1 + idx;
      });
    }
  }
  __syncthreads();

  // level 2: candidate slot s is block sl[s / G] * G + s % G
  const int n = ((n_sup - 1) << lgG) + (c & gmask) + 1;
  int32_t* out = blk + (size_t)q * m;
  if (n <= m) {
    for (int s = tid; s < m; s += 1024) out[s] = s < n ? (u.q.sl[s >> lgG] << lgG) + (s & gmask) : -1;
    return;
  }
  if (tid == 0) {
    out[0] = 0;
    out[m - 1] = c;
  }
  const int want = m - 2;
  if (want == 0) return;
  score_rows(S + (size_t)b * nb * DI, n, [&](int row) { return (u.q.sl[row >> lgG] << lgG) + (row & gmask); });
  __syncthreads();
  // slot 0 is block 0 and slot n - 1 is block c: both forced, not candidates
  uint32_t key[R2];
#pragma unroll
  for (int r = 0; r < R2; ++r) {
    const int idx = tid * R2 + r;
    key[r] = (idx >= 1 && idx <= n - 2) ? score_key(u.q.sc[idx]) : 0u;
  }
  select_top<16, R2, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
    if (take) out[1 + pos] = (u.q.sl[idx >> lgG] << lgG) + (idx & gmask);
  });
}

hipError_t launch_super_summary(const Dims& s, int lgG, const uint16_t* S, int start_super, uint16_t* S2,
                                hipStream_t st) {
  const int nsb = (s.nb + (1 << lgG) - 1) >> lgG;
  if (s.b == 0 || (!s.lens && start_super >= nsb)) return hipSuccess;
  const long long items = (long long)s.b * (s.lens ? 1 : nsb - start_super) * s.nL * (s.dI / 8);
  const int n_items = (int)items;
  dim3 grid((unsigned)((items + 255) / 256));
  if (s.dI == 64)
    HSA_LAUNCH((k_super_summary<64>), grid, dim3(256), 0, st, S, S2, s.nb, nsb, s.nL, lgG, start_super,
                       n_items, s.lens, s.L, s.B);
  else
    HSA_LAUNCH((k_super_summary<128>), grid, dim3(256), 0, st, S, S2, s.nb, nsb, s.nL, lgG, start_super,
                       n_items, s.lens, s.L, s.B);
  return hipGetLastError();
}

template <int NW, int R>
static hipError_t launch_l2_r(const Dims& s, int lgG, int m2, const uint16_t* qI, const uint16_t* S,
                              const int32_t* sup, int32_t* blk, hipStream_t st) {
  dim3 grid(s.b * s.nq), block(NW * 64);
#define HSA_L2(DI, NL)                                                                                   \
  HSA_LAUNCH((k_block_topm_l2<DI, NL, NW, R>), grid, block, 0, st, qI, S, sup, blk, s.L, s.nq, s.B, \
                     lgG, s.nb, m2, s.m, s.lens)
  if (s.dI == 64) {
    if (s.nL == 1) HSA_L2(64, 1); else if (s.nL == 2) HSA_L2(64, 2); else HSA_L2(64, 4);
  } else {
    if (s.nL == 1) HSA_L2(128, 1); else if (s.nL == 2) HSA_L2(128, 2); else HSA_L2(128, 4);
  }
#undef HSA_L2
  return hipGetLastError();
}

size_t block_topm_3level_ws_bytes(const Dims& s, int lgG) {
  Dims s1 = s;
  s1.B = s.B << lgG;
  s1.nb = (s.nb + (1 << lgG) - 1) >> lgG;
  return block_topm_ws_bytes(s1);
}

// The one-launch decode path applies: one summary per block, few queries,
// level-1 scores and list within the LDS the kernel holds.
static bool use_fused3(const Dims& s, int lgG, int m2) {
  const int c_max = (s.L - 1) / s.B;
  const int C_max = c_max >> lgG;
  return s.nL == 1 && s.b * s.nq < 512 && C_max - 1 <= kFused3MaxSuper && m2 <= kFused3MaxM2;
}

bool block_topm_3level_can_fold(const Dims& s, int lgG, int m2, int start_block) {
  // every query sits in the last block (so in the last super-block), the
  // only blocks and super-blocks that are re-summarised; with per-sequence
  // lengths one query per sequence, whose block is rebuilt
  if (!use_fused3(s, lgG, m2)) return false;
  if (s.lens) return s.nq == 1;
  const int c_max = (s.L - 1) / s.B;
  return start_block >= c_max && start_block < s.nb;
}

template <int DI, int R1, int R2>
static hipError_t launch_fused3_r(const Dims& s, int lgG, int m2, const uint16_t* qI, const uint16_t* S,
                                  const uint16_t* S2, int32_t* sup, int32_t* blk, hipStream_t st,
                                  const SummaryFold* fold, uint16_t* S2_out) {
  const int nq_total = s.b * s.nq;
  const int nsb = (s.nb + (1 << lgG) - 1) >> lgG;
  const int nsum = fold ? (s.lens ? 1 : s.nb - fold->start_block) : 0;
  dim3 grid(nq_total + s.b * nsum);
  HSA_LAUNCH((k_block_topm_3level_decode<DI, R1, R2>), grid, dim3(1024), 0, st, qI, S, S2, sup, blk, s.L,
                     s.nq, s.B, lgG, s.nb, nsb, m2, s.m, nq_total, fold ? fold->kI : nullptr,
                     fold ? fold->S : nullptr, S2_out, fold ? fold->start_block : s.nb, max(nsum, 1), s.lens);
  return hipGetLastError();
}

template <int DI, int R1>
static hipError_t launch_fused3_r1(const Dims& s, int lgG, int m2, int n2_max, const uint16_t* qI,
                                   const uint16_t* S, const uint16_t* S2, int32_t* sup, int32_t* blk, hipStream_t st,
                                   const SummaryFold* fold, uint16_t* S2_out) {
  if (n2_max <= 1024) return launch_fused3_r<DI, R1, 1>(s, lgG, m2, qI, S, S2, sup, blk, st, fold, S2_out);
  if (n2_max <= 2048) return launch_fused3_r<DI, R1, 2>(s, lgG, m2, qI, S, S2, sup, blk, st, fold, S2_out);
  if (n2_max <= 4096) return launch_fused3_r<DI, R1, 4>(s, lgG, m2, qI, S, S2, sup, blk, st, fold, S2_out);
  return launch_fused3_r<DI, R1, 8>(s, lgG, m2, qI, S, S2, sup, blk, st, fold, S2_out);
}

hipError_t launch_block_topm_3level(const Dims& s, int lgG, int m2, const uint16_t* qI, const uint16_t* S,
                                    const uint16_t* S2, int32_t* sup, int32_t* blk, void* ws, hipStream_t st,
                                    const SummaryFold* fold, uint16_t* S2_out) {
  if (s.b == 0 || s.nq == 0) return hipSuccess;
  if (use_fused3(s, lgG, m2)) {
    const int c_max = (s.L - 1) / s.B;
    const int n1_max = (c_max >> lgG) - 1;
    const int n2_max = min((c_max >> lgG) + 1, m2) << lgG;
    if (n2_max > 8192) return hipErrorInvalidValue;
    if (s.dI == 64)
      return n1_max <= 1024 ? launch_fused3_r1<64, 1>(s, lgG, m2, n2_max, qI, S, S2, sup, blk, st, fold, S2_out)
                            : launch_fused3_r1<64, 2>(s, lgG, m2, n2_max, qI, S, S2, sup, blk, st, fold, S2_out);
    return n1_max <= 1024 ? launch_fused3_r1<128, 1>(s, lgG, m2, n2_max, qI, S, S2, sup, blk, st, fold, S2_out)
                          : launch_fused3_r1<128, 2>(s, lgG, m2, n2_max, qI, S, S2, sup, blk, st, fold, S2_out);
  }
  if (fold) return hipErrorInvalidValue;  // the host folds only into the one-launch path
  Dims s1 = s;
  s1.B = s.B << lgG;
  s1.nb = (s.nb + (1 << lgG) - 1) >> lgG;
  s1.m = m2;
  hipError_t e = launch_block_topm(s1, qI, S2, sup, ws, st);
  if (e != hipSuccess) return e;
  // candidate slots of the query with the most: at most m2 super-blocks of G
  const int c_max = (s.L - 1) / s.B;
  const int n_max = min((c_max >> lgG) + 1, m2) << lgG;
  const int nq_total = s.b * s.nq;
  if (nq_total >= 512) {
    if (n_max <= 256) return launch_l2_r<4, 1>(s, lgG, m2, qI, S, sup, blk, st);
    if (n_max <= 512) return launch_l2_r<4, 2>(s, lgG, m2, qI, S, sup, blk, st);
    if (n_max <= 1024) return launch_l2_r<4, 4>(s, lgG, m2, qI, S, sup, blk, st);
  }
  if (n_max <= 1024) return launch_l2_r<16, 1>(s, lgG, m2, qI, S, sup, blk, st);
  if (n_max <= 2048) return launch_l2_r<16, 2>(s, lgG, m2, qI, S, sup, blk, st);
  if (n_max <= 4096) return launch_l2_r<16, 4>(s, lgG, m2, qI, S, sup, blk, st);
  if (n_max <= 8192) return launch_l2_r<16, 8>(s, lgG, m2, qI, S, sup, blk, st);
  return hipErrorInvalidValue;
}

}  // namespace hsa
