// Per-head chunk selection from the attention queries themselves.
//
// HiLS page (hils_attention pseudocode; section 2.1 landmark tokens,
// section 2.2 two-layer selection): the coarse layer scores each chunk by
// the attention query Q against the chunk's landmark vectors, keeps the top
// chunks and runs exact attention over the concatenated K/V of the kept
// chunks.  Here every query head ranks the chunks by its own Q_h against
// landmarks of its kv head's keys (max over landmarks), with the block rule
// of the shared indexer (first chunk and the query's own chunk kept, m in
// all), and attends over every causal token of its kept chunks.
//
// k_head_landmarks: LK[b, j, l, g] = bf16_rne(sum_r W[l, r] K[b, jB + r, g] / B),
//   accumulated in fp64, which is exact for bf16 keys whose exponents span
//   fewer than 45 bits, so the one rounding is the only one.  In decode the
//   newest chunk's landmarks are folded into the select launch.
// k_head_scores_mfma: per (sequence, kv head) a [chunk landmark rows] x
//   [(query, head-in-group) columns] contraction on v_mfma_f32_16x16x32_bf16
//   (fp32 accumulation), max over a chunk's landmarks, scores of the causal
//   chunks 1..c-1 written per (query, head) row.
// k_head_select: the exact select per (query, head) row; it also writes
//   each row's causal tokens of its kept chunks, as row indices s * Hkv + g
//   of K and V viewed as [L * Hkv, d], so the sparse attention kernel runs
//   each (query, head) as a one-head query.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace hsa {

__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  // round the 52-bit fraction to 7 bits, ties to even (normal range)
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;
  u &= ~0x00001FFFFFFFFFFFull;
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;  // exact: 8 significant bits
}

// The landmarks of chunk j of sequence b (all kv heads; rows at or past the
// sequence's length Lb count as zero), computed by the
// calling waves (wave of nw): a K row (Hkv * 128 bf16) is Hkv groups of 16
// lanes x 16 bytes; wave w takes groups w, w + nw, ...; lane = (row phase
// p = lane / 16, 16-byte column chunk lane % 16) sums rows p, p + 4, ...
// with 4 U rows of loads in flight, in fp64; the four row phases meet by
// lane shuffles.  fp64 sums of bf16 values are exact here, so the result
// does not depend on this order.  No LDS.  (U = 2 where the caller runs
// 1024-thread workgroups, whose 128 registers per lane would otherwise
// spill with four landmarks.)
template <int NL, int U = 8>
__device__ __forceinline__ void head_landmark_chunk(const uint16_t* __restrict__ K, const int8_t* __restrict__ W,
                                                    uint16_t* __restrict__ LK, int L, int Lb, int B, int nb, int Hkv,
                                                    int j, int b, int wave, int nw) {
  const int lane = lane_id();
  const int p = lane >> 4, cl = lane & 15;
  const int RW = Hkv * 128;
  const int rows = min(B, Lb - j * B);  // rows of the chunk inside the sequence (L is the row stride)
  for (int cg = wave; cg < Hkv; cg += nw) {
    const int col = (cg * 16 + cl) * 8;
    double acc[NL][8];
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[l][e] = 0.0;
    for (int r0 = 0; r0 < rows; r0 += 4 * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = min(r0 + 4 * u + p, rows - 1);
        v[u] = *reinterpret_cast<const u32x4*>(K + ((size_t)b * L + (size_t)j * B + r) * RW + col);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + 4 * u + p;
        if (r >= rows) continue;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          const double w = W ? (double)W[l * B + r] : 1.0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[l][2 * e] += w * (double)bf16_lo(v[u][e]);
            acc[l][2 * e + 1] += w * (double)bf16_hi(v[u][e]);
          }
        }
      }
    }
    const double inv_b = 1.0 / (double)B;  // exact: B is a power of two
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double x = acc[l][e];
        x += __shfl_xor(x, 16, kWave);
        x += __shfl_xor(x, 32, kWave);
        acc[l][e] = x;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = f64_to_bf16_rne(acc[l][2 * e] * inv_b) | (f64_to_bf16_rne(acc[l][2 * e + 1] * inv_b) << 16);
      if (p == 0) *reinterpret_cast<u32x4*>(LK + (((size_t)b * nb + j) * NL + l) * RW + col) = o;
    }
  }
}

// Workgroup (x, b): the landmarks of chunk start + x of sequence b; with
// per-sequence lengths (one query each), of chunk (Lb - 1) / B + x.
template <int NL>
__global__ __launch_bounds__(256) void k_head_landmarks(const uint16_t* __restrict__ K, const int8_t* __restrict__ W,
                                                        uint16_t* __restrict__ LK, int L, int B, int nb, int Hkv,
                                                        int start, const int32_t* __restrict__ lens) {
  const int Lb = seq_len_of(lens, L, blockIdx.y);
  const int j = (lens ? (Lb - 1) / B : start) + (int)blockIdx.x;
  if (j >= nb || j * B >= Lb) return;  // uniform
  head_landmark_chunk<NL>(K, W, LK, L, Lb, B, nb, Hkv, j, blockIdx.y, threadIdx.x / kWave, 4);
}

// Workgroup (x, y): 128 landmark rows (chunk j, landmark l: row j*NL + l) of
// kv head g against 64 (query, head) columns of sequence b, y = (b * Hkv +
// g) * ctiles + column tile.  Column p is query p / QPG, head g*QPG + p % QPG.
// Wave w takes rows 32w .. 32w+31 (two 16-row B operands) for all 64
// columns (four 16-column A operands); the accumulator holds 4 columns x 1
// row per lane; a chunk's NL landmark rows sit in adjacent lanes, reduced by
// an xor-shuffle maximum.
template <int NL>
__global__ __launch_bounds__(256) void k_head_scores_mfma(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ LK,
                                                          float* __restrict__ scores, int L, int nq, int B, int nb,
                                                          int m, int Hq, int Hkv, int ctiles,
                                                          const int32_t* __restrict__ lens) {
  constexpr int DI = 128, KS = DI / 32;
  const int QPG = Hq / Hkv;
  const int ncols = nq * QPG;
  const int bg = blockIdx.y / ctiles, ct = blockIdx.y % ctiles;
  const int b = bg / Hkv, g = bg % Hkv;
  const int Lb = seq_len_of(lens, L, b);
  const int col0 = ct * 64;
  const int c_last = query_pos(Lb, nq, (min(ncols, col0 + 64) - 1) / QPG) / B;
  if (c_last + 1 <= m) return;  // no query of the tile needs scores
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int jl = lane & 15, gq = lane >> 4;
  const int row0 = blockIdx.x * 128 + wave * 32;
  if (row0 / NL >= c_last) return;  // every chunk is non-causal or forced
  const int nrows = nb * NL;

  u32x4 bs[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = min(row0 + 16 * nt + jl, nrows - 1);
    const uint16_t* src = LK + (((size_t)b * nrows + row) * Hkv + g) * DI + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bs[nt][ks] = *reinterpret_cast<const u32x4*>(src + 32 * ks);
  }
  for (int mt = 0; mt < 4; ++mt) {
    if (col0 + 16 * mt >= ncols) break;  // uniform
    const int ca = min(col0 + 16 * mt + jl, ncols - 1);
    const uint16_t* qsrc = Q + (((size_t)b * nq + ca / QPG) * Hq + g * QPG + ca % QPG) * DI + 8 * gq;
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
      if constexpr (NL > 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = group_max_f<NL>(acc[e]);
      }
      const int row = row0 + 16 * nt + jl;
      const int j = row / NL;
      if (row % NL == 0 && row < nrows) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = col0 + 16 * mt + 4 * gq + e;
          if (col >= ncols) continue;
          const int i = col / QPG;
          const int c = query_pos(Lb, nq, i) / B;
          if (c + 1 > m && j >= 1 && j < c)
            scores[(((size_t)b * nq + i) * Hq + g * QPG + col % QPG) * nb + j] = acc[e];
        }
      }
    }
  }
}

// The select of the per-head rows (sequence, query, head), one row per
// group of NW waves (NW == 1: four rows per workgroup, one per wave): the
// exact top-(m-2) of chunks 1..c-1 by score with chunks 0 and c kept
// (select_top), the chunk list written ascending and -1 padded, then the
// row's token list written by the whole group from the list kept in LDS:
// entry e is token s = list[e / B] * B + e % B if s <= t, stored as
// s * Hkv + g (g = head / QPG), else -1.  The first nfold_wg workgroups
// instead rebuild the landmarks of chunks fold_start .. of each sequence
// when the host folds them in (no row of this launch reads landmarks, and
// the score launch before it read none of those chunks).
constexpr int kHeadListMax = 1024;  // chunk lists staged in LDS

template <int NW, int R>
__global__ __launch_bounds__(NW == 1 ? 256 : NW * 64) void k_head_select(
    const float* __restrict__ scores, int32_t* __restrict__ blk, int32_t* __restrict__ tok, int L, int nq, int B,
    int nb, int m, int Hq, int Hkv, int rows, int nfold_wg, const uint16_t* __restrict__ K,
    const int8_t* __restrict__ W, uint16_t* __restrict__ LK_out, int NL, int fold_start, int nfold,
    const int32_t* __restrict__ lens, bool vec) {
  constexpr int QPB = NW == 1 ? 4 : 1;  // rows per workgroup
  constexpr int GT = NW * kWave;        // threads per row
  __shared__ SelectSmem<NW> lds[QPB];
  __shared__ int32_t list[QPB][kHeadListMax];
  const int wave = threadIdx.x / kWave;
  if ((int)blockIdx.x < nfold_wg) {  // folded landmarks (uniform)
    const int bs = (int)blockIdx.x / nfold;
    const int Lb = seq_len_of(lens, L, bs);
    // per-sequence lengths (one query each): the chunk of the sequence's query
    const int j = (lens ? (Lb - 1) / B : fold_start) + (int)blockIdx.x % nfold;
    if (j >= nb || j * B >= Lb) return;
    const int nw = blockDim.x / kWave;
    if (NL == 1) head_landmark_chunk<1, 2>(K, W, LK_out, L, Lb, B, nb, Hkv, j, bs, wave, nw);
    else if (NL == 2) head_landmark_chunk<2, 2>(K, W, LK_out, L, Lb, B, nb, Hkv, j, bs, wave, nw);
    else head_landmark_chunk<4, 2>(K, W, LK_out, L, Lb, B, nb, Hkv, j, bs, wave, nw);
    return;
  }
  const int wg = (int)blockIdx.x - nfold_wg;
  const int q = NW == 1 ? wg * 4 + wave : wg;
  if (q >= rows) return;  // wave-uniform (NW == 1 only)
  SelectSmem<NW>& sm = lds[NW == 1 ? wave : 0];
  int32_t* lst = list[NW == 1 ? wave : 0];
  const int gtid = NW == 1 ? lane_id() : (int)threadIdx.x;
  const int qpg = Hq / Hkv;
  const int g = (q % Hq) / qpg;
  const int t = query_pos(seq_len_of(lens, L, q / (Hq * nq)), nq, (q / Hq) % nq);
  const int c = t / B;
  int32_t* out = blk + (size_t)q * m;
  int32_t* tq = tok ? tok + (size_t)q * m * B : nullptr;
  if (c + 1 <= m) {
    for (int j = gtid; j < m; j += GT) out[j] = j <= c ? j : -1;
    if (tq)
      for (int e = gtid; e < m * B; e += GT) tq[e] = e <= t ? e * Hkv + g : -1;
    return;
  }
  const int want = m - 2;
  const int n = c - 1;  // candidates: chunks 1 .. c-1 (index = chunk - 1)
  const bool staged = m <= kHeadListMax;
  if (gtid == 0) {
    out[0] = 0;
    out[m - 1] = c;
    if (staged) {
      lst[0] = 0;
      lst[m - 1] = c;
    }
  }
  if (want > 0) {
    uint32_t key[R];
    int off = 1;  // chunk of select slot s: s + off
    bool loaded = false;
    if constexpr (R >= 4) {
      if (vec) {  // (uniform) aligned rows: slot = chunk, R/4 16-byte loads per thread
        const float* sc = scores + (size_t)q * nb;
#pragma unroll
        for (int r = 0; r < R; r += 4) {
          const int j0 = gtid * R + r;
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
          if (j0 < nb) v = *reinterpret_cast<const f32x4*>(sc + j0);
#pragma unroll
          for (int e = 0; e < 4; ++e) key[r + e] = (j0 + e >= 1 && j0 + e <= n) ? score_key(v[e]) : 0u;
        }
        off = 0;
        loaded = true;
      }
    }
    if (!loaded) {
      const float* sc = scores + (size_t)q * nb + 1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = gtid * R + r;
        const float v = sc[idx < n ? idx : 0];  // branch-free: all loads in flight together
        key[r] = idx < n ? score_key(v) : 0u;
      }
    }
    // the group synchronises after the select anyway (below) before the
    // staged list is read, so the select's own closing barrier is not needed
    select_top<NW, R, false>(key, want, sm, [&](int pos, int idx, bool take, uint32_t) {
      if (!take) return;
      const int chunk = idx + off;
      out[1 + pos] = chunk;
      if (staged) {
        lst[1 + pos] = chunk;
      } else if (tq) {  // lists too long for LDS: each kept chunk's tokens from its thread
        for (int r = 0; r < B; ++r) tq[(size_t)(1 + pos) * B + r] = (chunk * B + r) * Hkv + g;
      }
    });
  }
  if (!tq) return;
  sel_sync<NW>();
  if (staged) {
    // 4 consecutive entries share a chunk (B is a multiple of 4)
    for (int e = gtid * 4; e < m * B; e += GT * 4) {
      const int s0 = lst[e / B] * B + e % B;
      i32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = s0 + k <= t ? (s0 + k) * Hkv + g : -1;
      *reinterpret_cast<i32x4*>(tq + e) = v;
    }
  } else {
    for (int e = gtid; e < B; e += GT) {  // the two forced chunks
      tq[e] = e * Hkv + g;
      const int s = c * B + e;
      tq[(size_t)(m - 1) * B + e] = s <= t ? s * Hkv + g : -1;
    }
  }
}

size_t head_scores_ws_bytes(const Dims& s) { return align_up((size_t)s.b * s.nq * s.Hq * s.nb * sizeof(float)); }

hipError_t launch_head_landmarks(const Dims& s, const uint16_t* K, const int8_t* W, int start, uint16_t* LK,
                                 hipStream_t st) {
  if (s.b == 0 || (!s.lens && start >= s.nb)) return hipSuccess;
  // per-sequence lengths: the chunks the new queries touch (one query: one)
  dim3 grid(s.lens ? (s.nq + s.B - 1) / s.B : s.nb - start, s.b);
  switch (s.nL) {
    case 1: HSA_LAUNCH((k_head_landmarks<1>), grid, dim3(256), 0, st, K, W, LK, s.L, s.B, s.nb, s.Hkv, start, s.lens); break;
    case 2: HSA_LAUNCH((k_head_landmarks<2>), grid, dim3(256), 0, st, K, W, LK, s.L, s.B, s.nb, s.Hkv, start, s.lens); break;
    case 4: HSA_LAUNCH((k_head_landmarks<4>), grid, dim3(256), 0, st, K, W, LK, s.L, s.B, s.nb, s.Hkv, start, s.lens); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool head_topm_can_fold(const Dims& s, int start_block) {
  // the rebuilt chunks start at the last one, which no query scores (a
  // query scores chunks below its own); with per-sequence lengths (one
  // query each) the rebuilt chunk is each sequence's own
  if (s.lens) return s.nq == 1;
  const int c_max = (s.L - 1) / s.B;
  return start_block >= c_max && start_block < s.nb;
}

template <int NW, int R>
static hipError_t launch_head_select_r(const Dims& s, const float* scores, int32_t* blk, int32_t* tok,
                                       const HeadFold* fold, hipStream_t st) {
  const int rows = s.b * s.nq * s.Hq;
  const int nfold = fold ? (s.lens ? 1 : s.nb - fold->start_block) : 0;
  const int nfold_wg = s.b * nfold;
  dim3 grid(nfold_wg + (NW == 1 ? (rows + 3) / 4 : rows)), block(NW == 1 ? 256 : NW * 64);
  // chunk-number slots need nb % 4 == 0 (aligned rows) and slots for chunks
  // 0 .. c_max - 1 of the latest query
  const int c_max = (s.L - 1) / s.B;
  const bool vec = R >= 4 && s.nb % 4 == 0 && (long long)NW * kWave * R >= c_max;
  HSA_LAUNCH((k_head_select<NW, R>), grid, block, 0, st, scores, blk, tok, s.L, s.nq, s.B, s.nb, s.m, s.Hq,
                     s.Hkv, rows, nfold_wg, fold ? fold->K : nullptr, fold ? fold->W : nullptr,
                     fold ? fold->LK : nullptr, s.nL, fold ? fold->start_block : s.nb, max(nfold, 1), s.lens, vec);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_head_select(int R, const Dims& s, const float* scores, int32_t* blk, int32_t* tok,
                                     const HeadFold* fold, hipStream_t st) {
  switch (R) {
    case 1: return launch_head_select_r<NW, 1>(s, scores, blk, tok, fold, st);
    case 2: return launch_head_select_r<NW, 2>(s, scores, blk, tok, fold, st);
    case 4: return launch_head_select_r<NW, 4>(s, scores, blk, tok, fold, st);
    case 8: return launch_head_select_r<NW, 8>(s, scores, blk, tok, fold, st);
    case 16: return launch_head_select_r<NW, 16>(s, scores, blk, tok, fold, st);
    case 32:
      if constexpr (NW > 1) return launch_head_select_r<NW, 32>(s, scores, blk, tok, fold, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

static int pick_r(int n, int nw) {
  int r = 1;
  while (r * 64 * nw < n) r <<= 1;
  return r;
}

hipError_t launch_head_topm(const Dims& s, const uint16_t* Q, const uint16_t* LK, int32_t* blk, void* ws,
                            hipStream_t st, int32_t* tok, const HeadFold* fold) {
  if (s.b == 0 || s.nq == 0) return hipSuccess;
  float* scores = static_cast<float*>(ws);
  const int c_max = (s.L - 1) / s.B;
  if (c_max + 1 > s.m) {
    const int ctiles = (s.nq * (s.Hq / s.Hkv) + 63) / 64;
    dim3 grid((s.nb * s.nL + 127) / 128, s.b * s.Hkv * ctiles);
#define HSA_HS(NL)                                                                                               \
  HSA_LAUNCH((k_head_scores_mfma<NL>), grid, dim3(256), 0, st, Q, LK, scores, s.L, s.nq, s.B, s.nb, s.m, \
             s.Hq, s.Hkv, ctiles, s.lens)
    if (s.nL == 1) HSA_HS(1); else if (s.nL == 2) HSA_HS(2); else HSA_HS(4);
#undef HSA_HS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // many rows: one wave per row (<= 512 candidates) or 4 waves per row;
  // few rows: 16 waves per row (shortest latency)
  const int rows = s.b * s.nq * s.Hq;
  const int n_max = c_max - 1;
  if (rows >= 512 && n_max <= 64 * 8) return launch_head_select<1>(pick_r(n_max, 1), s, scores, blk, tok, fold, st);
  if (rows >= 512 && n_max <= 4 * 64 * 32)
    return launch_head_select<4>(pick_r(n_max, 4), s, scores, blk, tok, fold, st);
  return launch_head_select<16>(pick_r(n_max, 16), s, scores, blk, tok, fold, st);
}

// The attention of the per-head lists: each (query, head) row is a one-head
// query over K and V viewed as [L * Hkv, 1, d].
static Dims attn_view(const Dims& s) {
  Dims v = s;
  v.nq = s.nq * s.Hq;
  v.Hq = 1;
  v.Hkv = 1;
  v.L = s.L * s.Hkv;
  v.k = s.m * s.B;
  v.lens = nullptr;  // the lists hold causal tokens only (as rows s * Hkv + g)
  return v;
}

size_t head_attn_ws_bytes(const Dims& s) { return sparse_attn_ws_bytes(attn_view(s)); }

hipError_t launch_head_attn(const Dims& s, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                            const int32_t* tok, float* O, float* lse, void* ws, hipStream_t st) {
  if (s.b == 0 || s.nq == 0) return hipSuccess;
  return launch_sparse_attn(attn_view(s), Q, K, V, tok, O, lse, ws, st);
}

}  // namespace hsa
