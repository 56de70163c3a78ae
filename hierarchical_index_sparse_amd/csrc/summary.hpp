// Summary of one key block (step 1), shared by the summary kernel and the
// decode block-score kernel that folds the newest block's summary in.
//
// HISA page (two-step method, step one): one summary vector per block,
// read here as the block mean; HiLS page (section 2.1): landmark l =
// sum_r W[l, r] kI[r] / B.  The block's B rows (d_index bf16 each) are read
// once with 16-byte loads, d_index/8 lanes per row; per-thread fp32 partial
// sums meet in LDS, are scaled by the exact power of two 1/B and rounded
// once to bf16 (nearest even).  Rows beyond L count as zero.
#pragma once

#include "common.hpp"

namespace hsa {

// Called by all NTH threads of a workgroup; red is the workgroup's LDS.
// L is the row stride of kI per sequence, Lb the sequence's length (rows
// at or past Lb count as zero).  With S2, the summary of the super-block of
// 2^lgG blocks holding block j is rebuilt too: the mean of its blocks'
// summaries (block j's fresh value, the others read from S; blocks past the
// sequence's last block, ceil(Lb / B) - 1, count as zero), summed in block
// order in fp32 and rounded once, the same arithmetic as the super-block
// summary kernel.  No other workgroup may be writing that super-block's
// blocks in S.
template <int DI, int NL, int NTH = 256>
__device__ __forceinline__ void summarise_block(const uint16_t* __restrict__ kI, const int8_t* __restrict__ W,
                                                uint16_t* __restrict__ S, int L, int Lb, int B, int nb, int j, int b,
                                                float (&red)[NL][NTH / (DI / 8)][DI],
                                                uint16_t* __restrict__ S2 = nullptr, int lgG = 0) {
  constexpr int LPR = DI / 8;     // lanes per row
  constexpr int RPI = NTH / LPR;  // rows per iteration of the workgroup
  const int tid = threadIdx.x;
  const int col8 = tid % LPR;
  const int r0 = tid / LPR;

  float acc[NL][8];
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;

  // every row load (and projection weight) of the thread is issued before
  // any is used: a block is at most 128 rows, NIT rounds of RPI rows
  constexpr int NIT = (128 + RPI - 1) / RPI;
  const size_t seq_base = (size_t)b * L;
  u32x4 v[NIT];
  float wl[NL][NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + it * RPI;
    const bool ok = r < B && j * B + r < Lb;
    v[it] = u32x4{0u, 0u, 0u, 0u};
    if (ok) v[it] = *reinterpret_cast<const u32x4*>(kI + (seq_base + j * B + r) * DI + col8 * 8);
#pragma unroll
    for (int l = 0; l < NL; ++l) wl[l][it] = ok ? (W ? (float)W[l * B + r] : 1.f) : 0.f;
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(v[it][e]);
      x[2 * e + 1] = bf16_hi(v[it][e]);
    }
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[l][e] += wl[l][it] * x[e];
  }
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[l][r0][col8 * 8 + e] = acc[l][e];
  __syncthreads();

  const float inv_b = 1.f / (float)B;  // exact: B is a power of two
  for (int o = tid; o < NL * DI; o += NTH) {
    const int l = o / DI, d = o % DI;
    float total = 0.f;
#pragma unroll 4
    for (int r = 0; r < RPI; ++r) total += red[l][r][d];
    const uint32_t own = f32_to_bf16_rne(total * inv_b);
    S[(((size_t)b * nb + j) * NL + l) * DI + d] = (uint16_t)own;
    if (S2) {
      const int J = j >> lgG, g0 = J << lgG, g1 = min((Lb + B - 1) / B, g0 + (1 << lgG));
      const int nsb = (nb + (1 << lgG) - 1) >> lgG;
      float sum = 0.f;
      for (int g = g0; g < g1; ++g) {
        const uint32_t v = g == j ? own : (uint32_t)S[(((size_t)b * nb + g) * NL + l) * DI + d];
        sum += __uint_as_float(v << 16);
      }
      S2[(((size_t)b * nsb + J) * NL + l) * DI + d] = (uint16_t)f32_to_bf16_rne(sum * __builtin_ldexpf(1.f, -lgG));
    }
  }
}

}  // namespace hsa
