// Step 1: block summaries.
//
// HISA page (two-step method, step one): every fixed-size block of B
// indexer keys gets one summary vector; read here as the block mean.  HiLS
// page (section 2.1): a chunk is represented by a few landmark vectors made
// by a projection of its tokens; here landmark l = sum_r W[l, r] kI[r] / B.
//
// One workgroup per (sequence, block).  The block's B rows (d_index bf16
// each, 128 or 256 bytes) are streamed once with 16-byte loads; a row is
// covered by d_index/8 consecutive lanes, so every load instruction reads
// whole rows.  Per-thread fp32 partial sums meet in LDS, are scaled by the
// exact power of two 1/B and rounded once to bf16 (nearest even).
// HBM-bound: B * d_index * 2 bytes read per nL * d_index * 2 bytes written.
#include "common.hpp"
#include "kernels.hpp"

namespace hsa {

template <int DI, int NL>
__global__ __launch_bounds__(256) void k_block_summary(const uint16_t* __restrict__ kI,
                                                       const int8_t* __restrict__ W, uint16_t* __restrict__ S,
                                                       int L, int B, int nb, int start_block) {
  constexpr int LPR = DI / 8;       // lanes per row
  constexpr int RPI = 256 / LPR;    // rows per iteration of the workgroup
  __shared__ float red[NL][RPI][DI];

  const int j = start_block + blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int col8 = tid % LPR;
  const int r0 = tid / LPR;

  float acc[NL][8];
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;

  const size_t seq_base = (size_t)b * L;
  for (int r = r0; r < B; r += RPI) {
    const int s = j * B + r;
    if (s >= L) break;
    const u32x4 v = *reinterpret_cast<const u32x4*>(kI + (seq_base + s) * DI + col8 * 8);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(v[e]);
      x[2 * e + 1] = bf16_hi(v[e]);
    }
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const float w = W ? (float)W[l * B + r] : 1.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[l][e] += w * x[e];
    }
  }
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[l][r0][col8 * 8 + e] = acc[l][e];
  __syncthreads();

  const float inv_b = 1.f / (float)B;  // exact: B is a power of two
  for (int o = tid; o < NL * DI; o += 256) {
    const int l = o / DI, d = o % DI;
    float total = 0.f;
#pragma unroll 4
    for (int r = 0; r < RPI; ++r) total += red[l][r][d];
    S[(((size_t)b * nb + j) * NL + l) * DI + d] = (uint16_t)f32_to_bf16_rne(total * inv_b);
  }
}

template <int DI>
static hipError_t launch_di(const Dims& s, const uint16_t* kI, const int8_t* W, int start, uint16_t* S,
                            hipStream_t st) {
  dim3 grid(s.nb - start, s.b);
  switch (s.nL) {
    case 1: hipLaunchKernelGGL((k_block_summary<DI, 1>), grid, dim3(256), 0, st, kI, W, S, s.L, s.B, s.nb, start); break;
    case 2: hipLaunchKernelGGL((k_block_summary<DI, 2>), grid, dim3(256), 0, st, kI, W, S, s.L, s.B, s.nb, start); break;
    case 4: hipLaunchKernelGGL((k_block_summary<DI, 4>), grid, dim3(256), 0, st, kI, W, S, s.L, s.B, s.nb, start); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_block_summary(const Dims& s, const uint16_t* kI, const int8_t* W, int start_block, uint16_t* S,
                                hipStream_t st) {
  if (start_block >= s.nb || s.b == 0) return hipSuccess;
  return s.dI == 64 ? launch_di<64>(s, kI, W, start_block, S, st) : launch_di<128>(s, kI, W, start_block, S, st);
}

}  // namespace hsa
