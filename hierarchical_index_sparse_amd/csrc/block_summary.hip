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
#include "summary.hpp"

namespace hsa {

// Workgroup (x, b) summarises block start + x of sequence b.  With
// per-sequence lengths, start is the block of sequence b's first new query,
// (Lb - nq) / B, and blocks at or past ceil(Lb / B) are skipped.
template <int DI, int NL>
__global__ __launch_bounds__(256) void k_block_summary(const uint16_t* __restrict__ kI,
                                                       const int8_t* __restrict__ W, uint16_t* __restrict__ S,
                                                       int L, int B, int nb, int start_block,
                                                       const int32_t* __restrict__ lens, int nq) {
  __shared__ float red[NL][256 / (DI / 8)][DI];
  const int b = blockIdx.y;
  const int Lb = seq_len_of(lens, L, b);
  const int j = (lens ? (Lb - nq) / B : start_block) + (int)blockIdx.x;
  if (j >= nb || j * B >= Lb) return;  // uniform
  summarise_block<DI, NL>(kI, W, S, L, Lb, B, nb, j, b, red);
}

template <int DI>
static hipError_t launch_di(const Dims& s, const uint16_t* kI, const int8_t* W, int start, uint16_t* S,
                            hipStream_t st) {
  // blocks the new queries touch: at most ceil(nq / B) + 1 per sequence
  dim3 grid(s.lens ? (s.nq + s.B - 1) / s.B + 1 : s.nb - start, s.b);
  switch (s.nL) {
    case 1: HSA_LAUNCH((k_block_summary<DI, 1>), grid, dim3(256), 0, st, kI, W, S, s.L, s.B, s.nb, start, s.lens, s.nq); break;
    case 2: HSA_LAUNCH((k_block_summary<DI, 2>), grid, dim3(256), 0, st, kI, W, S, s.L, s.B, s.nb, start, s.lens, s.nq); break;
    case 4: HSA_LAUNCH((k_block_summary<DI, 4>), grid, dim3(256), 0, st, kI, W, S, s.L, s.B, s.nb, start, s.lens, s.nq); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_block_summary(const Dims& s, const uint16_t* kI, const int8_t* W, int start_block, uint16_t* S,
                                hipStream_t st) {
  if (s.b == 0 || (!s.lens && start_block >= s.nb)) return hipSuccess;
  return s.dI == 64 ? launch_di<64>(s, kI, W, start_block, S, st) : launch_di<128>(s, kI, W, start_block, S, st);
}

}  // namespace hsa
