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
// order is token order.
//
// Kernel 1 (k_token_scores): one workgroup per (query, list entry) streams
// that block's kI rows (d_index/8 lanes per row, 16-byte loads) and writes
// the fp32 scores of its slots to the workspace.
// Kernel 2 (k_token_select): one workgroup per query; when n_valid <= k all
// candidates are written, otherwise the exact select of select.hpp runs over
// the slot scores.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace hsa {

__device__ __forceinline__ void candidate_count(int t, int B, int m, int& c, int& n_sel, int& n_valid) {
  c = t / B;
  n_sel = (c + 1 <= m) ? c + 1 : m;
  n_valid = (n_sel - 1) * B + (t - c * B + 1);
}

template <int DI>
__global__ __launch_bounds__(256) void k_token_scores(const uint16_t* __restrict__ qI,
                                                      const uint16_t* __restrict__ kI,
                                                      const int32_t* __restrict__ blk, float* __restrict__ scores,
                                                      int L, int nq, int B, int m, int k) {
  constexpr int LPR = DI / 8;
  constexpr int RPI = 256 / LPR;  // rows per workgroup iteration
  const int p = blockIdx.x;
  const int q = blockIdx.y;
  const int b = q / nq, i = q % nq;
  const int t = query_pos(L, nq, i);
  int c, n_sel, n_valid;
  candidate_count(t, B, m, c, n_sel, n_valid);
  if (n_valid <= k || p >= n_sel) return;
  const int j = blk[(size_t)q * m + p];

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
  for (int r0 = 0; r0 < B; r0 += RPI) {
    const int r = r0 + tid / LPR;
    float dot = 0.f;
    if (r < rows) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(kb + (size_t)r * DI + col8 * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += qv[2 * e] * bf16_lo(v[e]);
        dot += qv[2 * e + 1] * bf16_hi(v[e]);
      }
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) dot += shfl_xor(dot, o);
    if (r < rows && col8 == 0) out[r] = dot;
  }
}

template <int NW, int R>
__global__ __launch_bounds__(NW * 64) void k_token_select(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ blk, int32_t* __restrict__ tok,
                                                          int L, int nq, int B, int m, int k) {
  __shared__ int lds[select_lds_words<NW>()];
  const int q = blockIdx.x;
  const int i = q % nq;
  const int t = query_pos(L, nq, i);
  int c, n_sel, n_valid;
  candidate_count(t, B, m, c, n_sel, n_valid);
  const int32_t* bl = blk + (size_t)q * m;
  int32_t* out = tok + (size_t)q * k;
  if (n_valid <= k) {
    for (int slot = threadIdx.x; slot < k; slot += NW * 64)
      out[slot] = slot < n_valid ? bl[slot / B] * B + slot % B : -1;
    return;
  }
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const float* sc = scores + (size_t)q * m * B;
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = wave * kWave * R + r * kWave + lane;
    key[r] = idx < n_valid ? score_key(sc[idx]) : 0u;
  }
  select_top<NW, R>(key, k, lds, [&](int pos, int idx) { out[pos] = bl[idx / B] * B + idx % B; });
}

size_t token_topk_ws_bytes(const Dims& s) {
  if ((long long)s.k >= (long long)s.m * s.B) return 0;
  return align_up((size_t)s.b * s.nq * s.m * s.B * sizeof(float));
}

template <int NW>
static hipError_t launch_tsel(int R, const Dims& s, const float* sc, const int32_t* blk, int32_t* tok, hipStream_t st) {
  dim3 grid(s.b * s.nq), block(NW * 64);
#define HSA_TS(RR)                                                                                          \
  case RR:                                                                                                  \
    hipLaunchKernelGGL((k_token_select<NW, RR>), grid, block, 0, st, sc, blk, tok, s.L, s.nq, s.B, s.m, s.k); \
    break;
  switch (R) {
    HSA_TS(1) HSA_TS(2) HSA_TS(4) HSA_TS(8) HSA_TS(16) HSA_TS(32) HSA_TS(64)
    default: return hipErrorInvalidValue;
  }
#undef HSA_TS
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
    dim3 grid(s.m, nq_total);
    if (s.dI == 64)
      hipLaunchKernelGGL((k_token_scores<64>), grid, dim3(256), 0, st, qI, kI, blk, scores, s.L, s.nq, s.B, s.m, s.k);
    else
      hipLaunchKernelGGL((k_token_scores<128>), grid, dim3(256), 0, st, qI, kI, blk, scores, s.L, s.nq, s.B, s.m, s.k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    n_max = 1;  // every query keeps all of its candidates
  }
  if (nq_total >= 512 && n_max <= 4 * 64 * 64) {
    int r = 1;
    while (r * 256 < n_max) r <<= 1;
    return launch_tsel<4>(r, s, scores, blk, tok, st);
  }
  int r = 1;
  while (r * 1024 < n_max) r <<= 1;
  if (r > 32) return hipErrorInvalidValue;
  return launch_tsel<16>(r, s, scores, blk, tok, st);
}

}  // namespace hsa
