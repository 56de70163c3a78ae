// Host-side launchers of the library's kernels.  Each takes validated
// arguments (see api.cpp) and only enqueues work on `stream`.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hsa_sparse.h"

namespace hsa {

// Per-kernel timing (hsa_sparse_set_kernel_events): the start and stop
// events the next kernel of the current call records with its dispatch
// (both nullptr when not recording), and its name appended to the call's
// kernel list.
void kernel_slot(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Score buffers larger than the 256 MB last-level cache (MALL) are written
// with non-temporal stores: they are read back only once the whole buffer
// is written, so caching them on the way only evicts the rows the scorer
// itself re-reads.  (Smaller buffers stay cached for the select that
// follows.)
constexpr size_t kStreamStoreBytes = size_t(256) << 20;

// Every kernel of the library is launched through this: with recording on,
// the dispatch itself carries the kernel's start and stop events
// (hipExtLaunchKernelGGL), so timing a kernel adds no work to the stream.
#define HSA_LAUNCH(KERNEL, GRID, BLOCK, LDS, ST, ...)                                                      \
  do {                                                                                                     \
    hipEvent_t hsa_ev0_, hsa_ev1_;                                                                         \
    ::hsa::kernel_slot(#KERNEL, &hsa_ev0_, &hsa_ev1_);                                                     \
    if (hsa_ev0_ || hsa_ev1_)                                                                              \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, hsa_ev0_, hsa_ev1_, 0, __VA_ARGS__);             \
    else                                                                                                   \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, ST, __VA_ARGS__);                                       \
  } while (0)

struct Dims {
  int b, L, nq, dI, B, nL, m, k, Hq, Hkv, d;
  float scale;
  int nb;  // ceil(L / B)
  // device [b]: current length of each sequence (decode over a batch of
  // different lengths, n_q == 1); nullptr: every sequence has length L.
  // L stays the capacity and row stride.
  const int32_t* lens = nullptr;
};

// step 1
hipError_t launch_block_summary(const Dims& s, const uint16_t* kI, const int8_t* W, int start_block,
                                uint16_t* S, hipStream_t st);

// step 2: scores into `scores` [b*nq, nb] fp32, then the top-m select.
// With `fold`, the score kernel also summarises blocks fold->start_block ..
// nb-1 (allowed only when block_topm_can_fold says no query scores them).
struct SummaryFold {
  const uint16_t* kI;
  const int8_t* W;
  uint16_t* S;
  int start_block;
};
size_t block_topm_ws_bytes(const Dims& s);
bool block_topm_can_fold(const Dims& s, int start_block);
hipError_t launch_block_topm(const Dims& s, const uint16_t* qI, const uint16_t* S, int32_t* blk,
                             void* ws, hipStream_t st, const SummaryFold* fold = nullptr);

// step 2's block-score contraction without the selection (a measurement
// aid): out[q] = the highest score over query q's scored blocks 1..c-1
// (-inf when it scores none), in one MFMA launch that writes 4 bytes per
// query (per summary-tile chunk when there are few queries, then reduced).
size_t block_score_max_ws_bytes(const Dims& s);
hipError_t launch_block_score_max(const Dims& s, const uint16_t* qI, const uint16_t* S, float* out, void* ws,
                                  hipStream_t st);

// step 2 through super-blocks of 2^lgG blocks: S2 summaries of the
// super-blocks from start_super on, then level 1 (top-m2 super-blocks into
// sup [b*nq, m2]) and level 2 (top-m blocks among theirs into blk)
hipError_t launch_super_summary(const Dims& s, int lgG, const uint16_t* S, int start_super, uint16_t* S2,
                                hipStream_t st);
// With `fold`, the newest block's summary and its super-block's (into
// S2_out) are rebuilt inside the selection launch; allowed only when
// block_topm_3level_can_fold says no query reads them.
size_t block_topm_3level_ws_bytes(const Dims& s, int lgG);
bool block_topm_3level_can_fold(const Dims& s, int lgG, int m2, int start_block);
hipError_t launch_block_topm_3level(const Dims& s, int lgG, int m2, const uint16_t* qI, const uint16_t* S,
                                    const uint16_t* S2, int32_t* sup, int32_t* blk, void* ws, hipStream_t st,
                                    const SummaryFold* fold = nullptr, uint16_t* S2_out = nullptr);

// steps 2 and 3's scores for few queries (decode): the block lists and the
// token scores of launch_token_scores in one launch (with the summary fold
// as in launch_block_topm), only where block_token_fusable holds
bool block_token_fusable(const Dims& s, const SummaryFold* fold);
hipError_t launch_block_token_decode(const Dims& s, const uint16_t* qI, const uint16_t* S, const uint16_t* kI,
                                     int32_t* blk, float* scores, hipStream_t st, const SummaryFold* fold);

// step 3: scores into [b*nq, m*B] fp32, then the top-k select
size_t token_topk_ws_bytes(const Dims& s);
hipError_t launch_token_topk(const Dims& s, const uint16_t* qI, const uint16_t* kI, const int32_t* blk,
                             int32_t* tok, void* ws, hipStream_t st);

// step 4
size_t sparse_attn_ws_bytes(const Dims& s);
hipError_t launch_sparse_attn(const Dims& s, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                              const int32_t* tok, float* O, float* lse, void* ws, hipStream_t st);

// steps 3 and 4 for few queries (decode): the scorer alone
// (launch_token_scores, into the first token_topk_ws_bytes of ws; nothing
// when no query scores), then the select and the attention in one launch
// plus the merge (launch_select_attn: scores as written by the scorer, the
// attention partials in the next sparse_attn_ws_bytes).  Only for shapes
// where select_attn_fusable holds; same lists and outputs, bit for bit, as
// launch_token_topk + launch_sparse_attn.
hipError_t launch_token_scores(const Dims& s, const uint16_t* qI, const uint16_t* kI, const int32_t* blk, void* ws,
                               hipStream_t st);
bool select_attn_fusable(const Dims& s);
size_t select_attn_ws_bytes(const Dims& s);
hipError_t launch_select_attn(const Dims& s, const float* scores, const int32_t* blk, int32_t* tok, const uint16_t* Q,
                              const uint16_t* K, const uint16_t* V, float* O, float* lse, void* ws, hipStream_t st);

// the flat indexer (every causal token scored), the baseline of step 3
bool flat_topk_supported(const Dims& s);
size_t flat_topk_ws_bytes(const Dims& s);
hipError_t launch_flat_topk(const Dims& s, const uint16_t* qI, const uint16_t* kI, int32_t* tok, void* ws,
                            hipStream_t st);

// per-head selection from the attention queries: landmarks of K per kv
// head (LK [b, nb, nL, Hkv, 128]), per-(query, head) chunk top-m (scores
// [b*nq*Hq, nb] fp32 in ws), then the per-head lists' attention (token
// lists [b*nq*Hq, m*B] in tok)
hipError_t launch_head_landmarks(const Dims& s, const uint16_t* K, const int8_t* W, int start, uint16_t* LK,
                                 hipStream_t st);
size_t head_scores_ws_bytes(const Dims& s);
// With `fold` the landmarks of chunks fold->start_block .. are rebuilt in
// the select launch (only when head_topm_can_fold).  tok: the per-head token
// lists for launch_head_attn, written by the select (nullptr: none).
struct HeadFold {
  const uint16_t* K;
  const int8_t* W;
  uint16_t* LK;
  int start_block;
};
bool head_topm_can_fold(const Dims& s, int start_block);
hipError_t launch_head_topm(const Dims& s, const uint16_t* Q, const uint16_t* LK, int32_t* blk, void* ws,
                            hipStream_t st, int32_t* tok, const HeadFold* fold = nullptr);
size_t head_attn_ws_bytes(const Dims& s);
hipError_t launch_head_attn(const Dims& s, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                            const int32_t* tok, float* O, float* lse, void* ws, hipStream_t st);

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

}  // namespace hsa
