// Device-side helpers shared by the kernels of the library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hsa_sparse.h"

namespace hsa {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int32_t)))) int32_t i32x4;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even on the bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map of an fp32 score to uint32: a larger score gives a
// larger key; -0 and +0 give the same key.  Key 0 is never produced by a
// finite score and marks an empty slot.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// ---- cross-lane reductions and scans without LDS (DPP and gfx950's row
// swaps).  group_reduce<G>(x, op) combines x over every aligned group of G
// lanes (G a power of two <= 64) and gives every lane of the group the
// result; op must be commutative and associative.
namespace dpp {
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kHalfMirror = 0x141;  // lane i <-> 7 - i inside each 8-lane half row
constexpr int kMirror = 0x140;      // lane i <-> 15 - i inside each 16-lane row
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;  // row_shr:n
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
template <int G, typename Op>
__device__ __forceinline__ uint32_t group_reduce(uint32_t x, Op op) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G must be a power of two <= 64");
  if constexpr (G >= 2) x = op(x, dpp_mov<dpp::kQuadSwap1>(x));
  if constexpr (G >= 4) x = op(x, dpp_mov<dpp::kQuadSwap2>(x));
  if constexpr (G >= 8) x = op(x, dpp_mov<dpp::kHalfMirror>(x));
  if constexpr (G >= 16) x = op(x, dpp_mov<dpp::kMirror>(x));
  if constexpr (G >= 32) {
    // rows 0<->1 and 2<->3: the pair returned holds this lane's value and
    // its partner's in some order; op is symmetric, so combine both
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = op(r[0], r[1]);
  }
  if constexpr (G >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = op(r[0], r[1]);
  }
  return x;
}
template <int G>
__device__ __forceinline__ float group_sum_f(float v) {
  return __uint_as_float(group_reduce<G>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
template <int G>
__device__ __forceinline__ float group_max_f(float v) {
  return __uint_as_float(group_reduce<G>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

// Inclusive prefix sum over the wave (lane 0 first).
__device__ __forceinline__ int wave_incl_scan(int v) {
  int x = v;
  x += (int)dpp_mov<dpp::kShr1>((uint32_t)x);
  x += (int)dpp_mov<dpp::kShr2>((uint32_t)x);
  x += (int)dpp_mov<dpp::kShr4>((uint32_t)x);
  x += (int)dpp_mov<dpp::kShr8>((uint32_t)x);  // inclusive scan inside each 16-lane row
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Query position t of query i (queries are the last n_q tokens).
__device__ __forceinline__ int query_pos(int L, int nq, int i) { return L - nq + i; }

// Current length of sequence b: lens[b] for a batch of different lengths
// (clamped to [1, L], so a bad value cannot address past the cache), else L.
// L stays the row stride of the per-sequence arrays either way.
__device__ __forceinline__ int seq_len_of(const int32_t* __restrict__ lens, int L, int b) {
  return lens ? min(max(lens[b], 1), L) : L;
}

}  // namespace hsa
