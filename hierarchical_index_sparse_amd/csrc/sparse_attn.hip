// Step 4: exact softmax attention of each query over its kept K/V rows.
//
// HISA page: the indexer's output feeds the unchanged token-level sparse
// attention.  HiLS pseudocode, step 4: softmax(q K_sel^T * scale) V_sel over
// the concatenated rows of the kept chunks.
//
// One wave per (query, kv head, split of the token list).  The G = Hq/Hkv
// query heads that share a kv head form the 16-wide N side of
// v_mfma_f32_16x16x32_bf16 (zero-padded when G < 16), so every gathered K/V
// row (256 bytes) is read once for all G heads.  Per tile of 32 list
// entries:
//   * S^T = K_tile Q^T (2 x 4 MFMAs): A = 16 K rows (gathered with whole-row
//     coalesced loads straight into LDS), B = the query heads, held in
//     registers.  The accumulator layout gives each lane one head and 8
//     tokens, which is the A-operand layout P needs for P V, so no shuffle
//     of P is required.
//   * online softmax in the exp2 domain (running max and sum per head).
//   * O += P V (8 output tiles of 16 dims): each lane loads, for its 8
//     tokens, 16 contiguous bytes (dims 8j .. 8j+7) of each V row straight
//     from memory into registers (each load instruction still covers 4
//     whole rows); output tile c takes dims 8j + c, so its B operand is
//     element c of those 8 chunks (16-bit packing only; V needs no LDS).  P
//     is split into bf16 hi + lo parts (two MFMAs), which keeps P's rounding
//     error near 2^-17 instead of bf16's 2^-9.
// Splits (decode) write unnormalised partial results with their running max
// and sum; k_attn_merge combines them (log-sum-exp merge).  When the split
// count is a multiple of 4, the 4 waves of a workgroup hold 4 consecutive
// splits of one (query, kv head) and combine them in LDS first, so one
// partial per workgroup reaches memory and the merge reads a quarter.
#include "common.hpp"
#include "kernels.hpp"
#include "token_select.hpp"

namespace hsa {

constexpr int kPartStride = 130;  // 128 dims + running max + running sum
// K tiles go straight into LDS (global_load_lds_dwordx4), two buffers per
// wave, swizzled instead of padded: 16-byte chunk c of tile row r sits at
// unit 16 r + (c ^ (r & 15)).
constexpr int kKTileBytes = 32 * 256;
constexpr int kWaveLds = 2 * kKTileBytes;
// The running max per head is only moved when a tile's max exceeds it by more
// than this (log2 units), so O is rescaled on few tiles; P = exp2(s - max)
// then stays below 2^kLazyMax.
constexpr float kLazyMax = 8.f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Reductions over the lanes l, l^16, l^32, l^48 (the four lane rows that
// hold one head's tokens), with gfx950's row-swap permutes.
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wave's share of the attention: list positions [start, end) of query q
// for kv head g (item = this wave's (query, kv head, split) index).  The
// list entries are tl[pos - base] for pos <= last: with LIST_LDS, tl is an
// LDS copy of positions base .. last, else the query's row of the list in
// memory (base 0, last k - 1).  Splits write their partial result
// (combined across the workgroup's 4 waves first when `premerge`, which all
// 4 waves then reach); else O and lse.
template <bool SPLIT, bool LIST_LDS>
__device__ __forceinline__ void attend_list(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                            const uint16_t* __restrict__ V, const int32_t* __restrict__ tl,
                                            int base, int last, float* __restrict__ O, float* __restrict__ lse,
                                            float* __restrict__ part, unsigned char* stage_lds, int item, int q,
                                            int g, int L, int nq, int Hq, int Hkv, int start, int end,
                                            float scale_log2, const int32_t* __restrict__ lens, bool premerge) {
  const int wave = threadIdx.x / kWave;
  const int b = q / nq;
  const int G = Hq / Hkv;
  const int lane = lane_id();
  const int jl = lane & 15;
  const int gq = lane >> 4;

  // B operand of S^T = K Q^T: head jl, dims 8 gq + 32 ks .. + 7
  bf16x8 qf[4];
  {
    const uint16_t* qrow = Q + ((size_t)q * Hq + (size_t)g * G + jl) * 128 + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (jl < G) v = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
      qf[ks] = as_bf16x8(v);
    }
  }

  // this (sequence, kv head)'s rows; a row's byte offset fits 31 bits
  // (seq_len * n_heads_kv * 256 < 2^31, checked at the API)
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K + ((size_t)b * L * Hkv + g) * 128);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V + ((size_t)b * L * Hkv + g) * 128);
  const int row_bytes = Hkv * 256;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // byte offset of list entry `pos`'s row if it is a valid token of this
  // sequence, else -1
  const int Lb = seq_len_of(lens, L, b);  // entries at or past the sequence's length are skipped
  auto row_off = [&](int v) { return (v >= 0 && v < Lb) ? (int)__umul24((unsigned)v, (unsigned)row_bytes) : -1; };
  auto entry = [&](int pos) { return row_off(pos < end ? tl[pos - base] : -1); };
  // One tile's V rows straight into the P V operand layout: w[e] holds dims
  // 8 jl .. 8 jl + 7 of the lane's P token e (tokens 4 gq + e, then
  // 16 + 4 gq + e - 4); instruction e still reads 4 whole rows.
  auto vload = [&](int my, u32x4 (&w)[8]) {
    const int mine = max(my, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tr = (e < 4) ? 4 * gq + e : 16 + 4 * gq + (e - 4);
      const unsigned off = (unsigned)__shfl(mine, tr, kWave) + 16u * (unsigned)jl;
      w[e] = *reinterpret_cast<const u32x4*>(Vb + off);
    }
  };
  unsigned char* kst = stage_lds + (size_t)wave * kWaveLds;
  // K tile straight into LDS buffer kb: instruction i takes rows 4i .. 4i+3
  // (whole 256-byte rows, coalesced as before); lane 16 rr + cc lands in unit
  // 64 i + 16 rr + cc, so it loads chunk cc ^ (r & 15) of row r = 4i + rr
  auto kdma = [&](int my, unsigned char* kb) {
    const int mine = max(my, 0);
    const int rr = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + rr;
      const unsigned off = (unsigned)__shfl(mine, r, kWave) + 16u * (unsigned)(cc ^ (r & 15));
      __builtin_amdgcn_global_load_lds((const void*)(Kb + off),
                                       (__attribute__((address_space(3))) void*)(kb + 1024 * i), 16, 0, 0);
    }
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  u32x4 w[8];
  int my = entry(start + (lane & 31));
  int my_next = entry(start + 32 + (lane & 31));
  {
    // Issue order, kept by scheduling barriers: K_0 (into buffer 0), K_1
    // (buffer 1), V_0; then per tile t: the list entries of tile t+2 (one
    // load, always issued), [reads of K_t, softmax, P V], K_{t+2} (into the
    // buffer K_t was read from), V_{t+1}.  Before K_t is read the wave waits
    // until at most N of its vector-memory operations are in flight, N being
    // the count issued after K_t's last one that is certain in every case
    // (t = 0: K_1 if any, V_0, one list load; t >= 1: one list load, K_{t+1}
    // if any, V_t, one list load), so K_t is complete and what follows it
    // may still be in flight.
    kdma(my, kst);
    __builtin_amdgcn_sched_barrier(0);
    if (start + 32 < end) kdma(my_next, kst + kKTileBytes);
    __builtin_amdgcn_sched_barrier(0);
    vload(my, w);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int p0 = start; p0 < end; p0 += 32) {
    const uint32_t vmask = (uint32_t)ballot(my >= 0);
    // (the list entries of tile t+2: loaded here, turned into row offsets
    // where they are used, so nothing waits for them early)
    const int pos2 = p0 + 64 + (lane & 31);
    const int raw_next2 = tl[min(pos2, last) - base];  // always one load (the wait counts rely on it)
    const unsigned char* kt = kst + (((p0 - start) >> 5) & 1) * kKTileBytes;
    {
      // s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt (7) and
      // lgkmcnt (15) left alone
#define HSA_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (7 << 4) | (0xF << 8))
      __builtin_amdgcn_sched_barrier(0);
      constexpr int nl = LIST_LDS ? 0 : 1;  // vector-memory loads per list read
      if (p0 == start) {
        if (start + 32 < end) HSA_VMCNT(16 + nl);
        else HSA_VMCNT(8 + nl);
      } else {
        if (p0 + 32 < end) HSA_VMCNT(16 + 2 * nl);
        else HSA_VMCNT(8 + 2 * nl);
      }
#undef HSA_VMCNT
      __builtin_amdgcn_sched_barrier(0);
    }

    if (vmask != 0u) {
      // ---- S^T = K Q^T over two 16-token tiles (A = staged K rows)
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = gq + 4 * ks;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(kt + 16 * (16 * jl + (c ^ jl)));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(kt + 16 * (16 * (16 + jl) + (c ^ jl)));
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), qf[ks], s1, 0, 0, 0);
      }
      // ---- online softmax (lane: head jl, tokens 4gq+e and 16+4gq+e)
      float sv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = s0[e] * scale_log2;
        sv[4 + e] = s1[e] * scale_log2;
      }
      if (vmask != 0xFFFFFFFFu) {  // holes or the list's tail
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (!((vmask >> (4 * gq + e)) & 1u)) sv[e] = -INFINITY;
          if (!((vmask >> (16 + 4 * gq + e)) & 1u)) sv[4 + e] = -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mx = max_x32(max_x16(mx));
      if (ballot(mx > m_run + kLazyMax)) {
        // move the running max of every head that grew, rescale O and l
        const float m_new = mx > m_run + kLazyMax ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const float a = __shfl(alpha, 4 * gq + i2, kWave);  // rows of O are heads 4gq+i2
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) o[nt][i2] *= a;
        }
      }
      // P = exp2(s - m_run) <= 2^kLazyMax, split into bf16 hi (truncated)
      // + lo (the exact remainder, truncated): relative error <= 2^-16
      float psum = 0.f;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float pa = __builtin_amdgcn_exp2f(sv[e] - m_run);
        const float pb = __builtin_amdgcn_exp2f(sv[e + 1] - m_run);
        psum += pa + pb;
        const float ra = pa - __uint_as_float(__float_as_uint(pa) & 0xFFFF0000u);
        const float rb = pb - __uint_as_float(__float_as_uint(pb) & 0xFFFF0000u);
        ph[e / 2] = __builtin_amdgcn_perm(__float_as_uint(pb), __float_as_uint(pa), 0x07060302u);
        pl[e / 2] = __builtin_amdgcn_perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u);
      }
      l_run += psum;
      const bf16x8 p_hi = as_bf16x8(u32x4{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8 p_lo = as_bf16x8(u32x4{pl[0], pl[1], pl[2], pl[3]});

      // ---- O += P V; output tile c holds dims 8 jl + c, so its B operand is
      // element c of the lane's 8 V chunks, packed two tokens per register
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        u32x4 ev, od;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t x0 = w[2 * e2][pr], x1 = w[2 * e2 + 1][pr];
          ev[e2] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
          od[e2] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 vb = as_bf16x8(hh ? od : ev);
          f32x4 acc = o[2 * pr + hh];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi, vb, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo, vb, acc, 0, 0, 0);
          o[2 * pr + hh] = acc;
        }
      }
    }
    int my_next2;
    {
      // K_{t+2} into the buffer tile t was read from, then V_{t+1}
      __builtin_amdgcn_sched_barrier(0);
      my_next2 = row_off(pos2 < end ? raw_next2 : -1);
      wave_sync();  // tile t's LDS reads are done
      if (p0 + 64 < end) kdma(my_next2, const_cast<unsigned char*>(kt));
      __builtin_amdgcn_sched_barrier(0);
      if (p0 + 32 < end) vload(my_next, w);  // tile t's P V is done with w
      __builtin_amdgcn_sched_barrier(0);
    }
    my = my_next;
    my_next = my_next2;
  }

  l_run = sum_x32(sum_x16(l_run));
  if constexpr (SPLIT) {
    if (premerge) {  // uniform over the grid; every wave of the workgroup is here
      // this wave's partial into its own (no longer used) staging area, in
      // the partial layout; then each thread combines 8 columns of one head
      float* mine = reinterpret_cast<float*>(kst);
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        float* dst = mine + (4 * gq + i2) * kPartStride + 8 * jl;
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[c] = o[c][i2];
      }
      if (gq == 0) {
        mine[jl * kPartStride + 128] = m_run;
        mine[jl * kPartStride + 129] = l_run;
      }
      __syncthreads();
      const int h = threadIdx.x >> 4, d0 = 8 * (threadIdx.x & 15);
      if (h < G) {
        const float* src[4];
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          src[wi] = reinterpret_cast<const float*>(stage_lds + (size_t)wi * kWaveLds) + h * kPartStride;
          mw[wi] = src[wi][128];
          M = fmaxf(M, mw[wi]);
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, Ls = 0.f;
        if (M != -INFINITY) {
#pragma unroll
          for (int wi = 0; wi < 4; ++wi) {
            const float a = __builtin_amdgcn_exp2f(mw[wi] - M);  // 0 for a split without tokens
            Ls += a * src[wi][129];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += a * src[wi][d0 + e];
          }
        }
        float* dst = part + ((size_t)blockIdx.x * 16 + h) * kPartStride;
        *reinterpret_cast<f32x4*>(dst + d0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(dst + d0 + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        if (d0 == 0) {
          dst[128] = M;
          dst[129] = Ls;
        }
      }
      return;
    }
  }
  // outputs: lane holds heads 4gq+i, dims 8 jl + c (c = output tile)
#pragma unroll
  for (int i2 = 0; i2 < 4; ++i2) {
    const int head = 4 * gq + i2;
    const float l_h = __shfl(l_run, head, kWave);
    if (head >= G) continue;
    const float inv = SPLIT ? 1.f : (l_h > 0.f ? 1.f / l_h : 0.f);
    float* dst = SPLIT ? part + ((size_t)item * 16 + head) * kPartStride
                       : O + ((size_t)q * Hq + (size_t)g * G + head) * 128;
    *reinterpret_cast<f32x4*>(dst + 8 * jl) =
        f32x4{o[0][i2] * inv, o[1][i2] * inv, o[2][i2] * inv, o[3][i2] * inv};
    *reinterpret_cast<f32x4*>(dst + 8 * jl + 4) =
        f32x4{o[4][i2] * inv, o[5][i2] * inv, o[6][i2] * inv, o[7][i2] * inv};
  }
  if (gq == 0 && jl < G) {
    if constexpr (SPLIT) {
      float* dst = part + ((size_t)item * 16 + jl) * kPartStride;
      dst[128] = m_run;
      dst[129] = l_run;
    } else if (lse) {
      lse[(size_t)q * Hq + (size_t)g * G + jl] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

template <bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_sparse_attn(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V, const int32_t* __restrict__ tok,
                                                     float* __restrict__ O, float* __restrict__ lse,
                                                     float* __restrict__ part, int L, int nq, int Hq, int Hkv, int k,
                                                     int chunk, int nsplit, float scale_log2, int n_items,
                                                     const int32_t* __restrict__ lens, bool premerge) {
  // per wave: the staged K rows of one tile (V goes from memory straight
  // into the P V operand registers)
  __shared__ __attribute__((aligned(16))) unsigned char stage_lds[4 * kWaveLds];
  const int item = blockIdx.x * 4 + (int)threadIdx.x / kWave;
  if (item >= n_items) return;
  const int split = item % nsplit;
  const int qg = item / nsplit;
  const int q = qg / Hkv;
  const int start = split * chunk;
  attend_list<SPLIT, false>(Q, K, V, tok + (size_t)q * k, 0, k - 1, O, lse, part, stage_lds, item, q, qg % Hkv, L, nq,
                            Hq, Hkv, start, min(k, start + chunk), scale_log2, lens, premerge);
}

// Decode: the token select (step 3's top-k) and the attention in one
// launch.  A workgroup holds 4 consecutive splits of one (query, kv head),
// as k_sparse_attn's do when it pre-merges.  Its 8 waves first run the
// query's exact select, the same as k_token_select's, and keep in LDS the
// positions of the list its 4 splits attend to.  Waves 0-3 then attend as
// k_sparse_attn's waves do, with the same code, splits and pre-merge, so
// the partial results carry the same bits.  Waves 4-7 write the
// workgroup's part of the list to `tok` (kv head 0 only) and end.  Every
// workgroup of a query repeats the select.  That costs 4 bytes per
// candidate (the scores) and no time where the launch has one workgroup per
// CU or fewer, and it removes a launch, the list's round trip through memory
// and a launch gap from the step.
// Waves of a k_select_attn workgroup: all select, 4 attend.
constexpr int kSaWaves = 8;

template <int R, bool ONEBLK>
__global__ __launch_bounds__(kSaWaves * 64) void k_select_attn(const float* __restrict__ scores, const int32_t* __restrict__ blk,
                                                     int32_t* __restrict__ tok, const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                     float* __restrict__ part, int L, int nq, int B, int log2B, int m,
                                                     int k, int Hq, int Hkv, int chunk, int nsplit, float scale_log2,
                                                     const int32_t* __restrict__ lens) {
  constexpr int NW = kSaWaves;
  constexpr int NT = NW * kWave;
  __shared__ __attribute__((aligned(16))) unsigned char stage_lds[4 * kWaveLds];
  __shared__ SelectSmem<NW> sel;
  // the block list (m entries, padded to 4), then list positions
  // [p_lo, p_hi) and one dummy slot per lane
  extern __shared__ __attribute__((aligned(16))) int dyn_lds[];
  int* bl = dyn_lds;
  int* plist = dyn_lds + ((m + 3) & ~3);
  const int item0 = blockIdx.x * 4;
  const int qg = item0 / nsplit;
  const int s0 = item0 % nsplit;
  const int q = qg / Hkv, g = qg % Hkv;
  const int p_lo = s0 * chunk, p_hi = min(k, p_lo + 4 * chunk);
  const int dummy = 4 * chunk + lane_id();
  const bool selected = select_query_tokens<NW, R, ONEBLK, true>(
      scores, blk, q, L, nq, B, log2B, m, k, lens, p_lo, p_hi, sel, bl, [&](int slot, int v) { plist[slot - p_lo] = v; },
      [&](int pos, int v, bool take) { plist[(take && pos >= p_lo && pos < p_hi) ? pos - p_lo : dummy] = v; });
  if (!selected) __syncthreads();  // (the select ends with a barrier, keeping all does not)
  const int wave = (int)threadIdx.x / kWave;
  if (wave >= 4) {
    if (g == 0) {
      int32_t* out = tok + (size_t)q * k + p_lo;
      const int n = p_hi - p_lo, x = (int)threadIdx.x - 256, nx = NT - 256;
      if ((k & 3) == 0) {  // 16-byte aligned, n a multiple of 4
        for (int p = 4 * x; p < n; p += 4 * nx)
          *reinterpret_cast<u32x4*>(out + p) = *reinterpret_cast<const u32x4*>(plist + p);
      } else {
        for (int p = x; p < n; p += nx) out[p] = plist[p];
      }
    }
    return;
  }
  const int start = (s0 + wave) * chunk;
  attend_list<true, true>(Q, K, V, plist, p_lo, p_hi - 1, nullptr, nullptr, part, stage_lds, item0 + wave, q, g, L, nq,
                          Hq, Hkv, start, min(k, start + chunk), scale_log2, lens, true);
}

// Log-sum-exp merge of the splits of one (query, head), spread over CC
// workgroups of 128 / CC output columns each: the partials come from other
// XCDs' caches, so the merge is paced by how many loads the CUs keep in
// flight, and with few (query, head) rows more CUs must take part.  256
// threads = 8 * CC split groups x 32 / CC float4 column lanes; a group loads
// 4 splits' partials per round, merges them against the group's own running
// maximum, and the groups meet in LDS, rescaled to the overall maximum.
template <int CC>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part, float* __restrict__ O,
                                                    float* __restrict__ lse, int Hq, int Hkv, int nsplit) {
  constexpr int U = 4;                // splits per group and round
  constexpr int LANES = 32 / CC;      // float4 lanes per group
  constexpr int NG = 256 / LANES;     // split groups
  constexpr int COLS = 128 / CC;      // output columns of this workgroup
  __shared__ float red[NG][COLS + 1];
  __shared__ float gmax[NG];
  const int qh = blockIdx.x / CC;
  const int chunk = blockIdx.x % CC;
  const int q = qh / Hq, h = qh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G, head = h % G;
  const int tid = threadIdx.x;
  const float* base = part + ((size_t)(q * Hkv + g) * nsplit * 16 + head) * kPartStride;
  const size_t sstride = (size_t)16 * kPartStride;
  const int sg = tid / LANES, dq = tid % LANES;
  const int col = chunk * COLS + 4 * dq;

  float Mg = -INFINITY, Lt = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = sg; s0 < nsplit; s0 += NG * U) {
    float4 v[U];
    float mx[U], ls[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* p = base + (size_t)min(s0 + NG * u, nsplit - 1) * sstride;
      mx[u] = p[128];
      ls[u] = p[129];
      v[u] = *reinterpret_cast<const float4*>(p + col);
    }
    float Mn = Mg;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + NG * u < nsplit) Mn = fmaxf(Mn, mx[u]);
    if (Mn == -INFINITY) continue;  // no token in these splits
    const float r = exp2f(Mg - Mn);  // 0 on the first round
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
    Lt *= r;
    Mg = Mn;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + NG * u >= nsplit) break;
      const float wgt = exp2f(mx[u] - Mg);
      acc.x += wgt * v[u].x;
      acc.y += wgt * v[u].y;
      acc.z += wgt * v[u].z;
      acc.w += wgt * v[u].w;
      Lt += wgt * ls[u];
    }
  }
  red[sg][4 * dq] = acc.x;
  red[sg][4 * dq + 1] = acc.y;
  red[sg][4 * dq + 2] = acc.z;
  red[sg][4 * dq + 3] = acc.w;
  if (dq == 0) {
    red[sg][COLS] = Lt;
    gmax[sg] = Mg;
  }
  __syncthreads();
  // groups past the splits hold nothing: only min(NG, nsplit) are read
  const int ng = min(NG, nsplit);
  if (tid < COLS) {
    float M = -INFINITY;
    for (int k = 0; k < ng; ++k) M = fmaxf(M, gmax[k]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
      for (int k = 0; k < ng; ++k) {
        const float wk = exp2f(gmax[k] - M);  // 0 for a group without tokens
        a += wk * red[k][tid];
        l += wk * red[k][COLS];
      }
    }
    O[(size_t)qh * 128 + chunk * COLS + tid] = l > 0.f ? a / l : 0.f;
    if (lse && chunk == 0 && tid == 0) lse[qh] = l > 0.f ? (M + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

// Split plan: enough waves to fill the chip when there are few queries.
static void split_plan(const Dims& s, int& nsplit, int& chunk) {
  // at least 2 tiles (64 entries) per split (one-tile splits spend more on
  // each wave's start than they gain in waves), at most 1024 splits (the
  // merge reads a quarter of them after the in-workgroup pre-merge); at
  // most ~2048 waves in total
  const long long items = (long long)s.b * s.nq * s.Hkv;
  const int tiles = (s.k + 31) / 32;
  long long want = (items <= 0 || items >= 2048) ? 1 : (2048 + items - 1) / items;
  const long long cap = min((tiles + 1) / 2, 1024);
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  const int tiles_per = (int)((tiles + want - 1) / want);
  chunk = tiles_per * 32;
  nsplit = (s.k + chunk - 1) / chunk;
}

size_t sparse_attn_ws_bytes(const Dims& s) {
  int nsplit, chunk;
  split_plan(s, nsplit, chunk);
  if (nsplit <= 1) return 0;
  return align_up((size_t)s.b * s.nq * s.Hkv * nsplit * 16 * kPartStride * sizeof(float));
}

// Log-sum-exp merge of `nsplit` partials per (query, kv head) into O and
// lse: about 1024 merge workgroups, few (query, head) rows get more column
// chunks.
static hipError_t launch_merge(const Dims& s, const float* part, float* O, float* lse, int nsplit, hipStream_t st) {
  const long long rows = (long long)s.b * s.nq * s.Hq;
  const dim3 mb(256);
  if (rows >= 512)
    HSA_LAUNCH(k_attn_merge<1>, dim3((unsigned)rows), mb, 0, st, part, O, lse, s.Hq, s.Hkv, nsplit);
  else if (rows >= 256)
    HSA_LAUNCH(k_attn_merge<2>, dim3((unsigned)(rows * 2)), mb, 0, st, part, O, lse, s.Hq, s.Hkv, nsplit);
  else if (rows >= 128)
    HSA_LAUNCH(k_attn_merge<4>, dim3((unsigned)(rows * 4)), mb, 0, st, part, O, lse, s.Hq, s.Hkv, nsplit);
  else
    HSA_LAUNCH(k_attn_merge<8>, dim3((unsigned)(rows * 8)), mb, 0, st, part, O, lse, s.Hq, s.Hkv, nsplit);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const Dims& s, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                              const int32_t* tok, float* O, float* lse, void* ws, hipStream_t st) {
  const long long nq_total = (long long)s.b * s.nq;
  if (nq_total == 0) return hipSuccess;
  int nsplit, chunk;
  split_plan(s, nsplit, chunk);
  const int n_items = (int)(nq_total * s.Hkv * nsplit);
  const float scale_log2 = s.scale * 1.4426950408889634f;
  dim3 grid((n_items + 3) / 4), block(256);
  if (nsplit == 1) {
    HSA_LAUNCH((k_sparse_attn<false>), grid, block, 0, st, Q, K, V, tok, O, lse, nullptr, s.L, s.nq, s.Hq,
                       s.Hkv, s.k, chunk, nsplit, scale_log2, n_items, s.lens, false);
    return hipGetLastError();
  }
  float* part = static_cast<float*>(ws);
  // 4 splits per workgroup combined in LDS: n_items is then a multiple of 4
  // and every workgroup holds 4 splits of one (query, kv head)
  const bool premerge = nsplit % 4 == 0;
  HSA_LAUNCH((k_sparse_attn<true>), grid, block, 0, st, Q, K, V, tok, O, lse, part, s.L, s.nq, s.Hq, s.Hkv,
                     s.k, chunk, nsplit, scale_log2, n_items, s.lens, premerge);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(s, part, O, lse, premerge ? nsplit / 4 : nsplit, st);
}

// ---- decode: select and attention in one launch

constexpr size_t kMaxLdsBytes = 160 * 1024;

// Whether any query of the call scores its candidates (else every query
// keeps all of them), and the select's slots per thread over 8 waves.
static bool sa_scoring(const Dims& s) { return (long long)s.k < (long long)s.m * s.B && s.L > s.k; }
static int sa_slots(const Dims& s) {
  if (!sa_scoring(s)) return 1;
  int r = 1;
  while ((long long)r * kSaWaves * 64 < (long long)s.m * s.B) r <<= 1;
  return r;
}
static size_t sa_dyn_lds(const Dims& s, int chunk) {
  return sizeof(int) * ((size_t)((s.m + 3) & ~3) + 4 * (size_t)chunk + kWave);
}

bool select_attn_fusable(const Dims& s) {
  const long long nq_total = (long long)s.b * s.nq;
  if (nq_total == 0) return false;
  int nsplit, chunk;
  split_plan(s, nsplit, chunk);
  if (nsplit < 4 || nsplit % 4 != 0) return false;  // 4 splits of one (query, kv head) per workgroup
  if (sa_slots(s) > 32) return false;
  return sa_dyn_lds(s, chunk) + 4 * kWaveLds + sizeof(SelectSmem<kSaWaves>) <= kMaxLdsBytes;
}

size_t select_attn_ws_bytes(const Dims& s) { return token_topk_ws_bytes(s) + sparse_attn_ws_bytes(s); }

template <int R, bool ONEBLK>
static hipError_t launch_sa_k(const Dims& s, const float* scores, const int32_t* blk, int32_t* tok,
                              const uint16_t* Q, const uint16_t* K, const uint16_t* V, float* part, int chunk,
                              int nsplit, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_select_attn<R, ONEBLK>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sa_dyn_lds(s, chunk));
  if (e != hipSuccess) return e;
  const int n_wg = (int)((long long)s.b * s.nq * s.Hkv * nsplit / 4);
  HSA_LAUNCH((k_select_attn<R, ONEBLK>), dim3(n_wg), dim3(kSaWaves * 64), sa_dyn_lds(s, chunk), st, scores, blk, tok, Q, K, V,
             part, s.L, s.nq, s.B, __builtin_ctz((unsigned)s.B), s.m, s.k, s.Hq, s.Hkv, chunk, nsplit,
             s.scale * 1.4426950408889634f, s.lens);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_sa_r(const Dims& s, const float* scores, const int32_t* blk, int32_t* tok,
                              const uint16_t* Q, const uint16_t* K, const uint16_t* V, float* part, int chunk,
                              int nsplit, hipStream_t st) {
  if (R <= s.B) return launch_sa_k<R, true>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st);
  if constexpr (R > 8) return launch_sa_k<R, false>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st);
  return hipErrorInvalidValue;  // B >= 8
}

hipError_t launch_select_attn(const Dims& s, const float* scores, const int32_t* blk, int32_t* tok, const uint16_t* Q,
                              const uint16_t* K, const uint16_t* V, float* O, float* lse, void* ws, hipStream_t st) {
  if ((long long)s.b * s.nq == 0) return hipSuccess;
  if (!select_attn_fusable(s)) return hipErrorInvalidValue;
  int nsplit, chunk;
  split_plan(s, nsplit, chunk);
  float* part = static_cast<float*>(ws);
  hipError_t e;
  switch (sa_slots(s)) {
    case 1: e = launch_sa_r<1>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st); break;
    case 2: e = launch_sa_r<2>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st); break;
    case 4: e = launch_sa_r<4>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st); break;
    case 8: e = launch_sa_r<8>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st); break;
    case 16: e = launch_sa_r<16>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st); break;
    case 32: e = launch_sa_r<32>(s, scores, blk, tok, Q, K, V, part, chunk, nsplit, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_merge(s, part, O, lse, nsplit / 4, st);
}

}  // namespace hsa
