/*
 * hsa_sparse.h - hierarchical block-then-token sparse attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (HISA page, "北大团队改造DeepSeek注意力，速度快四倍还不丢精度",
 * two-step method; HiLS page, "把稀疏注意力做对 HiLS-Attention …", sections
 * 2.1-2.2 and its hils_attention pseudocode) replaces a flat top-k indexer
 * that scores every earlier token by four steps:
 *   1. summarise every block of B indexer keys into one vector (the mean) or
 *      into n_landmarks landmark vectors (fixed 0/1 projection of the block);
 *   2. score the causal blocks with the indexer rule (dot product with the
 *      query's indexer vector; max over landmarks) and keep m blocks, the
 *      first block and the query's own block always among them;
 *   3. score only the tokens of the kept blocks and keep k of them;
 *   4. run exact softmax attention over the k kept K/V rows (unchanged
 *      downstream sparse attention).
 *
 * Conventions shared by every entry point:
 *   - bf16 tensors are passed as raw bit patterns (uint16_t*).  Every tensor
 *     is contiguous, row-major, and lives in device memory on the current
 *     HIP device.
 *   - Each of the `batch` sequences has `seq_len` tokens; its n_q queries
 *     sit at the last n_q positions: query i has position t = seq_len-n_q+i.
 *     A token s is a candidate for the query at t only when s <= t.
 *   - Selection order is (score descending, index ascending): ties go to the
 *     lower block / token index.  Index lists are ascending and padded with
 *     -1.  When a query has at most m causal blocks (or at most k candidate
 *     tokens) all of them are kept without scoring.
 *   - m counts the two forced blocks (block 0 and block t / B).
 *   - Calls are asynchronous on `stream` (NULL = the default stream) and
 *     never synchronise the host; results are valid once the stream has
 *     reached them.  The library allocates no device memory: scratch space
 *     is the caller's `workspace`, sized by hsa_sparse_workspace_size()
 *     (hsa_forward_noalloc uses a fixed device array of the library
 *     instead).
 *   - Arguments are validated before anything is launched.  On an error
 *     nothing is written and nothing is enqueued.  hsa_sparse_last_error()
 *     returns a message for the calling thread's last failure.
 *
 * Supported shapes: head_dim == 128; d_index in {64, 128}; block a power of
 * two in [8, 128]; n_landmarks in {1, 2, 4}; n_heads_kv divides n_heads_q
 * with at most 16 query heads per kv head; top_m >= 2; top_k >= 1;
 * ceil(seq_len / block) - 2 <= 32768; top_m * block <= 32768 unless
 * top_k >= top_m * block (then no token scoring is needed);
 * batch * n_q <= 2^30; for attention, seq_len * n_heads_kv * 256 < 2^31
 * (a kv row's byte offset in its sequence is a 31-bit integer) and
 * batch * n_q * n_heads_q <= 2^30.
 */
#ifndef HSA_SPARSE_H
#define HSA_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hsa_sparse_status {
  HSA_SPARSE_OK = 0,
  HSA_SPARSE_INVALID_ARG = 1,          /* null pointer, inconsistent sizes */
  HSA_SPARSE_UNSUPPORTED = 2,          /* valid but outside the supported shapes */
  HSA_SPARSE_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < required size */
  HSA_SPARSE_HIP_ERROR = 4             /* a HIP call or kernel launch failed */
} hsa_sparse_status_t;

typedef struct hsa_sparse_shape {
  int32_t batch;        /* b: independent sequences */
  int32_t seq_len;      /* L: tokens per sequence, queries included */
  int32_t n_q;          /* queries per sequence (the last n_q positions) */
  int32_t d_index;      /* indexer vector width d_I */
  int32_t block;        /* B: tokens per key block */
  int32_t n_landmarks;  /* summary vectors per block: 1 = mean */
  int32_t top_m;        /* m: kept blocks per query, forced ones included */
  int32_t top_k;        /* k: kept tokens per query */
  int32_t n_heads_q;    /* Hq */
  int32_t n_heads_kv;   /* Hkv; query head h reads kv head h / (Hq / Hkv) */
  int32_t head_dim;     /* d */
  float scale;          /* softmax scale applied to q . k */
} hsa_sparse_shape_t;

/* Same object as hipStream_t. */
typedef struct ihipStream_t* hsa_sparse_stream_t;

enum {
  HSA_SPARSE_OP_BLOCK_SUMMARY = 0,
  HSA_SPARSE_OP_BLOCK_TOPM = 1,
  HSA_SPARSE_OP_TOKEN_TOPK = 2,
  HSA_SPARSE_OP_SPARSE_ATTN = 3,
  HSA_SPARSE_OP_FORWARD = 4,
  HSA_SPARSE_OP_FLAT_TOPK = 5,
  HSA_SPARSE_OP_HEAD_TOPM = 6,
  HSA_SPARSE_OP_FORWARD_HEADS = 7,
  HSA_SPARSE_OP_BLOCK_SCORE_MAX = 8
};

/* Bytes of device workspace the operation `op` needs for `shape`
 * (0 for an invalid shape or op).  Host-only arithmetic. */
size_t hsa_sparse_workspace_size(const hsa_sparse_shape_t* shape, int op);

/* Static text of a status code. */
const char* hsa_sparse_strerror(hsa_sparse_status_t status);

/* Detail of the calling thread's last failed call ("" if none). */
const char* hsa_sparse_last_error(void);

/*
 * Step 1, block summaries (HISA page, step one: one summary vector per
 * fixed-size block; HiLS page, section 2.1: landmark vectors per chunk).
 *   kI          [batch, seq_len, d_index] bf16, integer-valued in the
 *               workloads (then every sum below is exact in fp32).
 *   landmark_W  NULL for mean mode (n_landmarks must be 1), else
 *               [n_landmarks, block] int8 weights.
 *   start_block summaries are written for blocks start_block .. nb-1 only
 *               (nb = ceil(seq_len / block)); earlier ones are left as is.
 *   S           [batch, nb, n_landmarks, d_index] bf16 output:
 *               S[j, l] = bf16_rne(sum_r w[l, r] * kI[j*B + r] / B), with
 *               w = 1 in mean mode and rows beyond seq_len counted as 0.
 */
hsa_sparse_status_t hsa_block_summary(const hsa_sparse_shape_t* shape,
                                      const uint16_t* kI,
                                      const int8_t* landmark_W,
                                      int32_t start_block, uint16_t* S,
                                      hsa_sparse_stream_t stream);

/*
 * Step 2, block scores and top-m (HISA page, step one scoring with the
 * original indexer rule, and the always-kept first and last block; HiLS
 * page, section 2.2 coarse layer).
 *   qI   [batch, n_q, d_index] bf16 indexer queries.
 *   S    [batch, nb, n_landmarks, d_index] bf16 summaries (step 1).
 *   blk  [batch, n_q, top_m] int32 output: for the query at t with
 *        c = t / block, all of 0..c if c + 1 <= top_m, else
 *        {0, c} plus the best top_m - 2 blocks of 1..c-1 by
 *        score_j = max_l qI . S[j, l]; ascending, -1 padded.
 *   workspace  >= hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_BLOCK_TOPM).
 */
hsa_sparse_status_t hsa_block_topm(const hsa_sparse_shape_t* shape,
                                   const uint16_t* qI, const uint16_t* S,
                                   int32_t* blk, void* workspace,
                                   size_t workspace_bytes,
                                   hsa_sparse_stream_t stream);

/*
 * The block-score contraction of step 2 without its selection, for
 * measuring the contraction on its own (HISA page, complexity: the block
 * scores are the L^2/B term of O(L^2/B + L*m*B)).
 *   out  [batch, n_q] fp32: for the query at t with c = t / block and
 *        c + 1 > top_m, max over blocks 1..c-1 of score_j (the best score
 *        hsa_block_topm ranks); -inf when c + 1 <= top_m (nothing scored).
 *   workspace  >= hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_BLOCK_SCORE_MAX).
 * Scores run on the same bf16 MFMA tiling as hsa_block_topm's for many
 * queries, but each query's maximum is formed on chip, so one float per
 * query (per chunk of summary tiles, when there are few queries) is written.
 * Errors: as for hsa_block_topm.
 */
hsa_sparse_status_t hsa_block_score_max(const hsa_sparse_shape_t* shape,
                                        const uint16_t* qI, const uint16_t* S,
                                        float* out, void* workspace,
                                        size_t workspace_bytes,
                                        hsa_sparse_stream_t stream);

/*
 * Step 3, token scores and top-k inside the kept blocks (HISA page, step
 * two).
 *   qI, kI  as above; blk [batch, n_q, top_m] from step 2
 *           (hsa_block_topm or hsa_block_topm_3level): per query an
 *           ascending list of blocks <= c = t / block whose last entry is c,
 *           -1 padded; it may hold fewer than min(c + 1, top_m) blocks (the
 *           three-level selection can keep fewer).
 *   tok     [batch, n_q, top_k] int32 output: candidates are the tokens
 *           s <= t of the kept blocks; all of them if at most top_k, else
 *           the best top_k by qI . kI[s]; ascending, -1 padded.
 */
hsa_sparse_status_t hsa_token_topk(const hsa_sparse_shape_t* shape,
                                   const uint16_t* qI, const uint16_t* kI,
                                   const int32_t* blk, int32_t* tok,
                                   void* workspace, size_t workspace_bytes,
                                   hsa_sparse_stream_t stream);

/*
 * Step 4, exact softmax attention over the kept tokens (HISA page: the
 * downstream sparse attention is unchanged; HiLS pseudocode, step 4).
 *   Q    [batch, n_q, n_heads_q, head_dim] bf16.
 *   K, V [batch, seq_len, n_heads_kv, head_dim] bf16.
 *   tok  [batch, n_q, top_k] int32 token lists (-1 entries are skipped;
 *        every list must hold at least one valid entry in [0, seq_len)).
 *   O    [batch, n_q, n_heads_q, head_dim] fp32 output:
 *        softmax(scale * q_h . K[tok, g]) . V[tok, g] with g = h / (Hq/Hkv),
 *        accumulated in fp32.
 *   lse  NULL or [batch, n_q, n_heads_q] fp32: natural log of the softmax
 *        denominator, log sum_s exp(scale * q_h . K[s, g]).
 */
hsa_sparse_status_t hsa_sparse_attn(const hsa_sparse_shape_t* shape,
                                    const uint16_t* Q, const uint16_t* K,
                                    const uint16_t* V, const int32_t* tok,
                                    float* O, float* lse, void* workspace,
                                    size_t workspace_bytes,
                                    hsa_sparse_stream_t stream);

/*
 * Steps 1-4 in one call (the drop-in indexer plus the unchanged attention).
 *   S        in-out summary state [batch, nb, n_landmarks, d_index]: blocks
 *            from summary_start_block on are (re)computed from kI first;
 *            pass 0 to build all of them, or the first block touched by new
 *            tokens when the earlier summaries are already in S.
 *   blk_out  NULL or [batch, n_q, top_m]: also return the block lists.
 *   tok_out  NULL or [batch, n_q, top_k]: also return the token lists.
 *   O, lse   as in hsa_sparse_attn.
 */
hsa_sparse_status_t hsa_forward(const hsa_sparse_shape_t* shape,
                                const uint16_t* qI, const uint16_t* kI,
                                const int8_t* landmark_W,
                                int32_t summary_start_block, uint16_t* S,
                                const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, int32_t* blk_out,
                                int32_t* tok_out, float* O, float* lse,
                                void* workspace, size_t workspace_bytes,
                                hsa_sparse_stream_t stream);

/*
 * hsa_forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors are those of
 * hsa_forward.  Its scratch is a device array inside the library of
 * HSA_SPARSE_NOALLOC_SCRATCH_BYTES bytes, of which every GPU the library
 * runs on holds one copy until the process ends; its address on the
 * stream's device is looked up on the first call there.  The call makes no
 * allocation of its own.
 *   - A shape whose hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_FORWARD)
 *     exceeds HSA_SPARSE_NOALLOC_SCRATCH_BYTES is rejected with
 *     HSA_SPARSE_WORKSPACE_TOO_SMALL before anything is enqueued.
 *   - Every call on one GPU shares that GPU's scratch: calls whose work
 *     overlaps on the GPU (on different streams, or from several threads
 *     without ordering) race and give wrong results.  Calls in one stream's
 *     order are safe; the scratch keeps the last call's contents, and no
 *     call relies on them.
 */
#define HSA_SPARSE_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
hsa_sparse_status_t hsa_forward_noalloc(const hsa_sparse_shape_t* shape,
                                        const uint16_t* qI, const uint16_t* kI,
                                        const int8_t* landmark_W,
                                        int32_t summary_start_block, uint16_t* S,
                                        const uint16_t* Q, const uint16_t* K,
                                        const uint16_t* V, int32_t* blk_out,
                                        int32_t* tok_out, float* O, float* lse,
                                        hsa_sparse_stream_t stream);

/*
 * One decode step over a batch of sequences of different lengths (HISA
 * page: the drop-in indexer leaves the KV cache and the attention as they
 * are, and decode is where its per-token cost matters; the summary of the
 * partial last block is kept up to date as tokens are appended).
 *   shape      seq_len is the capacity: the row stride of kI, K and V per
 *              sequence and ceil(seq_len / block) summary blocks per
 *              sequence in S; n_q must be 1.
 *   seq_lens   device int32 [batch]: the current length L_b of sequence b,
 *              1 <= L_b <= seq_len (values outside are clamped).  The
 *              caller has written the new token's rows kI, K, V at L_b - 1.
 *   qI, Q      the new token of each sequence ([batch, 1, ...]).
 *   S          in-out summary state: on entry it must hold the summaries of
 *              the blocks before each sequence's last block (from earlier
 *              steps or hsa_block_summary); this call recomputes block
 *              (L_b - 1) / block of every sequence from its rows < L_b.
 *   The rest, and the results (for the query at t = L_b - 1, candidates
 *   limited to s <= t), are as for hsa_forward.  Workspace:
 *   hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_FORWARD).
 * Errors: as for hsa_forward; n_q != 1 or seq_lens == NULL is INVALID_ARG.
 */
hsa_sparse_status_t hsa_decode_step(const hsa_sparse_shape_t* shape,
                                    const int32_t* seq_lens,
                                    const uint16_t* qI, const uint16_t* kI,
                                    const int8_t* landmark_W, uint16_t* S,
                                    const uint16_t* Q, const uint16_t* K,
                                    const uint16_t* V, int32_t* blk_out,
                                    int32_t* tok_out, float* O, float* lse,
                                    void* workspace, size_t workspace_bytes,
                                    hsa_sparse_stream_t stream);

/*
 * The flat indexer, the method the hierarchical one replaces (HISA page:
 * the indexer scores each query against every previous token and keeps
 * the most relevant; with every block kept the hierarchical selection
 * reduces to it).  Provided as the baseline the hierarchical path is
 * measured against, and as a check of that reduction.
 *   Reads batch, seq_len, n_q, d_index and top_k of the shape.
 *   qI, kI  as for hsa_token_topk.
 *   tok     [batch, n_q, top_k] int32 output: for the query at t, all of
 *           0..t if t + 1 <= top_k, else the best top_k tokens of 0..t by
 *           qI . kI[s] (ties to the lower index); ascending, -1 padded.
 *   workspace  >= hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_FLAT_TOPK):
 *           every causal score in fp32 ([batch * n_q, seq_len] rounded up to
 *           a multiple of 4 per row) plus the chunk winners' lists when
 *           top_k < seq_len and seq_len > 8192.
 * Supported: d_index in {64, 128}; seq_len <= 2^30; top_k <= 8192 when
 *           top_k < seq_len.
 * Errors: as for the other entry points; nothing is launched on an error.
 */
hsa_sparse_status_t hsa_flat_topk(const hsa_sparse_shape_t* shape,
                                  const uint16_t* qI, const uint16_t* kI,
                                  int32_t* tok, void* workspace,
                                  size_t workspace_bytes,
                                  hsa_sparse_stream_t stream);

/*
 * Three-level selection: super-blocks -> blocks -> tokens (LSA page, latent
 * space and hierarchical clustering: the query descends a tree of key
 * groups from the root and scores only a few nodes per level).  Here the
 * tree is fixed: a super-block is `group` consecutive blocks, summarised by
 * the mean of their summaries and selected like a block (HISA page, step
 * one, with the first and the query's own super-block always kept); the
 * blocks are then selected among the blocks of the kept super-blocks only,
 * which bounds the per-query block work by ceil(nb / group) + top_m2 * group
 * instead of nb.  Supported: group a power of two in [1, 4096],
 * top_m2 >= 2, top_m2 * group <= 8192; the shape as for hsa_forward.
 *
 * hsa_super_summary: S [batch, nb, n_landmarks, d_index] bf16 block
 *   summaries (step 1) -> S2 [batch, nsb, n_landmarks, d_index] bf16 with
 *   nsb = ceil(nb / group):
 *   S2[J, l] = bf16_rne(sum_{g < group} S[J*group + g, l] / group), blocks
 *   past nb counted as 0 (sums in fp32: exact when the summaries' partial
 *   sums fit 24 bits, as for the integer-valued workloads).  Super-blocks
 *   start_super .. nsb-1 are written; earlier ones are left as they are.
 *
 * hsa_block_topm_3level: step 2 through super-blocks.
 *   qI, S as for hsa_block_topm; S2 from hsa_super_summary.
 *   sup  [batch, n_q, top_m2] int32 output, level 1: for the query at t
 *        with C = t / (block * group), all of 0..C if C + 1 <= top_m2,
 *        else {0, C} plus the best top_m2 - 2 of 1..C-1 by
 *        max_l qI . S2[J, l]; ascending, -1 padded.
 *   blk  [batch, n_q, top_m] int32 output, level 2: the candidates are the
 *        blocks j <= c = t / block of the super-blocks in sup; all of them
 *        if at most top_m, else {0, c} plus the best top_m - 2 of the other
 *        candidates by max_l qI . S[j, l]; ascending, -1 padded.
 *   workspace  the size hsa_sparse_workspace_size(shape,
 *        HSA_SPARSE_OP_BLOCK_TOPM) gives is enough for any group.
 *
 * hsa_forward_3level: hsa_forward with step 2 replaced by the two levels
 *   above.  S and S2 are in-out summary state: block summaries from
 *   summary_start_block on and super-block summaries from
 *   summary_start_block / group on are recomputed first.  sup_out is
 *   required; blk_out, tok_out, lse may be NULL.  Workspace:
 *   hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_FORWARD).  Stage events
 *   (hsa_sparse_set_stage_events) mark the same four steps, step 1 ending
 *   after the super-block summaries.
 *   seq_lens: NULL, or a decode step over sequences of different lengths as
 *   for hsa_decode_step: device int32 [batch], n_q must be 1, seq_len is
 *   the capacity (the row stride of kI, K, V, S and S2), the query of
 *   sequence b sits at L_b - 1, and this call rebuilds the summary of block
 *   (L_b - 1) / block and of the super-block holding it, counting only the
 *   sequence's own blocks (summary_start_block is then not read).  Lengths
 *   are clamped to [1, seq_len].
 * Errors: as for the other entry points; nothing is launched on an error.
 */
hsa_sparse_status_t hsa_super_summary(const hsa_sparse_shape_t* shape,
                                      int32_t group, const uint16_t* S,
                                      int32_t start_super, uint16_t* S2,
                                      hsa_sparse_stream_t stream);

hsa_sparse_status_t hsa_block_topm_3level(const hsa_sparse_shape_t* shape,
                                          int32_t group, int32_t top_m2,
                                          const uint16_t* qI,
                                          const uint16_t* S,
                                          const uint16_t* S2, int32_t* sup,
                                          int32_t* blk, void* workspace,
                                          size_t workspace_bytes,
                                          hsa_sparse_stream_t stream);

hsa_sparse_status_t hsa_forward_3level(const hsa_sparse_shape_t* shape,
                                       const int32_t* seq_lens,
                                       int32_t group, int32_t top_m2,
                                       const uint16_t* qI, const uint16_t* kI,
                                       const int8_t* landmark_W,
                                       int32_t summary_start_block,
                                       uint16_t* S, uint16_t* S2,
                                       const uint16_t* Q, const uint16_t* K,
                                       const uint16_t* V, int32_t* sup_out,
                                       int32_t* blk_out, int32_t* tok_out,
                                       float* O, float* lse, void* workspace,
                                       size_t workspace_bytes,
                                       hsa_sparse_stream_t stream);

/*
 * Per-head chunk selection from the attention queries (HiLS page,
 * hils_attention pseudocode: landmark scores are Q against the chunks'
 * landmarks, the top chunks are kept and exact attention runs over the
 * concatenated K/V of the kept chunks; sections 2.1-2.2).  Every query head
 * h selects its own chunks (blocks of `block` tokens) with its own Q_h,
 * against landmarks of its kv head g = h / (n_heads_q / n_heads_kv), and
 * attends over every causal token of them.  There is no token top-k: a
 * head's list is all tokens s <= t of its kept chunks.
 * Shape fields read: batch, seq_len, n_q, block, n_landmarks, top_m,
 * n_heads_q, n_heads_kv, head_dim, scale (d_index and top_k are not read).
 * Supported: head_dim 128; block a power of two in [8, 128]; n_landmarks in
 * {1, 2, 4}; n_heads_kv <= 16 dividing n_heads_q with at most 16 query
 * heads per kv head; top_m >= 2; top_m * block <= 131072;
 * ceil(seq_len / block) - 2 <= 32768; seq_len * n_heads_kv * 256 < 2^31.
 *
 * hsa_head_landmarks: K [batch, seq_len, n_heads_kv, head_dim] bf16 ->
 *   LK [batch, nb, n_landmarks, n_heads_kv, head_dim] bf16,
 *   LK[j, l, g] = bf16_rne(sum_r w[l, r] * K[j*B + r, g] / B) (w = 1 with
 *   landmark_W NULL, which needs n_landmarks == 1), rows past seq_len
 *   counted as 0, summed exactly (fp64) and rounded once.  Chunks
 *   start_block .. nb-1 are written.
 *
 * hsa_head_topm: blk [batch, n_q, n_heads_q, top_m] int32 output: for the
 *   query at t with c = t / block, per head, all of 0..c if c + 1 <= top_m,
 *   else {0, c} plus the best top_m - 2 chunks of 1..c-1 by
 *   max_l Q[h] . LK[j, l, g] (fp32 accumulation of bf16 products, so chunks
 *   whose scores differ by less than the fp32 rounding of the dot product
 *   may be ordered either way; ties to the lower index); ascending, -1
 *   padded.  Workspace: hsa_sparse_workspace_size(shape,
 *   HSA_SPARSE_OP_HEAD_TOPM) (the fp32 chunk scores).
 *
 * hsa_forward_heads: landmarks from summary_start_block on (LK is in-out
 *   state, as S is for hsa_forward), the per-head selection, then for each
 *   (query, head) exact softmax attention over its tokens:
 *   O [batch, n_q, n_heads_q, head_dim] fp32 and lse (NULL or
 *   [batch, n_q, n_heads_q]) as in hsa_sparse_attn.  blk_out: NULL or the
 *   chunk lists as for hsa_head_topm.  Workspace:
 *   hsa_sparse_workspace_size(shape, HSA_SPARSE_OP_FORWARD_HEADS) (lists of
 *   top_m * block tokens per (query, head) plus scratch).  Stage events
 *   mark landmarks (1), selection (2) and attention (4); event 3 is
 *   recorded right after 2.
 *   seq_lens: NULL, or a decode step over sequences of different lengths
 *   as for hsa_decode_step: device int32 [batch], n_q must be 1, seq_len
 *   is the capacity, the query of sequence b sits at L_b - 1 and this call
 *   rebuilds the landmarks of chunk (L_b - 1) / block of every sequence
 *   (summary_start_block is then not read).
 * Errors: as for the other entry points; nothing is launched on an error.
 */
hsa_sparse_status_t hsa_head_landmarks(const hsa_sparse_shape_t* shape,
                                       const uint16_t* K,
                                       const int8_t* landmark_W,
                                       int32_t start_block, uint16_t* LK,
                                       hsa_sparse_stream_t stream);

hsa_sparse_status_t hsa_head_topm(const hsa_sparse_shape_t* shape,
                                  const uint16_t* Q, const uint16_t* LK,
                                  int32_t* blk, void* workspace,
                                  size_t workspace_bytes,
                                  hsa_sparse_stream_t stream);

hsa_sparse_status_t hsa_forward_heads(const hsa_sparse_shape_t* shape,
                                      const int32_t* seq_lens,
                                      const int8_t* landmark_W,
                                      int32_t summary_start_block,
                                      const uint16_t* Q, const uint16_t* K,
                                      const uint16_t* V, uint16_t* LK,
                                      int32_t* blk_out, float* O, float* lse,
                                      void* workspace, size_t workspace_bytes,
                                      hsa_sparse_stream_t stream);

/*
 * Per-step timing of hsa_forward (profiling aid).  After this call, every
 * hsa_forward, hsa_decode_step, hsa_forward_3level and hsa_forward_heads
 * made by the calling thread records events[0] on its stream before step 1 and events[s] after
 * step s (s = 1..4); a NULL entry is not recorded.  Each recorded event costs the stream a few microseconds, which
 * matters for short (decode) steps, so record only the boundaries needed.
 * Where a decode-shaped call runs two steps in one launch, the events
 * follow the launches: with the token select inside the attention launch,
 * event 3 follows the token scorer and step 4 holds the select; with the
 * token scores inside the block top-m launch as well, event 3 follows
 * event 2 directly.
 * The events are the caller's hipEvent_t handles and must stay valid while
 * such calls are made.  n_events must be 5 with at least one non-NULL
 * entry, or 0 with events == NULL to stop recording.
 */
typedef struct ihipEvent_t* hsa_sparse_event_t;
hsa_sparse_status_t hsa_sparse_set_stage_events(hsa_sparse_event_t const* events, int n_events);

/*
 * Per-kernel timing (profiling aid).  After this call, kernel i (0-based,
 * in launch order) of every entry-point call made by the calling thread
 * carries start[i] and stop[i] in its dispatch, recorded when that kernel
 * starts and ends (hipExtLaunchKernelGGL); NULL entries and kernels past
 * n_events - 1 record nothing.  An event-carrying dispatch costs the stream
 * a few microseconds, so time a sample of calls where steps are short.
 * hsa_sparse_last_kernels() then names the kernels of the thread's last
 * call, comma-separated, in launch order.  The events are the caller's
 * hipEvent_t handles and must stay valid while such calls are made.
 * n_events in [1, 64] with non-NULL arrays, or 0 with both NULL to stop.
 */
hsa_sparse_status_t hsa_sparse_set_kernel_events(hsa_sparse_event_t const* start,
                                                 hsa_sparse_event_t const* stop,
                                                 int n_events);

/* Kernel names of the calling thread's last entry-point call while
 * per-kernel timing is on ("" otherwise).  Valid until the next call. */
const char* hsa_sparse_last_kernels(void);

#ifdef __cplusplus
}
#endif

#endif /* HSA_SPARSE_H */
