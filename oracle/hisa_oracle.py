"""CPU oracle for hierarchical block-then-token sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or run this module.  The product
path never calls it and shares no code with it.

Plain, slow, one query at a time, float64 (exact for the integer-valued
indexer inputs used in every workload).  bf16 tensors are passed as their raw
``uint16`` bit patterns.

Sources (page titles abbreviated; all statements below are restated, not
quoted):

* [HISA] "北大团队改造DeepSeek注意力，速度快四倍还不丢精度" (discuz.ruhao.net),
  the two-step method: step one cuts the context into fixed-size blocks, gives
  each block one summary vector, scores the summaries with the original
  indexer rule and keeps the best m blocks; step two scores only the tokens
  of those blocks with the same rule and keeps k tokens; the first and the
  last block are always kept.  The same page states that the downstream
  sparse attention is unchanged and that on short inputs the method falls
  back to the original flat indexer.
* [HiLS] "把稀疏注意力做对 HiLS-Attention …" (kwkr.cn/news/100279), section
  2.1 (landmark tokens made by a projection summarise each chunk), section 2.2
  (coarse chunk scoring, then exact attention inside the kept chunks) and the
  hils_attention pseudocode (score landmarks, keep top chunks, attend over the
  concatenated K/V of the kept chunks).

Readings where the pages are silent (each one is also listed in the design
notes of the repository):

* the block summary is the mean of the block's indexer keys, computed exactly
  and rounded once to bf16 (round to nearest even); rows beyond the sequence
  end count as zero and the divisor is always B;
* in landmark mode, landmark l of a block is sum_r W[l, r] * kI[row r] / B and
  a block's score is the maximum over its landmarks;
* m counts the two forced blocks; "the last block" is the block holding the
  query position t; a token s is a candidate only if s <= t;
* when the causal blocks (or candidate tokens) number at most m (or k), all
  of them are kept without scoring;
* ties are broken toward the lower index; lists are ascending, padded with -1;
* the indexer selection is shared by all heads; head h reads kv head
  h // (Hq / Hkv); the softmax scale is an input.

Parity pins for every function here are in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16 encoding
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even).

    bf16 keeps the fp64 sign and the top 7 of its 52 fraction bits, so the 45
    low fraction bits are rounded away in one step (no double rounding).
    Domain: zero, or 2**-126 <= |x| < 2**128 (no subnormals, no overflow).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    ax = np.abs(x)
    assert np.all((ax == 0) | ((ax >= 2.0 ** -126) & (ax < 2.0 ** 128))), "outside bf16 normal range"
    u = x.view(np.uint64)
    drop = np.uint64(45)
    half_minus_one = np.uint64((1 << 44) - 1)
    lsb = (u >> drop) & np.uint64(1)
    r = (u + half_minus_one + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = r.view(np.float64).astype(np.float32)  # exact: <= 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# step 1: block summaries  [HISA step one; HiLS section 2.1]
# ---------------------------------------------------------------------------


def block_summary(kI_bits: np.ndarray, block: int, W: np.ndarray | None = None) -> np.ndarray:
    """Summaries of one sequence's key blocks.

    kI_bits: [L, d] bf16 bits.  W: None (mean mode) or [nL, block] integer
    weights (landmark mode).  Returns [nb, nL, d] bf16 bits with
    nb = ceil(L / block).
    """
    L, d = kI_bits.shape
    nb = (L + block - 1) // block
    x = np.zeros((nb * block, d), np.float64)
    x[:L] = bf16_to_f64(kI_bits)
    x = x.reshape(nb, block, d)
    w = np.ones((1, block), np.float64) if W is None else np.asarray(W, np.float64)
    out = np.empty((nb, w.shape[0], d), np.uint16)
    for j in range(nb):
        for l in range(w.shape[0]):
            total = (w[l][:, None] * x[j]).sum(axis=0)
            out[j, l] = f64_to_bf16_rne(total / block)
    return out


# ---------------------------------------------------------------------------
# step 2: block scores and block selection  [HISA step one + forced blocks]
# ---------------------------------------------------------------------------


def block_scores(q_bits: np.ndarray, S_bits: np.ndarray, c: int) -> np.ndarray:
    """score_j = max over landmarks of qI . S[j, l], for blocks j = 0..c."""
    q = bf16_to_f64(q_bits)
    S = bf16_to_f64(S_bits[:c + 1])            # [c+1, nL, d]
    return (S @ q).max(axis=1)


def top_by_score(scores: np.ndarray, ids: np.ndarray, count: int) -> np.ndarray:
    """The `count` ids with the highest score; ties go to the lower id."""
    order = np.lexsort((ids, -scores))
    return ids[order[:count]]


def select_blocks(q_bits: np.ndarray, S_bits: np.ndarray, t: int, block: int, m: int) -> np.ndarray:
    """Kept blocks of the query at position t, ascending, padded with -1 to m."""
    assert m >= 2
    c = t // block
    out = np.full(m, -1, np.int32)
    if c + 1 <= m:
        out[:c + 1] = np.arange(c + 1)
        return out
    scores = block_scores(q_bits, S_bits, c)
    mid = np.arange(1, c)
    kept = top_by_score(scores[1:c], mid, m - 2)
    out[:] = np.sort(np.concatenate([[0, c], kept]))
    return out


# ---------------------------------------------------------------------------
# a third, coarser level: super-blocks of G blocks  [LSA page, latent space
# and hierarchical clustering: the query walks a tree from the root and
# scores only a few nodes per level; here the tree is fixed, contiguous
# runs of blocks, not learned]
# ---------------------------------------------------------------------------


def super_summary(S_bits: np.ndarray, group: int) -> np.ndarray:
    """Summaries of super-blocks of `group` consecutive blocks.

    Reading: a super-block summary is the mean of its blocks' summaries
    (landmark by landmark), summed exactly and rounded once to bf16; missing
    blocks past the end count as zero and the divisor is always `group`,
    like the token rule of block_summary.  S_bits [nb, nL, d] ->
    [ceil(nb / group), nL, d].
    """
    nb, nL, d = S_bits.shape
    nsb = (nb + group - 1) // group
    x = np.zeros((nsb * group, nL, d), np.float64)
    x[:nb] = bf16_to_f64(S_bits)
    x = x.reshape(nsb, group, nL, d)
    out = np.empty((nsb, nL, d), np.uint16)
    for J in range(nsb):
        out[J] = f64_to_bf16_rne(x[J].sum(axis=0) / group)
    return out


def select_blocks_3level(q_bits: np.ndarray, S_bits: np.ndarray, S2_bits: np.ndarray, t: int, block: int,
                         group: int, m2: int, m: int) -> np.ndarray:
    """Kept blocks of the query at position t through a super-block level.

    Reading: the super-blocks are selected exactly like blocks (select_blocks
    at super-block size block * group with m2 kept, the first and the
    query's own super-block forced); the candidate blocks are the blocks
    j <= c = t // block inside the kept super-blocks; all of them are kept if
    they number at most m, else blocks 0 and c plus the best m - 2 of the
    other candidates by block score (ties to the lower index).  Ascending,
    padded with -1 to m.
    """
    assert m >= 2 and m2 >= 2
    c = t // block
    sup = select_blocks(q_bits, S2_bits, t, block * group, m2)
    sup = sup[sup >= 0]
    cand = (sup[:, None] * group + np.arange(group)[None, :]).reshape(-1)
    cand = cand[cand <= c]
    out = np.full(m, -1, np.int32)
    if cand.size <= m:
        out[:cand.size] = cand
        return out
    scores = block_scores(q_bits, S_bits, c)
    mid = cand[(cand != 0) & (cand != c)]
    kept = top_by_score(scores[mid], mid, m - 2)
    out[:] = np.sort(np.concatenate([[0, c], kept]))
    return out


# ---------------------------------------------------------------------------
# step 3: token scores and token selection  [HISA step two]
# ---------------------------------------------------------------------------


def candidate_tokens(blocks: np.ndarray, t: int, block: int) -> np.ndarray:
    """Causal tokens (s <= t) of the kept blocks, ascending."""
    blocks = blocks[blocks >= 0]
    toks = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return toks[toks <= t]


def select_tokens(q_bits: np.ndarray, kI_bits: np.ndarray, blocks: np.ndarray, t: int,
                  block: int, k: int) -> np.ndarray:
    """Kept tokens of the query at position t, ascending, padded with -1 to k."""
    cand = candidate_tokens(blocks, t, block)
    out = np.full(k, -1, np.int32)
    if cand.size <= k:
        out[:cand.size] = cand
        return out
    scores = bf16_to_f64(kI_bits[cand]) @ bf16_to_f64(q_bits)
    out[:] = np.sort(top_by_score(scores, cand, k))
    return out


def flat_topk(q_bits: np.ndarray, kI_bits: np.ndarray, t: int, k: int) -> np.ndarray:
    """The original flat indexer: score every token s <= t, keep k."""
    cand = np.arange(t + 1)
    out = np.full(k, -1, np.int32)
    if cand.size <= k:
        out[:cand.size] = cand
        return out
    scores = bf16_to_f64(kI_bits[:t + 1]) @ bf16_to_f64(q_bits)
    out[:] = np.sort(top_by_score(scores, cand, k))
    return out


# ---------------------------------------------------------------------------
# step 4: sparse attention over the kept tokens  [HISA: unchanged attention;
# HiLS pseudocode step 4]
# ---------------------------------------------------------------------------


def sparse_attention(Q_bits: np.ndarray, K_bits: np.ndarray, V_bits: np.ndarray,
                     tokens: np.ndarray, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of one query over its kept K/V rows.

    Q_bits [Hq, d]; K_bits, V_bits [L, Hkv, d]; tokens: index list (-1 = pad).
    Returns O [Hq, d] and lse [Hq] (natural log of the softmax denominator).
    """
    Hq, d = Q_bits.shape
    Hkv = K_bits.shape[1]
    group = Hq // Hkv
    tok = tokens[tokens >= 0]
    q = bf16_to_f64(Q_bits)
    O = np.empty((Hq, d), np.float64)
    lse = np.empty(Hq, np.float64)
    for h in range(Hq):
        g = h // group
        k = bf16_to_f64(K_bits[tok, g])
        v = bf16_to_f64(V_bits[tok, g])
        z = scale * (k @ q[h])
        zmax = z.max()
        p = np.exp(z - zmax)
        denom = p.sum()
        O[h] = (p @ v) / denom
        lse[h] = zmax + np.log(denom)
    return O, lse


# ---------------------------------------------------------------------------
# per-head selection from the attention queries  [HiLS pseudocode: the
# landmark scores come from Q itself against the chunks' landmarks, and the
# exact attention runs over the concatenated K/V of the kept chunks]
# ---------------------------------------------------------------------------


def head_landmarks(K_bits: np.ndarray, block: int, W: np.ndarray | None = None) -> np.ndarray:
    """Landmarks of one sequence's attention keys, per kv head.

    K_bits [L, Hkv, d] -> [nb, nL, Hkv, d]: kv head g's landmarks are the
    block summary (block_summary) of its key rows K[:, g].  The float64 sums
    of bf16 keys are exact while the values' exponents span < 45 bits (true
    for the N(0, 1) keys of every workload), so one rounding to bf16.
    """
    return np.stack([block_summary(K_bits[:, g, :], block, W) for g in range(K_bits.shape[1])], axis=2)


def forward_query_heads(seq: dict, b: int, i: int, t: int, block: int, m: int, scale: float,
                        LK_bits: np.ndarray, attention: bool = True, blk_override: np.ndarray | None = None) -> dict:
    """Per-head chunk selection and attention for query i (position t) of sequence b.

    Query head h (kv head g = h // (Hq / Hkv)) ranks the causal chunks by
    max_l Q[h] . LK[j, l, g] with the block rule of select_blocks (first and
    own chunk kept, m in all), then attends over every token s <= t of its
    kept chunks.  blk_override [Hq, m] replaces the selection (to evaluate
    the attention of a given selection).  Returns blk [Hq, m], O [Hq, d],
    lse [Hq].
    """
    Q = seq["Q"][b, i]
    Hq, Hkv = Q.shape[0], seq["K"].shape[2]
    group = Hq // Hkv
    blk = np.empty((Hq, m), np.int32)
    res = {"blk": blk}
    if attention:
        res["O"] = np.empty((Hq, Q.shape[1]), np.float64)
        res["lse"] = np.empty(Hq, np.float64)
    for h in range(Hq):
        g = h // group
        blk[h] = select_blocks(Q[h], LK_bits[:, :, g, :], t, block, m) if blk_override is None else blk_override[h]
        if attention:
            tok = candidate_tokens(blk[h], t, block)
            O, lse = sparse_attention(Q[h:h + 1], seq["K"][b][:, g:g + 1], seq["V"][b][:, g:g + 1], tok, scale)
            res["O"][h], res["lse"][h] = O[0], lse[0]
    return res


# ---------------------------------------------------------------------------
# the whole path for one query
# ---------------------------------------------------------------------------


def forward_query_3level(seq: dict, b: int, i: int, t: int, block: int, group: int, m2: int, m: int, k: int,
                         scale: float, S_bits: np.ndarray, S2_bits: np.ndarray, attention: bool = True) -> dict:
    """forward_query with the block list chosen through super-blocks."""
    q = seq["qI"][b, i]
    blk = select_blocks_3level(q, S_bits, S2_bits, t, block, group, m2, m)
    tok = select_tokens(q, seq["kI"][b], blk, t, block, k)
    res = {"blk": blk, "tok": tok}
    if attention:
        res["O"], res["lse"] = sparse_attention(seq["Q"][b, i], seq["K"][b], seq["V"][b], tok, scale)
    return res


def forward_query(seq: dict, b: int, i: int, t: int, block: int, m: int, k: int,
                  scale: float, S_bits: np.ndarray | None = None,
                  attention: bool = True) -> dict:
    """Steps 1-4 for query i (position t) of sequence b.

    seq holds qI [b, nq, dI], kI [b, L, dI], optional W, and (for attention)
    Q [b, nq, Hq, d], K and V [b, L, Hkv, d], all bf16 bits.
    """
    if S_bits is None:
        S_bits = block_summary(seq["kI"][b], block, seq.get("W"))
    q = seq["qI"][b, i]
    blk = select_blocks(q, S_bits, t, block, m)
    tok = select_tokens(q, seq["kI"][b], blk, t, block, k)
    res = {"blk": blk, "tok": tok}
    if attention:
        res["O"], res["lse"] = sparse_attention(seq["Q"][b, i], seq["K"][b], seq["V"][b], tok, scale)
    return res


def scored_items(t: int, block: int, m: int, k: int) -> int:
    """How many block summaries plus tokens the oracle ranks (scores and compares
    in a top selection) for the query at t; forced blocks and the candidates
    of a list that keeps all of them are not ranked."""
    c = t // block
    n_blocks = 0 if c + 1 <= m else c - 1
    cand = (t + 1) if c + 1 <= m else (m - 1) * block + (t - c * block + 1)
    n_tokens = 0 if cand <= k else cand
    return n_blocks + n_tokens
