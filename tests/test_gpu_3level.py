"""GPU parity of the three-level selection (super-blocks -> blocks -> tokens).

Super-block summaries, super-block lists and block lists are compared bit
for bit with the oracle's super_summary, select_blocks at super-block size
and select_blocks_3level (pinned in test_oracle_3level.py); the token lists
and attention of hsa_forward_3level with the oracle's forward_query_3level
(lists bit for bit, O and lse within 2e-3).  The cases cover the level-1
paths of the block top-m launcher (MFMA scores for many queries, the GEMV
with landmarks), both level-2 workgroup shapes, the one-launch decode
kernel of both levels (with and without the newest summaries folded in),
super-blocks of one block (the two-level lists), every super-block kept,
the full decode_3level_1m shape on sampled sequences, and decode steps over
sequences of different lengths (seq_lens) against the oracle per sequence.
"""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload
from oracle import hisa_oracle as orc
from parity import ATOL, oracle_summaries

pytestmark = pytest.mark.gpu


def case(name, batch, L, nq, dI, B, nL, m, k, G, m2, Hq=4, Hkv=1):
    return Workload(name=name, batch=batch, seq_len=L, n_q=nq, d_index=dI, block=B, top_m=m, top_k=k,
                    n_heads_q=Hq, n_heads_kv=Hkv, n_landmarks=nL, group=G, top_m2=m2)


CASES = [
    # (workload, value range): small ranges give many tied scores
    (case("prefill_mfma_l1", 1, 6000, 600, 128, 16, 1, 12, 100, 4, 6), 2),
    (case("decode_one_launch_l1", 3, 20000, 2, 64, 16, 1, 20, 200, 8, 10), 2),
    (case("landmarks_gemv_l1", 2, 9000, 3, 128, 32, 4, 8, 150, 4, 5), 3),
    (case("lm2_prefill", 1, 3000, 700, 64, 8, 2, 10, 60, 8, 4), 2),
    (case("group1_is_two_level", 1, 2000, 300, 64, 16, 1, 6, 50, 1, 6), 2),
    (case("wide_level2", 1, 70000, 2, 128, 8, 1, 300, 600, 64, 40, Hq=8, Hkv=2), 2),
    (case("every_super_kept", 2, 1500, 50, 64, 16, 1, 5, 40, 8, 100), 2),
    (case("m_equals_2", 2, 5000, 20, 64, 16, 1, 2, 30, 4, 3), 2),
    # one-launch decode path at its widest: 1998 level-1 keys (R1 = 2) and
    # 4800 level-2 slots (R2 = 8)
    (case("one_launch_r2_r8", 2, 128000, 3, 64, 8, 1, 300, 400, 8, 600), 2),
    # fewer level-2 candidates than m (2 super-blocks of 8 blocks: at most 16
    # blocks for m = 31): the lists are shorter than min(c + 1, m) and the
    # token stage (block-major scoring here) must take their length from them
    (case("fewer_candidates_than_m", 2, 10100, 118, 128, 32, 1, 31, 209, 8, 2), 2),
    (case("fewer_candidates_decode", 3, 20000, 1, 64, 16, 1, 40, 100, 4, 3), 2),
    (case("fewer_candidates_keep_all", 1, 9000, 50, 64, 16, 1, 60, 960, 8, 2), 2),
    # the same in decode with the token select inside the attention launch:
    # at most 20 (select) or 12 (keep all) blocks for m = 40
    (case("fewer_candidates_select_attn", 2, 20000, 1, 64, 16, 1, 40, 256, 4, 5), 2),
    (case("fewer_candidates_select_attn_keep_all", 2, 20000, 1, 64, 16, 1, 40, 256, 4, 3), 2),
]


def make(w, vr):
    return datagen.make_inputs(w, q_range=vr, centre_range=max(1, vr // 2), noise_range=max(1, vr // 2))


def oracle_lists(inp, w, S, S2, b, i):
    q = inp["qI"][b, i]
    t = w.query_pos(i)
    sup = orc.select_blocks(q, S2, t, w.block * w.group, w.top_m2)
    blk = orc.select_blocks_3level(q, S, S2, t, w.block, w.group, w.top_m2, w.top_m)
    return sup, blk


@pytest.mark.parametrize("w,vr", CASES, ids=[c[0].name for c in CASES])
def test_three_level_all_queries(w, vr):
    inp = make(w, vr)
    dev = pipeline.to_device(inp)
    shape = _lib.shape_of(w)
    # stage by stage
    st = pipeline.alloc_outputs(w)
    _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, st["S"])
    _lib.hsa_super_summary(shape, w.group, st["S"], 0, st["S2"])
    _lib.hsa_block_topm_3level(shape, w.group, w.top_m2, dev["qI"], st["S"], st["S2"], st["sup"], st["blk"])
    torch.cuda.synchronize()
    g = pipeline.to_host(st)
    S = oracle_summaries(inp, w)
    assert np.array_equal(g["S"], S)
    S2 = np.stack([orc.super_summary(S[b], w.group) for b in range(w.batch)])
    assert np.array_equal(g["S2"], S2), "super-block summaries differ"
    for b in range(w.batch):
        for i in range(w.n_q):
            sup, blk = oracle_lists(inp, w, S[b], S2[b], b, i)
            ctx = f"{w.name} b={b} i={i} t={w.query_pos(i)}"
            assert np.array_equal(g["sup"][b, i], sup), f"super-block list differs: {ctx}"
            assert np.array_equal(g["blk"][b, i], blk), f"block list differs: {ctx}"
    # the fused entry point: same lists, then tokens and attention
    f = pipeline.to_host(pipeline.run_forward_3level(w, dev))
    for key in ("S", "S2", "sup", "blk"):
        assert np.array_equal(f[key], g[key]), key
    qs = [(b, i) for b in range(w.batch) for i in range(w.n_q)]
    if len(qs) > 150:
        rng = np.random.default_rng(3)
        qs = sorted(set([qs[j] for j in rng.choice(len(qs), 120, replace=False)] + qs[:8] + qs[-8:]))
    for b, i in qs:
        r = orc.forward_query_3level(inp, b, i, w.query_pos(i), w.block, w.group, w.top_m2, w.top_m, w.top_k,
                                     w.scale, S[b], S2[b])
        ctx = f"{w.name} b={b} i={i}"
        assert np.array_equal(f["tok"][b, i], r["tok"]), f"token list differs: {ctx}"
        assert np.abs(f["O"][b, i].astype(np.float64) - r["O"]).max() <= ATOL, ctx
        assert np.abs(f["lse"][b, i].astype(np.float64) - r["lse"]).max() <= ATOL, ctx


def test_group1_matches_two_level_forward():
    # super-blocks of one block with m2 = m: the two-level hsa_forward bits
    w = case("g1", 2, 5000, 40, 128, 32, 2, 7, 90, 1, 7)
    inp = make(w, 3)
    dev = pipeline.to_device(inp)
    a = pipeline.to_host(pipeline.run_forward(w, dev))
    b = pipeline.to_host(pipeline.run_forward_3level(w, dev))
    for key in ("S", "blk", "tok", "O", "lse"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key
    assert np.array_equal(b["S2"], b["S"])


def test_incremental_super_summaries():
    # summary_start_block > 0: only the touched blocks and super-blocks are
    # recomputed; with the earlier state in S and S2 the results equal a full call
    w = case("inc3", 2, 9000, 100, 64, 16, 1, 10, 120, 8, 6)
    inp = make(w, 2)
    dev = pipeline.to_device(inp)
    full = pipeline.to_host(pipeline.run_forward_3level(w, dev))
    start = (w.seq_len - w.n_q) // w.block
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, out["S"])
    _lib.hsa_super_summary(shape, w.group, out["S"], 0, out["S2"])
    out["S"][:, start:] = 0
    out["S2"][:, start // w.group:] = 0
    inc = pipeline.to_host(pipeline.run_forward_3level(w, dev, out, summary_start_block=start))
    for key in ("S", "S2", "sup", "blk", "tok", "O", "lse"):
        assert np.array_equal(inc[key], full[key], equal_nan=True), key


FOLD_CASES = [
    # (batch, L, n_q, d_index, B, G, m2, m, k): every query in the last block,
    # so the newest block's and super-block's summaries are rebuilt inside the
    # selection launch; the second has a partial last block and super-block
    (3, 20000, 1, 64, 16, 8, 10, 20, 200),
    (2, 128005, 2, 128, 8, 8, 600, 300, 400),
    (2, 7000, 3, 128, 32, 4, 3, 6, 64),
]


@pytest.mark.parametrize("batch,L,nq,dI,B,G,m2,m,k", FOLD_CASES)
def test_decode_fold_3level(batch, L, nq, dI, B, G, m2, m, k):
    w = case("fold3", batch, L, nq, dI, B, 1, m, k, G, m2)
    assert (L - nq) // B == (L - 1) // B
    inp = make(w, 2)
    dev = pipeline.to_device(inp)
    full = pipeline.to_host(pipeline.run_forward_3level(w, dev))
    c_max = (L - 1) // B
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, out["S"])
    _lib.hsa_super_summary(shape, w.group, out["S"], 0, out["S2"])
    out["S"][:, c_max:] = 0      # stale state for the newest block and super-block
    out["S2"][:, c_max // G:] = 0
    inc = pipeline.to_host(pipeline.run_forward_3level(w, dev, out, summary_start_block=c_max))
    for key in ("S", "S2", "sup", "blk", "tok", "O", "lse"):
        assert np.array_equal(inc[key], full[key], equal_nan=True), key
    S = oracle_summaries(inp, w)
    S2 = np.stack([orc.super_summary(S[b], G) for b in range(batch)])
    assert np.array_equal(inc["S"], S) and np.array_equal(inc["S2"], S2)
    for b in range(batch):
        for i in range(nq):
            r = orc.forward_query_3level(inp, b, i, w.query_pos(i), B, G, m2, m, k, w.scale, S[b], S2[b])
            assert np.array_equal(inc["blk"][b, i], r["blk"]), (b, i)
            assert np.array_equal(inc["tok"][b, i], r["tok"]), (b, i)
            assert np.abs(inc["O"][b, i].astype(np.float64) - r["O"]).max() <= ATOL


def test_decode_3level_1m_sampled():
    # the bench shape: batch 8, L = 1048576, super-blocks of 16 blocks; list
    # invariants on every sequence, the oracle on three of them
    w = WORKLOADS["decode_3level_1m"]
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    # bench.py's configuration: state built first, then the step from the
    # newest block (its summary and its super-block's folded into the launch)
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, out["S"])
    _lib.hsa_super_summary(shape, w.group, out["S"], 0, out["S2"])
    start = (w.seq_len - w.n_q) // w.block
    out["S"][:, start:] = 0
    out["S2"][:, start // w.group:] = 0
    g = pipeline.to_host(pipeline.run_forward_3level(w, dev, out, summary_start_block=start))
    t = w.query_pos(0)
    c, C = t // w.block, t // (w.block * w.group)
    for b in range(w.batch):
        sup, blk, tok = g["sup"][b, 0], g["blk"][b, 0], g["tok"][b, 0]
        assert sup[0] == 0 and sup[-1] == C and np.all(np.diff(sup) > 0)
        assert blk[0] == 0 and blk[-1] == c and np.all(np.diff(blk) > 0)
        assert set((blk // w.group).tolist()) <= set(sup.tolist())
        assert np.all(np.diff(tok) > 0) and set((tok // w.block).tolist()) <= set(blk.tolist())
        # the planted needle blocks survive both levels
        assert set(inp["needles"][b].tolist()) <= set(blk.tolist()), b
    for b in (0, 3, w.batch - 1):
        S = orc.block_summary(inp["kI"][b], w.block)
        assert np.array_equal(g["S"][b], S)
        S2 = orc.super_summary(S, w.group)
        assert np.array_equal(g["S2"][b], S2)
        r = orc.forward_query_3level(inp, b, 0, t, w.block, w.group, w.top_m2, w.top_m, w.top_k, w.scale, S, S2)
        assert np.array_equal(g["sup"][b, 0], orc.select_blocks(inp["qI"][b, 0], S2, t, w.block * w.group,
                                                                w.top_m2))
        assert np.array_equal(g["blk"][b, 0], r["blk"]), b
        assert np.array_equal(g["tok"][b, 0], r["tok"]), b
        assert np.abs(g["O"][b, 0].astype(np.float64) - r["O"]).max() <= ATOL
        assert np.abs(g["lse"][b, 0].astype(np.float64) - r["lse"]).max() <= ATOL


# (batch, capacity, d_index, B, n_L, G, m2, m, k, start lengths): the first
# takes the one-launch decode kernel with the newest block and super-block
# folded in, the second (landmarks) the block-summary and super-summary
# launches, the level-1 block top-m and the level-2 kernel
VARLEN_CASES = [
    (5, 20000, 64, 16, 1, 8, 10, 20, 200, [20000, 9999, 16 * 8 * 3 - 1, 16 * 8 * 3 + 1, 1]),
    (3, 9000, 128, 32, 4, 4, 5, 8, 150, [8998, 4096, 31]),
]


@pytest.mark.parametrize("batch,cap,dI,B,nL,G,m2,m,k,lens0", VARLEN_CASES, ids=["one_launch", "landmarks"])
def test_decode_3level_different_lengths(batch, cap, dI, B, nL, G, m2, m, k, lens0):
    # sequences of different lengths in one capacity-sized cache (seq_lens,
    # n_q = 1); state built over the whole capacity first, so the summaries
    # of every sequence's newest block and super-block are stale; then three
    # steps appending one token to every sequence (crossing block and
    # super-block boundaries) with the state carried between steps.  Each
    # sequence is compared with the oracle run on its first L_b rows.
    w = case("varlen3", batch, cap, 1, dI, B, nL, m, k, G, m2)
    inp = make(w, 2)
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, out["S"])
    _lib.hsa_super_summary(shape, G, out["S"], 0, out["S2"])
    for step in range(3):
        lens = [min(L + step, cap) for L in lens0]
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        g = pipeline.to_host(pipeline.run_forward_3level(w, dev, out, summary_start_block=0, seq_lens=lt))
        for b, Lb in enumerate(lens):
            t = Lb - 1
            ctx = f"step {step} b={b} L_b={Lb}"
            S_b = orc.block_summary(inp["kI"][b, :Lb], B, inp.get("W"))
            S2_b = orc.super_summary(S_b, G)
            assert np.array_equal(g["S"][b, :S_b.shape[0]], S_b), f"summaries differ: {ctx}"
            assert np.array_equal(g["S2"][b, :S2_b.shape[0]], S2_b), f"super-block summaries differ: {ctx}"
            r = orc.forward_query_3level(inp, b, 0, t, B, G, m2, m, k, w.scale, S_b, S2_b)
            sup = orc.select_blocks(inp["qI"][b, 0], S2_b, t, B * G, m2)
            assert np.array_equal(g["sup"][b, 0], sup), f"super-block list differs: {ctx}"
            assert np.array_equal(g["blk"][b, 0], r["blk"]), f"block list differs: {ctx}"
            assert np.array_equal(g["tok"][b, 0], r["tok"]), f"token list differs: {ctx}"
            assert np.abs(g["O"][b, 0].astype(np.float64) - r["O"]).max() <= ATOL, ctx
            assert np.abs(g["lse"][b, 0].astype(np.float64) - r["lse"]).max() <= ATOL, ctx


def test_standalone_token_topk_on_three_level_lists():
    # hsa_block_topm_3level's lists (shorter than min(c + 1, m) here: two
    # super-blocks of 4 blocks for m = 20) through the standalone
    # hsa_token_topk and hsa_sparse_attn, against the oracle
    w = case("standalone_short_lists", 2, 6000, 40, 64, 16, 1, 20, 90, 4, 2)
    inp = make(w, 2)
    dev = pipeline.to_device(inp)
    shape = _lib.shape_of(w)
    st = pipeline.alloc_outputs(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, st["S"])
    _lib.hsa_super_summary(shape, w.group, st["S"], 0, st["S2"])
    _lib.hsa_block_topm_3level(shape, w.group, w.top_m2, dev["qI"], st["S"], st["S2"], st["sup"], st["blk"])
    _lib.hsa_token_topk(shape, dev["qI"], dev["kI"], st["blk"], st["tok"])
    _lib.hsa_sparse_attn(shape, dev["Q"], dev["K"], dev["V"], st["tok"], st["O"], st["lse"])
    torch.cuda.synchronize()
    g = pipeline.to_host(st)
    S = oracle_summaries(inp, w)
    S2 = np.stack([orc.super_summary(S[b], w.group) for b in range(w.batch)])
    short = 0
    for b in range(w.batch):
        for i in range(w.n_q):
            t = w.query_pos(i)
            r = orc.forward_query_3level(inp, b, i, t, w.block, w.group, w.top_m2, w.top_m, w.top_k, w.scale, S[b],
                                         S2[b])
            ctx = f"b={b} i={i} t={t}"
            assert np.array_equal(g["blk"][b, i], r["blk"]), ctx
            assert np.array_equal(g["tok"][b, i], r["tok"]), ctx
            assert np.abs(g["O"][b, i].astype(np.float64) - r["O"]).max() <= ATOL, ctx
            short += int((r["blk"] >= 0).sum() < min(t // w.block + 1, w.top_m))
    assert short > 0  # the case does exercise lists shorter than min(c + 1, m)
