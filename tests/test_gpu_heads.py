"""GPU parity of the per-head chunk selection (hsa_head_landmarks,
hsa_head_topm, hsa_forward_heads) against the CPU oracle.

The landmarks are summed exactly (fp64) on both sides and compared bit for
bit.  The chunk scores are fp32 dot products of float-valued bf16 vectors,
so two chunks whose exact scores differ by less than the rounding of a
128-term dot product may be ranked either way: each (query, head) list is
checked for the forced chunks and its shape, then against the exact (fp64)
scores with a bound on that rounding: every kept chunk's score plus its
bound must reach every dropped chunk's score minus its bound (any list
an exact fp32 top-m could produce passes; a wrong chunk outside the band
fails).  Lists equal to the oracle's are counted.  Attention is compared
with the oracle evaluated on the GPU's lists, within 2e-3.
"""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload
from oracle import hisa_oracle as orc
from parity import ATOL

pytestmark = pytest.mark.gpu

# rounding bound of a 128-term fp32 dot product of exact products, in any
# summation order: (n - 1) * 2^-24 * sum |terms|, doubled for margin
GAMMA = 2 * 127 * 2.0 ** -24


def case(name, batch, L, nq, B, nL, m, Hq, Hkv):
    return Workload(name=name, batch=batch, seq_len=L, n_q=nq, d_index=128, block=B, top_m=m, top_k=m * B,
                    n_heads_q=Hq, n_heads_kv=Hkv, n_landmarks=nL, per_head=True)


def exact_scores(q, LKg):
    """q [d], LKg [nb, nL, d] (float64): chunk scores max_l q . LK[j, l] and
    their fp32 rounding bounds."""
    prod = LKg * q
    s = prod.sum(-1)
    err = GAMMA * np.abs(prod).sum(-1)
    return s.max(1), err.max(1)


def check_list(blk, t, B, m, score, eps, ctx):
    c = t // B
    kept = blk[blk >= 0]
    assert np.all(blk[kept.size:] == -1) and np.all(np.diff(kept) > 0), ctx
    if c + 1 <= m:
        assert np.array_equal(kept, np.arange(c + 1)), ctx
        return
    assert kept.size == m and kept[0] == 0 and kept[-1] == c, ctx
    if m == 2:
        return
    mid = kept[1:-1]
    dropped = np.setdiff1d(np.arange(1, c), mid)
    lo = (score[mid] + eps[mid]).min()
    hi = (score[dropped] - eps[dropped]).max()
    assert lo >= hi, f"kept chunk below a dropped one beyond the fp32 bound: {ctx} ({lo} < {hi})"


def check_heads(w, inp, g, LK, queries, attn_queries, stats):
    Hq, Hkv = w.n_heads_q, w.n_heads_kv
    qpg = Hq // Hkv
    LKf = orc.bf16_to_f64(LK)
    for b, i in queries:
        t = w.query_pos(i)
        Qf = orc.bf16_to_f64(inp["Q"][b, i])
        for h in range(Hq):
            score, eps = exact_scores(Qf[h], LKf[b][:, :, h // qpg, :])
            ctx = f"{w.name} b={b} i={i} t={t} h={h}"
            check_list(g["blk"][b, i, h], t, w.block, w.top_m, score, eps, ctx)
            ref = orc.select_blocks(inp["Q"][b, i, h], LK[b][:, :, h // qpg, :], t, w.block, w.top_m)
            stats["lists"] += 1
            stats["equal"] += int(np.array_equal(ref, g["blk"][b, i, h]))
    for b, i in attn_queries:
        t = w.query_pos(i)
        r = orc.forward_query_heads(inp, b, i, t, w.block, w.top_m, w.scale, LK[b], blk_override=g["blk"][b, i])
        ctx = f"{w.name} b={b} i={i}"
        assert np.abs(g["O"][b, i].astype(np.float64) - r["O"]).max() <= ATOL, ctx
        assert np.abs(g["lse"][b, i].astype(np.float64) - r["lse"]).max() <= ATOL, ctx


CASES = [
    case("decode_gqa8", 3, 5000, 1, 32, 4, 8, 16, 2),
    case("prefill_gqa4", 1, 1200, 1200, 16, 1, 6, 8, 2),
    case("mha_lm2", 2, 3000, 5, 64, 2, 5, 4, 4),
    case("keep_all", 1, 300, 300, 32, 1, 20, 2, 1),
    case("m_equals_2", 2, 2000, 3, 16, 1, 2, 4, 1),
    case("ragged_wide_select", 1, 40017, 2, 8, 1, 300, 16, 1),
    case("qpg16_lm4", 1, 4096, 64, 64, 4, 8, 16, 1),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_per_head_selection(w):
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    shape = _lib.shape_of(w)
    st = pipeline.alloc_outputs(w)
    _lib.hsa_head_landmarks(shape, dev["K"], dev.get("W"), 0, st["LK"])
    _lib.hsa_head_topm(shape, dev["Q"], st["LK"], st["blk"])
    torch.cuda.synchronize()
    g = pipeline.to_host(st)
    LK = np.stack([orc.head_landmarks(inp["K"][b], w.block, inp.get("W")) for b in range(w.batch)])
    assert np.array_equal(g["LK"], LK), "landmarks differ"
    f = pipeline.to_host(pipeline.run_forward_heads(w, dev))
    assert np.array_equal(f["LK"], g["LK"]) and np.array_equal(f["blk"], g["blk"])
    qs = [(b, i) for b in range(w.batch) for i in range(w.n_q)]
    aq = qs
    if len(qs) > 60:
        rng = np.random.default_rng(1)
        qs = sorted(set([qs[j] for j in rng.choice(len(qs), min(200, len(qs)), replace=False)] + qs[:4] + qs[-4:]))
        aq = qs[::5] + qs[-2:]
    stats = {"lists": 0, "equal": 0}
    check_heads(w, inp, f, LK, qs, aq, stats)
    print(f"{w.name}: {stats['equal']} of {stats['lists']} lists equal to the oracle's")


def test_incremental_landmarks():
    # summary_start_block > 0 with stale state from there on gives the bits
    # of a full call
    w = case("inc_heads", 2, 3000, 2, 32, 2, 6, 8, 2)
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    full = pipeline.to_host(pipeline.run_forward_heads(w, dev))
    start = (w.seq_len - w.n_q) // w.block
    out = pipeline.alloc_outputs(w)
    _lib.hsa_head_landmarks(_lib.shape_of(w), dev["K"], dev["W"], 0, out["LK"])
    out["LK"][:, start:] = 0
    inc = pipeline.to_host(pipeline.run_forward_heads(w, dev, out, summary_start_block=start))
    for key in ("LK", "blk", "O", "lse"):
        assert np.array_equal(inc[key], full[key], equal_nan=True), key


@pytest.mark.parametrize("batch,L,nq,B,nL,m,Hq,Hkv", [
    (3, 5000, 1, 32, 4, 8, 16, 2),       # decode: the newest chunk's landmarks folded into the score launch
    (2, 7001, 2, 64, 1, 6, 8, 8),        # two queries in the last, partial chunk
    (1, 100, 1, 16, 2, 20, 4, 1),        # every chunk kept: no score launch, landmarks on their own
])
def test_decode_fold_heads(batch, L, nq, B, nL, m, Hq, Hkv):
    w = case("fold_heads", batch, L, nq, B, nL, m, Hq, Hkv)
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    full = pipeline.to_host(pipeline.run_forward_heads(w, dev))
    c_max = (L - 1) // B
    out = pipeline.alloc_outputs(w)
    _lib.hsa_head_landmarks(_lib.shape_of(w), dev["K"], dev.get("W"), 0, out["LK"])
    out["LK"][:, c_max:] = 0
    inc = pipeline.to_host(pipeline.run_forward_heads(w, dev, out, summary_start_block=c_max))
    for key in ("LK", "blk", "O", "lse"):
        assert np.array_equal(inc[key], full[key], equal_nan=True), key
    LK = np.stack([orc.head_landmarks(inp["K"][b], B, inp.get("W")) for b in range(batch)])
    assert np.array_equal(inc["LK"], LK)
    stats = {"lists": 0, "equal": 0}
    qs = [(b, i) for b in range(batch) for i in range(nq)]
    check_heads(w, inp, inc, LK, qs, qs, stats)


def test_one_head_matches_shared_indexer_kernels():
    # Hq = Hkv = 1, nL = 1: the per-head path's landmarks are the block
    # summaries of K.  Every list passes the exact-score margin check; O and
    # lse match the oracle evaluated on the GPU's lists; and wherever the
    # list equals the shared-indexer oracle's (qI := Q, kI := K, k = m * B),
    # O matches that path's output too
    w = case("one_head", 2, 2500, 3, 16, 1, 7, 1, 1)
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    g = pipeline.to_host(pipeline.run_forward_heads(w, dev))
    shared = {"qI": inp["Q"][:, :, 0], "kI": inp["K"][:, :, 0], "Q": inp["Q"], "K": inp["K"], "V": inp["V"]}
    equal = 0
    for b in range(w.batch):
        S = orc.block_summary(inp["K"][b][:, 0], w.block)
        assert np.array_equal(g["LK"][b][:, :, 0], S)
        Sf = orc.bf16_to_f64(S)
        for i in range(w.n_q):
            t = w.query_pos(i)
            score, eps = exact_scores(orc.bf16_to_f64(inp["Q"][b, i, 0]), Sf)
            check_list(g["blk"][b, i, 0], t, w.block, w.top_m, score, eps, f"one_head b={b} i={i}")
            r = orc.forward_query_heads(inp, b, i, t, w.block, w.top_m, w.scale, S[:, :, None, :],
                                        blk_override=g["blk"][b, i])
            assert np.abs(g["O"][b, i] - r["O"]).max() <= ATOL, (b, i)
            assert np.abs(g["lse"][b, i] - r["lse"]).max() <= ATOL, (b, i)
            rs = orc.forward_query(shared, b, i, t, w.block, w.top_m, w.top_m * w.block, w.scale, S_bits=S)
            if np.array_equal(rs["blk"], g["blk"][b, i, 0]):
                equal += 1
                assert np.abs(g["O"][b, i] - rs["O"]).max() <= ATOL, (b, i)
    print(f"one_head: {equal} of {w.batch * w.n_q} lists equal to the shared-indexer oracle's")


def test_head_decode_512k():
    # the bench shape: every head's list is checked for shape and forced
    # chunks, every planted needle chunk is kept by its head, and every
    # sequence's 32 head lists are checked against the exact scores, with
    # O and lse against the oracle on the GPU's lists
    w = WORKLOADS["head_decode_512k"]
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    # bench.py's configuration: landmarks built first, then the step from the
    # newest chunk (its landmarks folded into the select launch)
    out = pipeline.alloc_outputs(w)
    _lib.hsa_head_landmarks(_lib.shape_of(w), dev["K"], dev["W"], 0, out["LK"])
    start = (w.seq_len - w.n_q) // w.block
    out["LK"][:, start:] = 0
    g = pipeline.to_host(pipeline.run_forward_heads(w, dev, out, summary_start_block=start))
    del dev, out
    torch.cuda.empty_cache()
    t = w.query_pos(0)
    c = t // w.block
    for b in range(w.batch):
        for h in range(w.n_heads_q):
            blk = g["blk"][b, 0, h]
            assert blk[0] == 0 and blk[-1] == c and np.all(np.diff(blk) > 0), (b, h)
        for gk in range(w.n_heads_kv):
            j, h = inp["head_needles"][b, gk]
            assert j in g["blk"][b, 0, h], (b, gk, j, h)
    stats = {"lists": 0, "equal": 0}
    for b in range(w.batch):
        LKb = orc.head_landmarks(inp["K"][b], w.block, inp["W"])
        assert np.array_equal(g["LK"][b], LKb), f"landmarks of sequence {b} differ"
        sub = {"Q": inp["Q"][b:b + 1], "K": inp["K"][b:b + 1], "V": inp["V"][b:b + 1], "W": inp["W"]}
        check_heads(w.with_(batch=1), sub, {k: v[b:b + 1] for k, v in g.items()}, LKb[None], [(0, 0)], [(0, 0)],
                    stats)
    print(f"head_decode_512k: {stats['equal']} of {stats['lists']} lists equal to the oracle's")


def _check_varlen_step(w, inp, g, lens, stats):
    qpg = w.n_heads_q // w.n_heads_kv
    for b, Lb in enumerate(lens):
        t = Lb - 1
        LK_b = orc.head_landmarks(inp["K"][b, :Lb], w.block, inp.get("W"))
        assert np.array_equal(g["LK"][b, :LK_b.shape[0]], LK_b), f"landmarks differ: b={b} L_b={Lb}"
        LKf = orc.bf16_to_f64(LK_b)
        Qf = orc.bf16_to_f64(inp["Q"][b, 0])
        for h in range(w.n_heads_q):
            score, eps = exact_scores(Qf[h], LKf[:, :, h // qpg, :])
            check_list(g["blk"][b, 0, h], t, w.block, w.top_m, score, eps, f"b={b} L_b={Lb} h={h}")
            ref = orc.select_blocks(inp["Q"][b, 0, h], LK_b[:, :, h // qpg, :], t, w.block, w.top_m)
            stats["lists"] += 1
            stats["equal"] += int(np.array_equal(ref, g["blk"][b, 0, h]))
        seq = {"Q": inp["Q"][b:b + 1], "K": inp["K"][b:b + 1, :Lb], "V": inp["V"][b:b + 1, :Lb]}
        r = orc.forward_query_heads(seq, 0, 0, t, w.block, w.top_m, w.scale, LK_b, blk_override=g["blk"][b, 0])
        assert np.abs(g["O"][b, 0].astype(np.float64) - r["O"]).max() <= ATOL, (b, Lb)
        assert np.abs(g["lse"][b, 0].astype(np.float64) - r["lse"]).max() <= ATOL, (b, Lb)


def test_per_head_decode_different_lengths():
    # one decode step over sequences of different lengths (seq_lens, n_q = 1):
    # each sequence against the oracle run on its own first L_b rows; then
    # three steps appending a token to every sequence, carrying LK, across
    # a chunk boundary
    w = case("varlen_heads", 5, 6000, 1, 32, 4, 8, 16, 2)
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    _lib.hsa_head_landmarks(_lib.shape_of(w), dev["K"], dev["W"], 0, out["LK"])
    stats = {"lists": 0, "equal": 0}
    for lens in ([6000, 3001, 32 * 7, 32 * 8 + 1, 1], [5998, 32 * 40 - 2, 32 * 8 - 1, 9, 2]):
        for step in range(3 if lens[0] == 5998 else 1):
            cur = [L + step for L in lens]
            lt = torch.tensor(cur, dtype=torch.int32, device="cuda")
            g = pipeline.to_host(pipeline.run_forward_heads(w, dev, out, seq_lens=lt))
            _check_varlen_step(w, inp, g, cur, stats)
    print(f"varlen heads: {stats['equal']} of {stats['lists']} lists equal to the oracle's")
