"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Index sets (summaries, block lists, token lists) must match bit for bit;
attention outputs and log-sum-exp within a max-abs error of 2e-3.
Every case compares every query: the small cases, tiny_prefill_4k, the
full-size decode workloads (one query per sequence) and the full-size
prefill workloads (oracle results computed before the GPU is initialised,
tests/oracle_cache.py); list invariants are checked on every query too.
"""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload
from oracle import hisa_oracle as orc
from parity import (ATOL, check_list_invariants, check_queries, check_summaries, oracle_summaries)

pytestmark = pytest.mark.gpu


def small(name, **kw):
    base = dict(batch=1, n_heads_q=1, n_heads_kv=1, n_landmarks=1)
    base.update(kw)
    return Workload(name=name, **base)


# tie-heavy small cases: small integer ranges give many equal scores
SMALL_CASES = [
    (small("ragged_b8", seq_len=300, n_q=300, d_index=64, block=8, top_m=4, top_k=10), 2),
    (small("gqa_lm2", seq_len=1000, n_q=77, d_index=128, block=16, top_m=5, top_k=37,
           n_heads_q=4, n_heads_kv=2, n_landmarks=2), 2),
    (small("lm4_g16", seq_len=2048, n_q=2048, d_index=128, block=32, top_m=6, top_k=100,
           n_heads_q=16, n_heads_kv=1, n_landmarks=4), 3),
    (small("m2_forced_only", batch=3, seq_len=517, n_q=5, d_index=64, block=16, top_m=2, top_k=20,
           n_heads_q=8, n_heads_kv=8), 2),
    (small("k1", batch=2, seq_len=4100, n_q=3, d_index=128, block=128, top_m=3, top_k=1,
           n_heads_q=2, n_heads_kv=1), 8),
    (small("keep_all", seq_len=64, n_q=64, d_index=64, block=8, top_m=100, top_k=1000), 2),
    # k >= m * B: every list is its candidate enumeration (two 1024-slot
    # chunks, k not a multiple of 4)
    (small("enumerate_ragged", batch=2, seq_len=3000, n_q=5, d_index=64, block=16, top_m=70, top_k=1123,
           n_heads_q=4, n_heads_kv=2), 2),
    (small("decode_wide_select", batch=2, seq_len=40000, n_q=2, d_index=64, block=16, top_m=300,
           top_k=1000, n_heads_q=16, n_heads_kv=1), 2),
    (small("prefill_r64_select", seq_len=20000, n_q=512, d_index=128, block=128, top_m=100,
           top_k=300, n_heads_q=2, n_heads_kv=1), 2),
    # a chunk of queries against a long context: block-major token scoring
    (small("chunk_block_major", seq_len=20000, n_q=300, d_index=64, block=16, top_m=40, top_k=200,
           n_heads_q=2, n_heads_kv=1), 2),
    # decode with 2048 scored blocks: the one-launch block top-m at its limit (R = 2)
    (small("decode_fused_r2", batch=3, seq_len=32790, n_q=2, d_index=128, block=16, top_m=40, top_k=300,
           n_heads_q=4, n_heads_kv=1), 2),
    # decode with the token select inside the attention launch: a thread's
    # 32 slots span two blocks (R > B), and two kv heads (each workgroup of
    # a query repeats its select; kv head 0 writes the list)
    (small("decode_select_attn_multiblock", batch=2, seq_len=40000, n_q=1, d_index=64, block=16, top_m=600,
           top_k=1000, n_heads_q=8, n_heads_kv=1), 2),
    (small("decode_select_attn_gqa2", batch=3, seq_len=30000, n_q=1, d_index=64, block=32, top_m=100,
           top_k=512, n_heads_q=8, n_heads_kv=2), 2),
    # decode with the token scores inside the block top-m launch too (8
    # workgroups per query): 1873 and 998 scored blocks (32 and 16 keys per
    # lane of the block select), one and two queries per sequence
    (small("decode_block_token_r32", batch=4, seq_len=30000, n_q=1, d_index=64, block=16, top_m=100,
           top_k=512, n_heads_q=8, n_heads_kv=1), 2),
    (small("decode_block_token_r16_nq2", batch=3, seq_len=16000, n_q=2, d_index=128, block=16, top_m=64,
           top_k=512, n_heads_q=4, n_heads_kv=1), 2),
    # the same launch with fewer workgroups per query: 40 queries (6 per
    # query) and 64 queries (4 per query, the fewest it takes)
    (small("decode_block_token_p6", batch=40, seq_len=6000, n_q=1, d_index=64, block=16, top_m=30,
           top_k=200, n_heads_q=4, n_heads_kv=1), 2),
    (small("decode_block_token_p4", batch=64, seq_len=6000, n_q=1, d_index=128, block=16, top_m=30,
           top_k=200, n_heads_q=4, n_heads_kv=1), 2),
]


def make_small(w, rng_range):
    return datagen.make_inputs(w, q_range=rng_range, centre_range=max(1, rng_range // 2),
                               noise_range=max(1, rng_range // 2))


@pytest.mark.parametrize("w,vr", SMALL_CASES, ids=[c[0].name for c in SMALL_CASES])
def test_small_case_all_queries(w, vr):
    inp = make_small(w, vr)
    dev = pipeline.to_device(inp)
    gpu = pipeline.to_host(pipeline.run_stages(w, dev))
    torch.cuda.synchronize()
    S = oracle_summaries(inp, w)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    check_queries(gpu, inp, w, S, [(b, i) for b in range(w.batch) for i in range(w.n_q)])
    # the fused entry point gives the same bits
    fwd = pipeline.to_host(pipeline.run_forward(w, dev))
    for key in ("S", "blk", "tok", "O", "lse"):
        assert np.array_equal(fwd[key], gpu[key], equal_nan=True), key


def test_dense_when_everything_is_kept():
    # m covers every block and k every token: dense causal attention (torch, fp64, CPU)
    w = small("dense", seq_len=96, n_q=96, d_index=64, block=8, top_m=12, top_k=96, n_heads_q=4, n_heads_kv=1)
    inp = datagen.make_inputs(w)
    gpu = pipeline.to_host(pipeline.run_forward(w, pipeline.to_device(inp)))
    q = torch.tensor(orc.bf16_to_f64(inp["Q"][0])).permute(1, 0, 2)[None]
    k = torch.tensor(orc.bf16_to_f64(inp["K"][0])).permute(1, 0, 2).repeat_interleave(4, 0)[None]
    v = torch.tensor(orc.bf16_to_f64(inp["V"][0])).permute(1, 0, 2).repeat_interleave(4, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale)[0]
    err = np.abs(gpu["O"][0] - ref.permute(1, 0, 2).numpy()).max()
    assert err <= 2e-3


def test_empty_calls_write_nothing():
    w = small("empty", batch=0, seq_len=128, n_q=4, d_index=64, block=16, top_m=3, top_k=8)
    dev = pipeline.to_device(datagen.make_inputs(w.with_(batch=1)))
    out = pipeline.alloc_outputs(w.with_(batch=1))
    pipeline.run_forward(w, dev, out)
    torch.cuda.synchronize()
    assert torch.all(out["blk"] == -7) and torch.all(out["tok"] == -7)


def test_incremental_summaries():
    # hsa_forward with summary_start_block > 0 recomputes only the newest
    # blocks: with the earlier summaries already in S the results equal a
    # full forward (the decode / chunked-prefill state update)
    w = small("incremental", batch=2, seq_len=3000, n_q=200, d_index=128, block=32, top_m=6,
              top_k=150, n_heads_q=4, n_heads_kv=1, n_landmarks=2)
    inp = datagen.make_inputs(w, q_range=4, centre_range=2, noise_range=2)
    dev = pipeline.to_device(inp)
    full = pipeline.to_host(pipeline.run_forward(w, dev))
    start = (w.seq_len - w.n_q) // w.block
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], dev["W"], 0, out["S"])
    out["S"][:, start:] = 0  # stale state for the blocks the new queries touch
    inc = pipeline.to_host(pipeline.run_forward(w, dev, out, summary_start_block=start))
    for key in ("S", "blk", "tok", "O", "lse"):
        assert np.array_equal(inc[key], full[key], equal_nan=True), key


DECODE_FOLD_CASES = [
    # (seq_len, n_q, block, d_index, n_landmarks): the first three put every
    # query in the last block, so the newest block's summary is folded into
    # the block-score launch; the last spans two blocks (separate launch)
    (5000, 1, 32, 64, 1),
    (5000, 5, 32, 128, 4),
    (5024, 1, 32, 128, 2),
    (5000, 40, 32, 64, 2),
]


# batches whose block top-m launch has fewer workgroups per query (6 and 4)
# and the summary-fold workgroups past the first round of the chip
DECODE_FOLD_CASES_WIDE = [(5000, 1, 32, 64, 1, 40), (5000, 1, 32, 128, 1, 64)]


@pytest.mark.parametrize("L,nq,B,dI,nL,batch", [c + (3,) for c in DECODE_FOLD_CASES] + DECODE_FOLD_CASES_WIDE)
def test_incremental_decode_summaries(L, nq, B, dI, nL, batch):
    # decode-shaped calls with only the newest blocks re-summarised: the same
    # bits as a full forward, and every query equal to the oracle
    w = small("decode_inc", batch=batch, seq_len=L, n_q=nq, d_index=dI, block=B, top_m=6, top_k=150,
              n_heads_q=8, n_heads_kv=2, n_landmarks=nL)
    inp = datagen.make_inputs(w, q_range=3, centre_range=2, noise_range=2)
    dev = pipeline.to_device(inp)
    full = pipeline.to_host(pipeline.run_forward(w, dev))
    start = (L - nq) // B
    out = pipeline.alloc_outputs(w)
    _lib.hsa_block_summary(_lib.shape_of(w), dev["kI"], dev.get("W"), 0, out["S"])
    out["S"][:, start:] = 0
    inc = pipeline.to_host(pipeline.run_forward(w, dev, out, summary_start_block=start))
    for key in ("S", "blk", "tok", "O", "lse"):
        assert np.array_equal(inc[key], full[key], equal_nan=True), key
    S = oracle_summaries(inp, w)
    check_summaries(inc["S"], S)
    check_list_invariants(inc, w)
    check_queries(inc, inp, w, S, [(b, i) for b in range(w.batch) for i in range(nq)])


def test_attention_lists_with_holes():
    # hsa_sparse_attn skips -1 entries and entries >= seq_len anywhere in a
    # list (the lists the indexer writes only pad at the end)
    rng = np.random.default_rng(11)
    b, L, nq, Hq, Hkv, k = 2, 700, 9, 8, 2, 512  # 16 tiles: the split + merge path
    w = small("holes", batch=b, seq_len=L, n_q=nq, d_index=64, block=16, top_m=4, top_k=k,
              n_heads_q=Hq, n_heads_kv=Hkv)
    inp = datagen.make_inputs(w)
    tok = np.full((b, nq, k), -1, np.int32)
    for bb in range(b):
        for i in range(nq):
            n = int(rng.integers(1, k + 1))
            sel = np.sort(rng.choice(L, size=n, replace=False)).astype(np.int32)
            pos = np.sort(rng.choice(k, size=n, replace=False))
            tok[bb, i, pos] = sel
            junk = rng.random(k) < 0.05
            tok[bb, i, junk & (tok[bb, i] < 0)] = L + 5  # out of range: skipped
    dev = pipeline.to_device(inp)
    shape = _lib.shape_of(w)
    O = torch.empty((b, nq, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((b, nq, Hq), dtype=torch.float32, device="cuda")
    _lib.hsa_sparse_attn(shape, dev["Q"], dev["K"], dev["V"], torch.from_numpy(tok).cuda(), O, lse)
    O, lse = O.cpu().numpy(), lse.cpu().numpy()
    for bb in range(b):
        for i in range(nq):
            valid = tok[bb, i][(tok[bb, i] >= 0) & (tok[bb, i] < L)]
            ro, rl = orc.sparse_attention(inp["Q"][bb, i], inp["K"][bb], inp["V"][bb], valid, w.scale)
            assert np.abs(O[bb, i] - ro).max() <= 2e-3
            assert np.abs(lse[bb, i] - rl).max() <= 2e-3


def test_repeat_runs_are_bitwise_identical():
    w = WORKLOADS["tiny_prefill_4k"]
    dev = pipeline.to_device(datagen.make_inputs(w))
    a = pipeline.to_host(pipeline.run_forward(w, dev))
    b = pipeline.to_host(pipeline.run_forward(w, dev))
    for key in a:
        assert np.array_equal(a[key], b[key]), key


_cache = {}


def workload_inputs(name):
    if name not in _cache:
        _cache.clear()
        w = WORKLOADS[name]
        inp = datagen.make_inputs(w)
        _cache[name] = (w, inp)
    return _cache[name]


def test_tiny_prefill_4k_all_queries():
    w, inp = workload_inputs("tiny_prefill_4k")
    gpu = pipeline.to_host(pipeline.run_forward(w, pipeline.to_device(inp)))
    S = oracle_summaries(inp, w)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    check_queries(gpu, inp, w, S, [(0, i) for i in range(w.n_q)])


def run_bench_configuration(w, inp):
    """The launch configuration bench.py times: summaries of the context built
    first (state), then the step re-summarises from the first block the
    queries touch (in decode, folded into the block-selection launch)."""
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    _lib.hsa_block_summary(_lib.shape_of(w), dev["kI"], dev.get("W"), 0, out["S"])
    start = (w.seq_len - w.n_q) // w.block
    out["S"][:, start:] = 0  # stale: the step must rebuild these
    gpu = pipeline.to_host(pipeline.run_forward(w, dev, out, summary_start_block=start))
    del dev, out
    torch.cuda.empty_cache()
    return gpu


@pytest.mark.parametrize("name", ["decode_128k", "decode_512k", "landmark_decode_1m"])
def test_full_size_decode_workload(name):
    # every query (one per sequence) against the oracle
    w, inp = workload_inputs(name)
    gpu = run_bench_configuration(w, inp)
    S = oracle_summaries(inp, w)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    check_queries(gpu, inp, w, S, [(b, 0) for b in range(w.batch)])
    if w.needles:
        for b in range(w.batch):
            assert set(inp["needles"][b].tolist()) <= set(gpu["blk"][b, 0].tolist())


def _first_difference(a, b):
    bad = np.argwhere(np.any(a.reshape(a.shape[0], -1) != b.reshape(b.shape[0], -1), axis=1))
    return int(bad[0, 0]) if bad.size else None


@pytest.mark.parametrize("name", [pytest.param(n, marks=pytest.mark.oracle_all(n))
                                  for n in ("chunked_prefill_512k", "prefill_64k")])
def test_full_size_prefill_every_query(name):
    # every query of the full-size prefill workloads against the oracle
    # (computed before the GPU was initialised, tests/oracle_cache.py):
    # block and token lists bit for bit, O and lse within 2e-3
    import oracle_cache
    w, inp, S, ref = oracle_cache.get(name)
    gpu = run_bench_configuration(w, inp)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    for key in ("blk", "tok"):
        i = _first_difference(gpu[key][0], ref[key])
        assert i is None, f"{name}: {key} list of query {i} (t={w.query_pos(i)}) differs from the oracle's"
    for key in ("O", "lse"):
        err = np.abs(gpu[key][0].astype(np.float64) - ref[key])
        worst = float(err.max())
        i = int(np.argmax(err.reshape(w.n_q, -1).max(axis=1)))
        assert worst <= ATOL, f"{name}: {key} max-abs error {worst:.3g} > {ATOL} at query {i}"
        print(f"{name}: {w.n_q} queries, {key} max-abs error {worst:.2e}")


@pytest.mark.parametrize("name,L,nq,dI,B,m,k", [
    # the block select at its capacity: 32770 blocks, 32768 scored per query
    ("max_block_select", 8 * 32770, 2, 64, 8, 64, 512),
    # the token select at its capacity: 256 kept blocks of 128 (32768
    # candidates), 8192 kept (the longest staged list)
    ("max_token_select", 65536, 2, 128, 128, 256, 8192),
])
def test_maximum_select_sizes(name, L, nq, dI, B, m, k):
    w = small(name, batch=2, seq_len=L, n_q=nq, d_index=dI, block=B, top_m=m, top_k=k, n_heads_q=2,
              n_heads_kv=1)
    inp = make_small(w, 3)
    dev = pipeline.to_device(inp)
    gpu = pipeline.to_host(pipeline.run_forward(w, dev))
    S = oracle_summaries(inp, w)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    check_queries(gpu, inp, w, S, [(b, i) for b in range(w.batch) for i in range(nq)])


@pytest.mark.parametrize("name,L,m,k", [
    # 375 splits of 2 tiles: more than 256, not a multiple of 4, so every
    # split's partial goes to the merge
    ("splits_375_unmerged", 40000, 200, 24000),
    # 512 splits (the most a 32768-entry list gets), pre-merged 4 to a
    # workgroup: 128 partials per row reach the merge
    ("splits_512_premerged", 50000, 256, 32768),
])
def test_one_query_with_a_long_list(name, L, m, k):
    # one query and one kv head: the split plan's cap, not the wave target,
    # sets the split count
    w = small(name, batch=1, seq_len=L, n_q=1, d_index=128, block=128, top_m=m, top_k=k, n_heads_q=16,
              n_heads_kv=1)
    inp = make_small(w, 3)
    gpu = pipeline.to_host(pipeline.run_forward(w, pipeline.to_device(inp)))
    S = oracle_summaries(inp, w)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    check_queries(gpu, inp, w, S, [(0, 0)])


@pytest.mark.parametrize("name,batch,L,nq,dI,B,m,k,Hq,Hkv", [
    # 2 kv heads: chunks of 1024 queries (2048 rows), 9 of them, none split
    ("chunked_attention_two_seqs", 2, 12000, 9216, 64, 64, 16, 256, 4, 2),
    # the same with a last chunk of 208 queries (416 rows: split and merged)
    ("chunked_attention_ragged_tail", 1, 12000, 9424, 64, 64, 16, 256, 4, 2),
    # one kv head: chunks of 2048 queries, the last of one query
    ("chunked_attention_one_query_tail", 1, 9000, 8193, 128, 32, 12, 300, 16, 1),
])
def test_prefill_chunked_attention(name, batch, L, nq, dI, B, m, k, Hq, Hkv):
    # long prefills run the attention in launches of ceil(2048 / Hkv)
    # queries: the outputs are the unchunked entry points' (bit for bit
    # where no chunk is split), and every query at a chunk edge (plus a
    # sample) matches the oracle
    w = small(name, batch=batch, seq_len=L, n_q=nq, d_index=dI, block=B, top_m=m, top_k=k, n_heads_q=Hq,
              n_heads_kv=Hkv)
    inp = make_small(w, 4)
    dev = pipeline.to_device(inp)
    ref = pipeline.to_host(pipeline.run_stages(w, dev))
    got = pipeline.to_host(pipeline.run_forward(w, dev))
    cq = -(-2048 // Hkv)  # queries per chunk
    split_tail = nq % cq != 0 and (nq % cq) * Hkv < 2048
    for key in ("S", "blk", "tok") + (() if split_tail else ("O", "lse")):
        assert np.array_equal(got[key], ref[key]), key
    assert np.abs(got["O"] - ref["O"]).max() <= ATOL and np.abs(got["lse"] - ref["lse"]).max() <= ATOL
    del dev
    torch.cuda.empty_cache()
    S = oracle_summaries(inp, w)
    edges = {e for c in range(1, nq // cq + 1) for e in (c * cq - 1, c * cq)} | {0, nq - 1}
    edges &= set(range(nq))
    rng = np.random.default_rng(2)
    qs = sorted(edges | set(int(x) for x in rng.integers(0, nq, 10)))
    check_queries(got, inp, w, S, [(b, i) for b in range(batch) for i in qs])
