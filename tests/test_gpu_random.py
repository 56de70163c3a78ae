"""GPU parity on a seeded sweep of randomly drawn small configurations.

Each case draws batch, context length, query count, d_index, block size,
landmarks, m, k, head counts and the integer value range (small ranges give
many tied scores) from a fixed seed, runs hsa_forward once and compares
with the oracle: every block summary bit for bit, the list invariants on
every query, and the block list, token list, O and lse of a sample of up to
40 queries per case.  The ranges are chosen so that the draws reach every
launch path (tiled, block-major and per-query token scoring; one-wave,
four-wave and sixteen-wave selects; the one-launch decode block top-m;
enumerated lists when k >= m * B; GQA packing; landmark summaries).
"""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import datagen, pipeline
from hierarchical_index_sparse_amd.workloads import Workload
from parity import check_list_invariants, check_queries, check_summaries, oracle_summaries

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw(idx: int):
    rng = np.random.default_rng(1000 + idx)
    B = int(rng.choice([8, 16, 32, 64, 128]))
    L = int(rng.integers(1, 6001))
    # few queries (decode-like) or many (prefill-like)
    nq = int(rng.integers(1, 4)) if rng.random() < 0.4 else int(rng.integers(1, min(L, 700) + 1))
    nq = min(nq, L)
    batch = int(rng.integers(1, 4)) if nq * L < 2_000_000 else 1
    dI = int(rng.choice([64, 128]))
    nL = int(rng.choice([1, 1, 2, 4]))
    m = int(rng.integers(2, 41))
    # keep every list (k >= m * B) in about one case in six
    k = m * B + int(rng.integers(0, 50)) if rng.random() < 0.17 else int(rng.integers(1, min(m * B, 800) + 1))
    if k < m * B and m * B > 32768:
        m = max(2, 32768 // B)
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8, 16]))
    vr = int(rng.choice([1, 2, 3, 8]))
    w = Workload(name=f"rand{idx}", batch=batch, seq_len=L, n_q=nq, d_index=dI, block=B, top_m=m, top_k=k,
                 n_heads_q=Hq, n_heads_kv=Hkv, n_landmarks=nL)
    return w, vr


CASES = [draw(i) for i in range(N_CASES)]


def describe(c):
    w, vr = c
    return (f"{w.name}-b{w.batch}-L{w.seq_len}-q{w.n_q}-d{w.d_index}-B{w.block}-nL{w.n_landmarks}-m{w.top_m}"
            f"-k{w.top_k}-h{w.n_heads_q}x{w.n_heads_kv}-v{vr}")


@pytest.mark.parametrize("w,vr", CASES, ids=[describe(c) for c in CASES])
def test_random_configuration(w, vr):
    print(describe((w, vr)), flush=True)
    inp = datagen.make_inputs(w, q_range=vr, centre_range=max(1, vr // 2), noise_range=max(1, vr // 2))
    gpu = pipeline.to_host(pipeline.run_forward(w, pipeline.to_device(inp)))
    torch.cuda.synchronize()
    S = oracle_summaries(inp, w)
    check_summaries(gpu["S"], S)
    check_list_invariants(gpu, w)
    rng = np.random.default_rng(7)
    pairs = [(b, i) for b in range(w.batch) for i in range(w.n_q)]
    if len(pairs) > 40:
        # the last query of every sequence and a seeded sample of the rest
        last = [(b, w.n_q - 1) for b in range(w.batch)]
        rest = [pairs[j] for j in rng.choice(len(pairs), 40 - len(last), replace=False)]
        pairs = sorted(set(last + rest))
    check_queries(gpu, inp, w, S, pairs)


# ---------------------------------------------------------------- 3-level

def draw3(idx: int):
    rng = np.random.default_rng(5000 + idx)
    B = int(rng.choice([8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    L = int(rng.integers(1, 40001))
    nq = int(rng.integers(1, 4)) if rng.random() < 0.6 else int(rng.integers(1, min(L, 600) + 1))
    batch = int(rng.integers(1, 3))
    dI = int(rng.choice([64, 128]))
    nL = int(rng.choice([1, 1, 1, 2, 4]))
    m2 = int(rng.integers(2, min(8192 // G, 64) + 1))
    m = int(rng.integers(2, 50))
    k = int(rng.integers(1, min(m * B, 600) + 1))
    if m * B > 32768:
        m = 32768 // B
    vr = int(rng.choice([1, 2, 3]))
    w = Workload(name=f"r3_{idx}", batch=batch, seq_len=L, n_q=min(nq, L), d_index=dI, block=B, top_m=m,
                 top_k=k, n_heads_q=4, n_heads_kv=1, n_landmarks=nL, group=G, top_m2=m2)
    return w, vr


CASES3 = [draw3(i) for i in range(30)]


@pytest.mark.parametrize("w,vr", CASES3, ids=[f"{c[0].name}-L{c[0].seq_len}-q{c[0].n_q}-B{c[0].block}-G{c[0].group}"
                                              f"-m2{c[0].top_m2}-m{c[0].top_m}-nL{c[0].n_landmarks}" for c in CASES3])
def test_random_three_level(w, vr):
    from oracle import hisa_oracle as orc
    from parity import ATOL
    inp = datagen.make_inputs(w, q_range=vr, centre_range=max(1, vr // 2), noise_range=max(1, vr // 2))
    g = pipeline.to_host(pipeline.run_forward_3level(w, pipeline.to_device(inp)))
    torch.cuda.synchronize()
    S = oracle_summaries(inp, w)
    check_summaries(g["S"], S)
    S2 = np.stack([orc.super_summary(S[b], w.group) for b in range(w.batch)])
    assert np.array_equal(g["S2"], S2), "super-block summaries differ"
    rng = np.random.default_rng(3)
    pairs = [(b, i) for b in range(w.batch) for i in range(w.n_q)]
    if len(pairs) > 30:
        pairs = sorted(set([pairs[j] for j in rng.choice(len(pairs), 28, replace=False)] +
                           [(b, w.n_q - 1) for b in range(w.batch)]))
    for b, i in pairs:
        t = w.query_pos(i)
        ctx = f"{w.name} b={b} i={i} t={t}"
        sup = orc.select_blocks(inp["qI"][b, i], S2[b], t, w.block * w.group, w.top_m2)
        assert np.array_equal(g["sup"][b, i], sup), f"super-block list differs: {ctx}"
        r = orc.forward_query_3level(inp, b, i, t, w.block, w.group, w.top_m2, w.top_m, w.top_k, w.scale, S[b],
                                     S2[b])
        assert np.array_equal(g["blk"][b, i], r["blk"]), f"block list differs: {ctx}"
        assert np.array_equal(g["tok"][b, i], r["tok"]), f"token list differs: {ctx}"
        assert np.abs(g["O"][b, i].astype(np.float64) - r["O"]).max() <= ATOL, ctx
        assert np.abs(g["lse"][b, i].astype(np.float64) - r["lse"]).max() <= ATOL, ctx


# ---------------------------------------------------------------- per head

def drawh(idx: int):
    rng = np.random.default_rng(9000 + idx)
    B = int(rng.choice([8, 16, 32, 64, 128]))
    L = int(rng.integers(1, 20001))
    nq = int(rng.integers(1, 4)) if rng.random() < 0.6 else int(rng.integers(1, min(L, 300) + 1))
    batch = int(rng.integers(1, 3))
    nL = int(rng.choice([1, 2, 4]))
    m = int(rng.integers(2, 40))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8, 16]))
    w = Workload(name=f"rh_{idx}", batch=batch, seq_len=L, n_q=min(nq, L), d_index=128, block=B, top_m=m,
                 top_k=m * B, n_heads_q=Hq, n_heads_kv=Hkv, n_landmarks=nL, per_head=True)
    return w


CASESH = [drawh(i) for i in range(30)]


@pytest.mark.parametrize("w", CASESH, ids=[f"{w.name}-b{w.batch}-L{w.seq_len}-q{w.n_q}-B{w.block}-nL{w.n_landmarks}"
                                           f"-m{w.top_m}-h{w.n_heads_q}x{w.n_heads_kv}" for w in CASESH])
def test_random_per_head(w):
    from oracle import hisa_oracle as orc
    from test_gpu_heads import check_heads
    inp = datagen.make_inputs(w)
    g = pipeline.to_host(pipeline.run_forward_heads(w, pipeline.to_device(inp)))
    torch.cuda.synchronize()
    LK = np.stack([orc.head_landmarks(inp["K"][b], w.block, inp.get("W")) for b in range(w.batch)])
    assert np.array_equal(g["LK"], LK), "landmarks differ"
    rng = np.random.default_rng(4)
    pairs = [(b, i) for b in range(w.batch) for i in range(w.n_q)]
    if len(pairs) > 12:
        pairs = sorted(set([pairs[j] for j in rng.choice(len(pairs), 10, replace=False)] +
                           [(b, w.n_q - 1) for b in range(w.batch)]))
    stats = {"lists": 0, "equal": 0}
    check_heads(w, inp, g, LK, pairs, pairs[:4], stats)
