"""GPU parity of the flat indexer (hsa_flat_topk) against the CPU oracle.

The flat indexer scores every causal token and keeps the top-k; the oracle's
flat_topk is pinned in test_oracle_pins.py (rank counting).  Token lists
must match bit for bit.  The cases cover a single 8192-token chunk, one to
three merge levels with both merge widths, ties across chunk boundaries, the
keep-all path, and the reduction of the hierarchical selection to the flat one when
every block is kept (HISA page, short inputs), all on the GPU.
"""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload
from oracle import hisa_oracle as orc

pytestmark = pytest.mark.gpu


def indexer_case(name, batch, L, nq, dI, k, vr=8, seed=0):
    w = Workload(name=name, batch=batch, seq_len=L, n_q=nq, d_index=dI, block=128, top_m=2, top_k=k,
                 n_heads_q=1, n_heads_kv=1, n_landmarks=1, seed=seed)
    inp = datagen.make_inputs(w, attention=False, q_range=vr, centre_range=max(1, vr // 2),
                              noise_range=max(1, vr // 2))
    return w, inp


def run_flat(w, inp):
    shape = _lib.shape_of(w)
    dev = pipeline.to_device({"qI": inp["qI"], "kI": inp["kI"]})
    tok = torch.full((w.batch, w.n_q, w.top_k), -7, dtype=torch.int32, device="cuda")
    _lib.hsa_flat_topk(shape, dev["qI"], dev["kI"], tok)
    torch.cuda.synchronize()
    return tok.cpu().numpy()


def check(w, inp, tok, queries):
    for b, i in queries:
        t = w.seq_len - w.n_q + i
        ref = orc.flat_topk(inp["qI"][b, i], inp["kI"][b], t, w.top_k)
        assert np.array_equal(tok[b, i], ref), (w.name, b, i, t)


CASES = [
    # name, batch, L, n_q, d_I, k, value range (small ranges: many ties)
    ("single_chunk", 2, 3000, 300, 64, 100, 2),
    ("keep_all_prefix", 1, 700, 700, 128, 256, 8),
    ("one_merge", 1, 70000, 5, 128, 1000, 2),
    ("one_merge_d64", 2, 40000, 3, 64, 16, 1),
    ("three_levels_wide", 1, 5 * 32768 + 11, 2, 64, 8192, 2),  # 21 chunks, 16-wave merges of 4
    ("two_levels", 2, 70000, 3, 128, 2048, 1),                 # 9 chunks, 4-wave merges of 4
    ("wide_merge", 1, 70000, 2, 64, 4096, 2),                  # 9 chunks, 16-wave merges of 8
    # contexts up to 65536: one whole-row select per query, launched in
    # groups of row length (1024 R keys, R = 1 .. 64); heavy ties
    ("row_select_every_group", 1, 65536, 65536, 64, 300, 1),
    ("row_select_batch", 2, 9000, 4500, 128, 2048, 2),
]


@pytest.mark.parametrize("name,batch,L,nq,dI,k,vr", CASES, ids=[c[0] for c in CASES])
def test_flat_topk_matches_oracle(name, batch, L, nq, dI, k, vr):
    w, inp = indexer_case(name, batch, L, nq, dI, k, vr)
    tok = run_flat(w, inp)
    qs = [(b, i) for b in range(batch) for i in range(nq)]
    if len(qs) > 120:  # every query near the keep-all edge and a spread of the rest
        rng = np.random.default_rng(5)
        # the keep-all edge and the row-length group edges (t + 1 = 512 R, 1024 R)
        edges = {k} | {512 * r for r in (2, 4, 8, 16, 32, 64, 128)}
        edge = [(b, i) for (b, i) in qs if min(abs((L - nq + i + 1) - e) for e in edges) <= 2]
        qs = sorted(set(edge + [qs[j] for j in rng.choice(len(qs), 100, replace=False)] + qs[-4:]))
    check(w, inp, tok, qs)


def test_hierarchical_reduces_to_flat_on_gpu():
    # with m covering every block the hierarchical token lists are the flat ones
    w = Workload(name="reduce", batch=2, seq_len=2000, n_q=2000, d_index=64, block=16, top_m=125, top_k=50,
                 n_heads_q=1, n_heads_kv=1, n_landmarks=1)
    inp = datagen.make_inputs(w, attention=False, q_range=3, centre_range=2, noise_range=2)
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, out["S"])
    _lib.hsa_block_topm(shape, dev["qI"], out["S"], out["blk"])
    _lib.hsa_token_topk(shape, dev["qI"], dev["kI"], out["blk"], out["tok"])
    flat = torch.full_like(out["tok"], -7)
    _lib.hsa_flat_topk(shape, dev["qI"], dev["kI"], flat)
    torch.cuda.synchronize()
    assert torch.equal(out["tok"], flat)


def test_flat_prefill_64k_sampled():
    # the full prefill_64k indexer shape (what the comparison in bench.py runs)
    w = WORKLOADS["prefill_64k"]
    inp = datagen.make_inputs(w, attention=False)
    tok = run_flat(w, inp)
    rng = np.random.default_rng(9)
    qs = [(0, int(i)) for i in rng.choice(w.n_q, 24, replace=False)]
    qs += [(0, 0), (0, w.top_k - 1), (0, w.top_k), (0, 32767), (0, 32768), (0, w.n_q - 1)]
    check(w, inp, tok, qs)
    # lists are ascending, -1 padded, causal
    valid = tok >= 0
    t = np.arange(w.n_q)[None, :, None]
    assert np.all(tok[valid[..., :]] <= np.broadcast_to(t, tok.shape)[valid])
    d = np.diff(np.where(valid, tok, np.iinfo(np.int32).max), axis=-1)
    assert np.all(d[valid[..., 1:]] > 0)
