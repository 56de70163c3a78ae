"""GPU parity of hsa_block_score_max, the score-only build of the block-score
contraction (the MFMA tiling of step 2 with each query's maximum formed on
chip): for every query, the highest score over its scored blocks 1..c-1,
or -inf when it scores none, against the oracle's block scores.  Scores are
exact (integer-valued indexer vectors), so the maxima are compared bit for
bit."""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload
from oracle import hisa_oracle as orc

pytestmark = pytest.mark.gpu


def oracle_max(inp, S, w, b, i):
    t = w.query_pos(i)
    c = t // w.block
    if c + 1 <= w.top_m:
        return -np.inf
    return float(orc.block_scores(inp["qI"][b, i], S[b], c)[1:c].max())


def run(w, inp):
    dev = pipeline.to_device(inp)
    shape = _lib.shape_of(w)
    S = torch.zeros((w.batch, w.n_blocks, w.n_landmarks, w.d_index), dtype=torch.bfloat16, device="cuda")
    _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, S)
    out = torch.full((w.batch, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
    _lib.hsa_block_score_max(shape, dev["qI"], S, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), pipeline.to_host({"S": S})["S"]


def case(name, **kw):
    base = dict(batch=1, n_heads_q=1, n_heads_kv=1, n_landmarks=1)
    base.update(kw)
    return Workload(name=name, **base)


CASES = [
    case("prefill_b16", seq_len=3000, n_q=3000, d_index=64, block=16, top_m=5, top_k=50),
    case("prefill_lm4_ragged", batch=2, seq_len=5003, n_q=777, d_index=128, block=32, top_m=6, top_k=100,
         n_landmarks=4),
    case("chunk_many_tiles", seq_len=200000, n_q=130, d_index=128, block=64, top_m=20, top_k=300),
    case("chunk_lm2_d64", seq_len=70000, n_q=70, d_index=64, block=8, top_m=9, top_k=100, n_landmarks=2),
    case("decode_shape", batch=3, seq_len=9000, n_q=1, d_index=128, block=16, top_m=8, top_k=64),
    case("nothing_scored", seq_len=500, n_q=500, d_index=64, block=128, top_m=8, top_k=64),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_block_score_max_small(w):
    inp = datagen.make_inputs(w, attention=False, q_range=3, centre_range=2, noise_range=2)
    got, S = run(w, inp)
    ref_S = np.stack([orc.block_summary(inp["kI"][b], w.block, inp.get("W")) for b in range(w.batch)])
    assert np.array_equal(S, ref_S)
    ref = np.array([[oracle_max(inp, ref_S, w, b, i) for i in range(w.n_q)] for b in range(w.batch)])
    assert np.array_equal(got, ref.astype(np.float32)), np.argwhere(got != ref.astype(np.float32))[:5]


@pytest.mark.parametrize("name", ["prefill_64k", "chunked_prefill_512k"])
def test_block_score_max_full_size(name):
    w = WORKLOADS[name]
    inp = datagen.make_inputs(w, attention=False)
    got, S = run(w, inp)
    ref_S = np.stack([orc.block_summary(inp["kI"][0], w.block, inp.get("W"))])
    assert np.array_equal(S, ref_S)
    ref = np.array([oracle_max(inp, ref_S, w, 0, i) for i in range(w.n_q)], dtype=np.float32)
    bad = np.argwhere(got[0] != ref)
    assert bad.size == 0, f"{bad.size} maxima differ, first at query {bad[0, 0]}"
