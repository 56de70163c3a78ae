"""GPU parity of hsa_decode_step: decode over a batch of different lengths.

Each sequence b has its own current length L_b inside a cache of capacity
seq_len; its query sits at t = L_b - 1 and the summary of its partial last
block is rebuilt from the rows < L_b.  Every sequence is compared with the
oracle run on that sequence alone (summaries of its first L_b rows, query at
L_b - 1): summaries and index lists bit for bit, O and lse within 2e-3.  A
multi-step loop appends one token per sequence per step, carrying the
summary state S between steps, across block boundaries.
"""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import Workload
from oracle import hisa_oracle as orc
from parity import ATOL

pytestmark = pytest.mark.gpu


def varlen_case(batch, cap, dI, B, m, k, nL, Hq=8, Hkv=2, vr=3):
    w = Workload(name="varlen", batch=batch, seq_len=cap, n_q=1, d_index=dI, block=B, top_m=m, top_k=k,
                 n_heads_q=Hq, n_heads_kv=Hkv, n_landmarks=nL)
    # queries of the workload sit at position cap - 1; each step uses the
    # query arrays as the new token of every sequence, whatever its length
    inp = datagen.make_inputs(w, q_range=vr, centre_range=max(1, vr // 2), noise_range=max(1, vr // 2))
    return w, inp


def run_step(w, dev, out, lens):
    shape = _lib.shape_of(w)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    _lib.hsa_decode_step(shape, lens_t, dev["qI"], dev["kI"], dev.get("W"), out["S"], dev["Q"], dev["K"], dev["V"],
                         out["blk"], out["tok"], out["O"], out["lse"])
    torch.cuda.synchronize()
    return pipeline.to_host(out)


def check_step(w, inp, gpu, lens):
    for b, Lb in enumerate(lens):
        t = Lb - 1
        S_b = orc.block_summary(inp["kI"][b, :Lb], w.block, inp.get("W"))
        nb_b = S_b.shape[0]
        assert np.array_equal(gpu["S"][b, :nb_b], S_b), f"summaries differ: b={b} L_b={Lb}"
        r = orc.forward_query(inp, b, 0, t, w.block, w.top_m, w.top_k, w.scale, S_bits=S_b)
        ctx = f"b={b} L_b={Lb}"
        assert np.array_equal(gpu["blk"][b, 0], r["blk"]), f"block list differs: {ctx}"
        assert np.array_equal(gpu["tok"][b, 0], r["tok"]), f"token list differs: {ctx}"
        assert np.abs(gpu["O"][b, 0].astype(np.float64) - r["O"]).max() <= ATOL, ctx
        assert np.abs(gpu["lse"][b, 0].astype(np.float64) - r["lse"]).max() <= ATOL, ctx


CASES = [
    # batch, capacity, d_I, B, m, k, n_L: the first two take the one-launch
    # block top-m (<= 2048 scored blocks, one summary per block), the next
    # two the GEMV + select pair (landmarks, or more blocks)
    (6, 5000, 64, 32, 6, 150, 1),
    (5, 4100, 128, 128, 3, 40, 1),
    (5, 3000, 128, 16, 8, 100, 4),
    (4, 40000, 64, 16, 20, 300, 1),
    # a capacity with no scoring at all: the summary update runs on its own
    (3, 100, 64, 16, 8, 40, 1),
    # the block top-m with the token scores in one launch, then the select
    # inside the attention launch (lengths with c + 1 < m, = m and > m,
    # keeping all candidates or scoring them)
    (8, 20000, 128, 16, 64, 512, 1),
    (6, 12000, 64, 16, 40, 256, 1),
]


def lens_for(cap, B, m, batch):
    # full, ragged, block boundary, just past one, the c + 1 == m edge, one token
    picks = [cap, cap - 37, 7 * B, 7 * B + 1, m * B, 1, cap // 2 + 3, B]
    return [int(min(cap, max(1, x))) for x in picks[:batch]]


@pytest.mark.parametrize("batch,cap,dI,B,m,k,nL", CASES)
def test_decode_step_per_sequence(batch, cap, dI, B, m, k, nL):
    w, inp = varlen_case(batch, cap, dI, B, m, k, nL)
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    # state: summaries of the whole capacity (blocks before each sequence's
    # last block are complete; the last one is rebuilt by the step)
    _lib.hsa_block_summary(_lib.shape_of(w), dev["kI"], dev.get("W"), 0, out["S"])
    lens = lens_for(cap, B, m, batch)
    check_step(w, inp, run_step(w, dev, out, lens), lens)


def test_decode_loop_across_block_boundaries():
    # four steps, one token appended to every sequence per step; S carried
    w, inp = varlen_case(4, 3000, 64, 16, 6, 80, 1)
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    lens = [2998 - 2, 16 * 40 - 2, 16 * 6 - 1, 5]  # crosses a block boundary on the way
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, out["S"])
    for step in range(4):
        cur = [L + step for L in lens]
        check_step(w, inp, run_step(w, dev, out, cur), cur)


def test_decode_step_equals_forward_at_full_length():
    # every sequence at full length: the bits of hsa_forward's decode call
    w, inp = varlen_case(3, 9000, 128, 64, 10, 300, 1)
    dev = pipeline.to_device(inp)
    a = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, a["S"])
    ref = pipeline.to_host(pipeline.run_forward(w, dev, a, summary_start_block=(w.seq_len - 1) // w.block))
    c = pipeline.alloc_outputs(w)
    _lib.hsa_block_summary(shape, dev["kI"], None, 0, c["S"])
    got = run_step(w, dev, c, [w.seq_len] * w.batch)
    for key in ("S", "blk", "tok", "O", "lse"):
        assert np.array_equal(got[key], ref[key], equal_nan=True), key


def test_decode_varlen_128k_sampled():
    # the bench configuration: batch 32, capacity 131072, seeded lengths in
    # [65536, 131072]; every list checked for invariants, 6 sequences against
    # the oracle
    from hierarchical_index_sparse_amd.workloads import WORKLOADS
    w = WORKLOADS["decode_varlen_128k"]
    inp = datagen.make_inputs(w)
    lens = [int(x) for x in inp["seq_lens"]]
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    _lib.hsa_block_summary(_lib.shape_of(w), dev["kI"], None, 0, out["S"])
    gpu = run_step(w, dev, out, lens)
    for b, Lb in enumerate(lens):
        c = (Lb - 1) // w.block
        blk = gpu["blk"][b, 0]
        assert blk[0] == 0 and blk[-1] == c and np.all(np.diff(blk) > 0), b
        tok = gpu["tok"][b, 0]
        assert np.all(np.diff(tok) > 0) and tok[-1] <= Lb - 1 and set(tok // w.block) <= set(blk.tolist()), b
    picks = sorted({0, w.batch - 1, int(np.argmin(lens)), int(np.argmax(lens)), 7, 19})
    sub = {"S": gpu["S"][picks], "blk": gpu["blk"][picks], "tok": gpu["tok"][picks], "O": gpu["O"][picks],
           "lse": gpu["lse"][picks]}
    sub_inp = {k: (v[picks] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
    check_step(w.with_(batch=len(picks)), sub_inp, sub, [lens[b] for b in picks])
