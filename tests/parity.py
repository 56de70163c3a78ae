"""Helpers shared by the GPU parity tests: run the oracle on chosen queries
and compare with the GPU results (index sets bit-exact, attention within
a max-abs error of 2e-3, the bound set for bf16 inputs with fp32
accumulation)."""
from __future__ import annotations

import numpy as np

from oracle import hisa_oracle as orc

ATOL = 2e-3


def oracle_summaries(inp: dict, w) -> np.ndarray:
    return np.stack([orc.block_summary(inp["kI"][b], w.block, inp.get("W")) for b in range(w.batch)])


def check_summaries(gpu_S: np.ndarray, ora_S: np.ndarray, start_block: int = 0):
    assert gpu_S.shape == ora_S.shape
    bad = np.argwhere(gpu_S[:, start_block:] != ora_S[:, start_block:])
    assert bad.size == 0, f"{len(bad)} summary values differ, first at {bad[0]}"


def check_queries(gpu: dict, inp: dict, w, ora_S: np.ndarray, queries, attention: bool = True,
                  stats: dict | None = None):
    """Compare GPU outputs with the oracle for (b, i) pairs."""
    worst = 0.0
    for b, i in queries:
        t = w.query_pos(i)
        r = orc.forward_query(inp, b, i, t, w.block, w.top_m, w.top_k, w.scale, S_bits=ora_S[b],
                              attention=attention)
        ctx = f"{w.name} b={b} i={i} t={t}"
        assert np.array_equal(gpu["blk"][b, i], r["blk"]), f"block list differs: {ctx}"
        assert np.array_equal(gpu["tok"][b, i], r["tok"]), f"token list differs: {ctx}"
        if attention:
            err = np.abs(gpu["O"][b, i].astype(np.float64) - r["O"]).max()
            lerr = np.abs(gpu["lse"][b, i].astype(np.float64) - r["lse"]).max()
            assert err <= ATOL, f"O max-abs error {err:.3g} > {ATOL}: {ctx}"
            assert lerr <= ATOL, f"lse error {lerr:.3g} > {ATOL}: {ctx}"
            worst = max(worst, err)
    if stats is not None:
        stats["max_abs_err"] = max(stats.get("max_abs_err", 0.0), worst)
    return worst


def check_list_invariants(gpu: dict, w, chunk: int = 256):
    """Properties of every query's lists that hold at any size."""
    B, m, k = w.block, w.top_m, w.top_k
    for i0 in range(0, w.n_q, chunk):
        blk = gpu["blk"][:, i0:i0 + chunk]
        tok = gpu["tok"][:, i0:i0 + chunk]
        t = w.seq_len - w.n_q + np.arange(i0, i0 + blk.shape[1])
        c = t // B
        n_sel = np.minimum(c + 1, m)
        # block lists: ascending, -1 padded, 0 and c present
        valid = blk >= 0
        assert np.array_equal(valid.sum(-1), np.broadcast_to(n_sel, valid.shape[:2]))
        assert np.all(blk[..., 0] == 0)
        last = np.take_along_axis(blk, np.broadcast_to((n_sel - 1)[None, :, None], blk.shape[:2] + (1,)), -1)[..., 0]
        assert np.array_equal(last, np.broadcast_to(c, last.shape))
        d = np.diff(np.where(valid, blk, np.iinfo(np.int32).max), axis=-1)
        assert np.all(d[valid[..., 1:]] > 0)
        assert np.all(blk[~valid] == -1)
        # token lists: ascending, -1 padded, causal, inside kept blocks
        n_valid = (n_sel - 1) * B + (t - c * B + 1)
        tv = tok >= 0
        assert np.array_equal(tv.sum(-1), np.broadcast_to(np.minimum(n_valid, k), tv.shape[:2]))
        assert np.all(tok[~tv] == -1)
        assert np.all(tok <= t[None, :, None])
        dt = np.diff(np.where(tv, tok, np.iinfo(np.int32).max), axis=-1)
        assert np.all(dt[tv[..., 1:]] > 0)
        # every kept token's block is a kept block: sorted search in the block list
        for b in range(blk.shape[0]):
            for r in range(blk.shape[1]):
                bl = blk[b, r][valid[b, r]]
                tb = tok[b, r][tv[b, r]] // B
                pos = np.searchsorted(bl, tb)
                assert np.all(pos < bl.size) and np.array_equal(bl[np.minimum(pos, bl.size - 1)], tb)
