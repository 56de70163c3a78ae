"""Oracle results for every query of the full-size prefill workloads.

prefill_64k (65 536 queries) and chunked_prefill_512k (4 096 queries) are
compared with the CPU oracle query by query, all of them.  The oracle is
plain numpy and runs one query at a time, so it is spread over a pool of
forked worker processes that write straight into shared (anonymous,
MAP_SHARED) arrays.  Forking is only safe before the parent process
initialises the GPU runtime, so `precompute` runs from the test session's
collection hook (tests/conftest.py), before any GPU call; `get` then hands
each test the inputs, the oracle summaries and the oracle's blk, tok, O and
lse for every query.
"""
from __future__ import annotations

import mmap
import os
import time

import numpy as np

from hierarchical_index_sparse_amd import datagen
from hierarchical_index_sparse_amd.workloads import WORKLOADS
from oracle import hisa_oracle as orc

ALL_QUERY_WORKLOADS = ("prefill_64k", "chunked_prefill_512k")

_done: dict = {}
_state: dict = {}


def _shared(shape, dtype) -> np.ndarray:
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    return np.frombuffer(mmap.mmap(-1, max(n, 1)), dtype=dtype, count=int(np.prod(shape))).reshape(shape)


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _run_chunk(args):
    i0, i1 = args
    w, inp, S, res = _state["w"], _state["inp"], _state["S"], _state["res"]
    for i in range(i0, i1):
        r = orc.forward_query(inp, 0, i, w.query_pos(i), w.block, w.top_m, w.top_k, w.scale, S_bits=S[0])
        res["blk"][i] = r["blk"]
        res["tok"][i] = r["tok"]
        res["O"][i] = r["O"]
        res["lse"][i] = r["lse"]
    return i1 - i0


def workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def precompute(names=ALL_QUERY_WORKLOADS, log=print) -> None:
    """Run the oracle on every query of each named workload (batch 1).
    Must run before this process initialises the GPU."""
    import multiprocessing as mp
    for name in names:
        if name in _done:
            continue
        w = WORKLOADS[name]
        assert w.batch == 1 and not w.group and not w.per_head and not w.varlen_min
        t0 = time.perf_counter()
        inp = datagen.make_inputs(w)
        S = np.stack([orc.block_summary(inp["kI"][0], w.block, inp.get("W"))])
        nq = w.n_q
        res = {"blk": _shared((nq, w.top_m), np.int32), "tok": _shared((nq, w.top_k), np.int32),
               "O": _shared((nq, w.n_heads_q, w.head_dim), np.float64),
               "lse": _shared((nq, w.n_heads_q), np.float64)}
        _state.update(w=w, inp=inp, S=S, res=res)
        step = 64
        chunks = [(i, min(nq, i + step)) for i in range(0, nq, step)]
        n, last = 0, time.perf_counter()
        with mp.get_context("fork").Pool(workers(), initializer=_worker_init) as pool:
            for done in pool.imap_unordered(_run_chunk, chunks):
                n += done
                if time.perf_counter() - last > 20.0:  # progress for long runs
                    last = time.perf_counter()
                    log(f"[oracle_cache] {name}: {n} of {nq} queries")
        _state.clear()
        assert n == nq
        _done[name] = (w, inp, S, res)
        log(f"[oracle_cache] {name}: oracle on all {nq} queries in {time.perf_counter() - t0:.1f} s "
            f"on {workers()} worker processes")


def get(name):
    """(workload, inputs, oracle summaries [1, nb, nL, dI], oracle results)."""
    if name not in _done:
        raise RuntimeError(f"oracle results for {name} were not precomputed before the GPU was initialised "
                           "(tests/conftest.py runs oracle_cache.precompute when these tests are collected)")
    return _done[name]
