#!/usr/bin/env python3
"""Throughput of hierarchical block-then-token sparse attention on one GPU.

One step = one hsa_forward call over the workload's whole batch: block
summaries of the blocks the queries touch, block top-m, token top-k and
sparse attention, with inputs already resident in HBM (hsa_decode_step for
sequences of different lengths, hsa_forward_3level for workloads with
super-blocks, hsa_forward_heads for per-head selection).  Prints one JSON
line.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Kernel times come from start/stop events that each kernel's dispatch
carries (hsa_sparse_set_kernel_events, hipExtLaunchKernelGGL): an untimed
pass times every kernel of a step and names the dominant (longest) one; in
the timed region that kernel's dispatches carry events on every 8th step
(an event-carrying dispatch costs the stream a few microseconds).  The
roofline entry divides that kernel's algorithmic bytes (or flops) per
launch, computed in closed form below, by its average duration over those
steps.  Stage times (an untimed pass with the stage events of
hsa_sparse_set_stage_events, a few microseconds of stream time each) are
reported alongside.
The CPU baseline times the plain CPU oracle on a stratified sample of the
same workload's queries, before the GPU is touched.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from hierarchical_index_sparse_amd import datagen  # noqa: E402
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
STAGES = ("block_summary", "block_topm", "token_topk", "sparse_attn")


# --------------------------------------------------------------- work model


def level1_counts(w: Workload, t):
    """Three-level selection: super-blocks scored at level 1 and candidate
    blocks scored at level 2 per query at position t."""
    c = t // w.block
    C = c // w.group
    scored_super = np.where(C + 1 <= w.top_m2, 0, C - 1)
    n_cand = (np.minimum(C + 1, w.top_m2) - 1) * w.group + (c - C * w.group) + 1
    scored_blocks = np.where(n_cand <= w.top_m, 0, n_cand)
    return scored_super, scored_blocks


def per_query_counts(w: Workload, t=None):
    """Closed-form per-query sizes: scored blocks, candidate tokens, kept tokens
    (queries at positions t; by default the last n_q positions).  With
    super-blocks the scored "blocks" are the level-1 super-blocks plus the
    level-2 candidate blocks."""
    if t is None:
        t = w.seq_len - w.n_q + np.arange(w.n_q, dtype=np.int64)
    t = np.asarray(t, dtype=np.int64)
    c = t // w.block
    if w.group:
        scored_blocks = sum(level1_counts(w, t))
        n_cand = (np.minimum(c // w.group + 1, w.top_m2) - 1) * w.group + (c - c // w.group * w.group) + 1
        n_sel = np.minimum(n_cand, w.top_m)
    else:
        scored_blocks = np.where(c + 1 <= w.top_m, 0, c - 1)
        n_sel = np.minimum(c + 1, w.top_m)
    n_valid = (n_sel - 1) * w.block + (t - c * w.block + 1)
    scored_tokens = np.where(n_valid <= w.top_k, 0, n_valid)
    kept = np.minimum(n_valid, w.top_k)
    return scored_blocks, scored_tokens, kept


def head_work(w: Workload) -> dict:
    """Per-head selection: landmarks of the touched chunks (K rows of every kv
    head read, nL landmark rows written), chunk scores (each kv head's
    landmark rows read once per query for its QPG heads), no token stage,
    attention over every causal token of each head's kept chunks (one kv
    head's K and V row per token and head)."""
    b, nq, Hq, Hkv, nL, d = w.batch, w.n_q, w.n_heads_q, w.n_heads_kv, w.n_landmarks, w.head_dim
    t = w.seq_len - nq + np.arange(nq, dtype=np.int64)
    c = t // w.block
    scored = np.where(c + 1 <= w.top_m, 0, c - 1)
    n_valid = (np.minimum(c + 1, w.top_m) - 1) * w.block + (t - c * w.block + 1)
    start = (w.seq_len - nq) // w.block
    rows = min(w.seq_len, w.n_blocks * w.block) - start * w.block
    lm_bytes = b * (rows * Hkv * d * 2 + (w.n_blocks - start) * nL * Hkv * d * 2)
    sel_bytes = b * (scored.sum() * nL * Hkv * d * 2 + nq * Hq * d * 2 + nq * Hq * w.top_m * 4)
    sel_flops = 2.0 * d * nL * Hq * b * scored.sum()
    attn_bytes = b * Hq * (n_valid.sum() * d * 2 * 2 + nq * d * (2 + 4))
    attn_flops = 4.0 * d * Hq * b * n_valid.sum()
    return {
        "block_summary": {"bytes": float(lm_bytes), "flops": 0.0},
        "block_topm": {"bytes": float(sel_bytes), "flops": float(sel_flops)},
        "token_topk": {"bytes": 0.0, "flops": 0.0},
        "sparse_attn": {"bytes": float(attn_bytes), "flops": float(attn_flops)},
    }


def algorithmic_work(w: Workload, lens=None) -> dict:
    """Bytes each step must move (and flops it must do), per stage.  With
    per-sequence lengths (one query each) every sequence counts at its own
    length and re-summarises its own last block."""
    if w.per_head:
        return head_work(w)
    b, nq = w.batch, w.n_q
    dI, nL, d = w.d_index, w.n_landmarks, w.head_dim
    if lens is None:
        sb, st, kept = (x * b for x in per_query_counts(w))
        start = (w.seq_len - nq) // w.block
        summ_rows = b * (min(w.seq_len, w.n_blocks * w.block) - start * w.block)
        summ_blocks = b * (w.n_blocks - start)
    else:
        t = np.asarray(lens, dtype=np.int64) - 1
        sb, st, kept = per_query_counts(w, t)
        summ_rows = int((t + 1 - (t // w.block) * w.block).sum())
        summ_blocks = b
    summ_bytes = summ_rows * dI * 2 + summ_blocks * nL * dI * 2
    topm_flops = 2.0 * dI * nL * sb.sum()
    topm_bytes = b * nq * dI * 2 + sb.sum() * nL * dI * 2 + b * nq * w.top_m * 4
    if w.group:
        # super-blocks from the first touched block's on are re-summarised
        # (their G block summaries read, one row written); level 1 writes and
        # level 2 reads the top_m2 lists
        start = (w.seq_len - nq) // w.block
        n_super = b * (w.n_super - start // w.group)
        summ_bytes += n_super * (w.group + 1) * nL * dI * 2
        topm_bytes += 2 * b * nq * w.top_m2 * 4
    topk_bytes = st.sum() * dI * 2 + b * nq * w.top_k * 4 + b * nq * w.top_m * 4
    attn_bytes = (kept.sum() * w.n_heads_kv * d * 2 * 2 + b * nq * w.n_heads_q * d * (2 + 4)
                  + b * nq * w.top_k * 4)
    attn_flops = 4.0 * d * w.n_heads_q * kept.sum()
    return {
        "block_summary": {"bytes": float(summ_bytes), "flops": 0.0},
        "block_topm": {"bytes": float(topm_bytes), "flops": float(topm_flops)},
        "token_topk": {"bytes": float(topk_bytes), "flops": float(2.0 * dI * st.sum())},
        "sparse_attn": {"bytes": float(attn_bytes), "flops": float(attn_flops)},
    }


KERNEL_STAGE = {
    "k_block_summary": "block_summary", "k_super_summary": "block_summary", "k_head_landmarks": "block_summary",
    "k_block_scores": "block_topm", "k_block_scores_mfma": "block_topm", "k_block_select": "block_topm",
    "k_block_scores_max": "block_topm", "k_block_topm_tile": "block_topm",
    "k_block_topm_decode": "block_topm", "k_block_topm_l2": "block_topm", "k_block_topm_3level_decode": "block_topm",
    "k_head_scores_mfma": "block_topm", "k_head_select": "block_topm",
    "k_token_scores": "token_topk", "k_token_scores_tiled": "token_topk", "k_bm_scores": "token_topk",
    "k_token_select": "token_topk", "k_token_enum": "token_topk",
    "k_sparse_attn": "sparse_attn", "k_attn_merge": "sparse_attn", "k_select_attn": "sparse_attn",
    "k_block_token_decode": "block_topm",
}


def kernel_work(w: Workload, kernel: str, lens=None) -> dict:
    """Algorithmic bytes and flops of one launch of `kernel` in one step, and
    the roof it is measured against.  Kernels that split a stage in two
    count the intermediate they hand over (fp32 scores, 4 bytes each) on
    both sides; a kernel that is the whole stage gets the stage's figure."""
    stage = KERNEL_STAGE.get(kernel)
    work = algorithmic_work(w, lens)
    b, nq, dI, nL = w.batch, w.n_q, w.d_index, w.n_landmarks
    if w.per_head:
        t = w.seq_len - nq + np.arange(nq, dtype=np.int64)
        c = t // w.block
        scored = float(b * w.n_heads_q * np.where(c + 1 <= w.top_m, 0, c - 1).sum())
        rows = b * nq * w.n_heads_q
        sel = work["block_topm"]
        if kernel == "k_head_scores_mfma":
            return {"bytes": sel["bytes"] - rows * w.top_m * 4 + scored * 4, "flops": sel["flops"], "bound": "hbm"}
        if kernel == "k_head_select":
            return {"bytes": scored * 4 + rows * w.top_m * 4 + rows * w.top_m * w.block * 4, "flops": 0.0,
                    "bound": "hbm"}
    else:
        if lens is None:
            sb, st, kept = (x * b for x in per_query_counts(w))
        else:
            sb, st, kept = per_query_counts(w, np.asarray(lens, dtype=np.int64) - 1)
        sb, st = float(sb.sum()), float(st.sum())
        nqt = b * nq
        if kernel in ("k_block_scores_mfma", "k_block_scores_max"):
            out = 4.0 * nqt if kernel == "k_block_scores_max" else sb * 4
            return {"bytes": out, "flops": 2.0 * dI * nL * sb, "bound": "mfma"}
        if kernel == "k_block_scores":
            return {"bytes": nqt * dI * 2 + sb * nL * dI * 2 + sb * 4, "flops": 2.0 * dI * nL * sb, "bound": "hbm"}
        if kernel == "k_block_select":
            return {"bytes": sb * 4 + nqt * w.top_m * 4, "flops": 0.0, "bound": "hbm"}
        if kernel in ("k_token_scores", "k_token_scores_tiled", "k_bm_scores"):
            # prefill scorers contract a tile of queries against kI rows that
            # many queries share (served from LDS, L2 and the MALL): MFMA roof
            bound = "hbm" if kernel == "k_token_scores" else "mfma"
            return {"bytes": nqt * dI * 2 + st * dI * 2 + st * 4, "flops": 2.0 * dI * st, "bound": bound}
        if kernel == "k_token_select":
            return {"bytes": st * 4 + nqt * w.top_k * 4, "flops": 0.0, "bound": "hbm"}
        if kernel == "k_block_token_decode":
            # the block top-m and the token scorer: both stages' bytes, less
            # the block lists the scorer would read back
            tb = work["block_topm"]
            return {"bytes": tb["bytes"] + st * dI * 2 + st * 4, "flops": tb["flops"] + 2.0 * dI * st,
                    "bound": "hbm"}
        if kernel == "k_select_attn":
            # the token select (scores and block lists in) and the attention
            # (the list it selects stays on chip; the list written out is
            # counted where the attention would read it)
            a = work["sparse_attn"]
            return {"bytes": a["bytes"] + st * 4 + nqt * w.top_m * 4, "flops": a["flops"], "bound": "hbm"}
    if stage is None:
        return {"bytes": 0.0, "flops": 0.0, "bound": "hbm"}
    # prefill attention gathers K/V rows that many queries share (a working
    # set far smaller than the bytes gathered, served from L2 and the MALL):
    # its roof is the bf16 MFMA rate of S = q K^T and O = P V; decode
    # attention streams each sequence's rows once: HBM
    bound = "mfma" if kernel == "k_sparse_attn" and regime(w) == "prefill" else "hbm"
    return {"bytes": work[stage]["bytes"], "flops": work[stage]["flops"], "bound": bound}


def regime(w: Workload) -> str:
    """"decode": one query per sequence, every byte of a step read once;
    "prefill": many queries per sequence re-reading shared rows."""
    return "decode" if w.n_q == 1 else "prefill"


# ----------------------------------------------------- hardware traffic


CSRC = os.path.join(ROOT, "hierarchical_index_sparse_amd", "csrc")


def kernel_source_hash(kernel: str) -> str:
    """sha256 of the .hip file that defines `kernel` and of the local headers
    it includes (directly or through other headers), in a fixed order."""
    import glob
    import hashlib
    import re
    inc_dirs = [CSRC, os.path.normpath(os.path.join(CSRC, os.pardir, os.pardir, "include"))]
    defining = [f for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
                if f"void {kernel}(" in open(f).read()]
    seen, todo = [], list(defining)
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.append(f)
        for name in re.findall(r'^#include "([^"]+)"', open(f).read(), flags=re.M):
            for d in inc_dirs:
                path = os.path.join(d, name)
                if os.path.exists(path):
                    todo.append(path)
                    break
    h = hashlib.sha256()
    for f in defining + sorted(set(seen) - set(defining), key=os.path.basename):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str, kernel: str):
    """Memory-fabric bytes per launch from the committed FETCH_SIZE /
    WRITE_SIZE record (profiles/<workload>_traffic.txt), each scaled by what
    the same counter read for a device copy of known size; None if there is
    no record for this kernel or its sources changed since it was taken.
    These counters count the bytes between the L2 caches and the fabric, so
    reads served by the MALL are included: an upper bound on DRAM bytes."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        rec[k.strip()] = v.strip()
    if rec.get("kernel") != kernel or rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    copy_kib = float(rec["copy_bytes"]) / 1024.0
    fetch_scale = copy_kib / float(rec["copy_fetch_size_kib"])
    write_scale = copy_kib / float(rec["copy_write_size_kib"])
    return 1024.0 * (float(rec["fetch_size_kib_per_dispatch"]) * fetch_scale
                     + float(rec["write_size_kib_per_dispatch"]) * write_scale)


# -------------------------------------------------------------- CPU oracle


_ORC_STATE = {}


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_one(args):
    from oracle import hisa_oracle as orc
    b, i = args
    w, inp, S = _ORC_STATE["w"], _ORC_STATE["inp"], _ORC_STATE["S"]
    lens = inp.get("seq_lens")
    t = w.query_pos(i) if lens is None else int(lens[b]) - 1
    if w.per_head:
        orc.forward_query_heads(inp, b, i, t, w.block, w.top_m, w.scale, S[b])
    elif w.group:
        orc.forward_query_3level(inp, b, i, t, w.block, w.group, w.top_m2, w.top_m, w.top_k, w.scale, S[b],
                                 _ORC_STATE["S2"][b])
    else:
        orc.forward_query(inp, b, i, t, w.block, w.top_m, w.top_k, w.scale, S_bits=S[b])
    return 1


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w: Workload, inp: dict, sample: int) -> dict:
    """Time the CPU oracle on an evenly spaced sample of the workload's queries."""
    import multiprocessing as mp

    from oracle import hisa_oracle as orc
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cores = max(1, min(cores, 16))
    t0 = time.perf_counter()
    lens = inp.get("seq_lens")
    if w.per_head:
        S = [orc.head_landmarks(inp["K"][b], w.block, inp.get("W")) for b in range(w.batch)]
    else:
        S = [orc.block_summary(inp["kI"][b] if lens is None else inp["kI"][b, :int(lens[b])], w.block,
                               inp.get("W")) for b in range(w.batch)]
    S2 = [orc.super_summary(x, w.group) for x in S] if w.group else None
    t_summary = time.perf_counter() - t0
    total = w.batch * w.n_q
    n = min(sample, total)
    flat = np.unique(np.linspace(0, total - 1, n).round().astype(np.int64))
    queries = [(int(x // w.n_q), int(x % w.n_q)) for x in flat]
    _ORC_STATE.update(w=w, inp=inp, S=S, S2=S2)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores, initializer=_oracle_worker_init) as pool:
        done = sum(pool.map(_oracle_one, queries, chunksize=max(1, len(queries) // (4 * cores))))
    wall = time.perf_counter() - t0
    _ORC_STATE.clear()
    # the summaries are built once per sequence: charge them in full
    # (they are handed on to parity_check under the underscore keys)
    return {
        "_S": S,
        "_S2": S2,
        "value": done / (wall + t_summary),
        "unit": "queries/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{done} of {total} queries, evenly spaced over the batch and positions; "
                  f"{'landmarks' if w.per_head else 'block summaries'}"
                  f"{' and super-block summaries' if w.group else ''} of all {w.batch} sequence(s) "
                  f"built once ({t_summary:.2f} s); "
                  f"{wall:.1f} s wall on {cores} worker processes",
    }


def parity_check(w: Workload, inp: dict, S, S2, gpu: dict, pairs) -> dict:
    """The oracle against the GPU outputs of the benchmarked configuration on
    the sampled (sequence, query) pairs: index sets bit for bit, O and lse
    within the 2e-3 max-abs bound.  gpu[key][n] holds pair n's row."""
    from oracle import hisa_oracle as orc
    lens = inp.get("seq_lens")
    exact, err_o, err_l = True, 0.0, 0.0
    for n, (b, i) in enumerate(pairs):
        t = w.query_pos(i) if lens is None else int(lens[b]) - 1
        if w.group:
            r = orc.forward_query_3level(inp, b, i, t, w.block, w.group, w.top_m2, w.top_m, w.top_k, w.scale, S[b],
                                         S2[b])
        else:
            r = orc.forward_query(inp, b, i, t, w.block, w.top_m, w.top_k, w.scale, S_bits=S[b])
        exact = exact and bool(np.array_equal(gpu["blk"][n], r["blk"]) and np.array_equal(gpu["tok"][n], r["tok"]))
        err_o = max(err_o, float(np.abs(gpu["O"][n].astype(np.float64) - r["O"]).max()))
        err_l = max(err_l, float(np.abs(gpu["lse"][n].astype(np.float64) - r["lse"]).max()))
    return {"queries": len(pairs), "index_sets_exact": exact, "max_abs_err_O": err_o, "max_abs_err_lse": err_l,
            "tolerance": PARITY_ATOL, "pass": exact and err_o <= PARITY_ATOL and err_l <= PARITY_ATOL}


PARITY_ATOL = 2e-3
PARITY_SAMPLE = 16


# ------------------------------------------------------------- HIP events


class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0


# ------------------------------------------------------- flat indexer


def flat_comparison(w: Workload, dev: dict, shape, S, start_block: int, steps: int, hip) -> dict | None:
    """Time hsa_flat_topk (score every causal token, keep top-k) on the same
    indexer inputs, against the hierarchical indexer called step by step:
    hsa_block_summary (the blocks a step re-summarises), hsa_block_topm and
    hsa_token_topk (scorer and select), so that no part of the indexer is
    hidden in a launch that hsa_forward shares with another step - the
    comparison the HISA page reports.  None when the flat indexer does not
    support the shape."""
    import torch

    from hierarchical_index_sparse_amd import _lib
    need = _lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_FLAT_TOPK)
    if need == 0 and w.top_k < w.seq_len:
        return None  # unsupported shape
    tok = torch.empty((w.batch, w.n_q, w.top_k), dtype=torch.int32, device="cuda")
    blk = torch.empty((w.batch, w.n_q, w.top_m), dtype=torch.int32, device="cuda")
    n = max(3, min(steps, 10))
    stream = torch.cuda.current_stream().cuda_stream

    def timed(call):
        call()
        torch.cuda.synchronize()
        ev = [(hip.create(), hip.create()) for _ in range(n)]
        for a, b in ev:
            hip.record(a, stream)
            call()
            hip.record(b, stream)
        torch.cuda.synchronize()
        ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in ev]))
        for a, b in ev:
            hip.destroy(a)
            hip.destroy(b)
        return ms

    ws_b = torch.empty(max(_lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_BLOCK_TOPM), 1),
                       dtype=torch.uint8, device="cuda")
    ws_t = torch.empty(max(_lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_TOKEN_TOPK), 1),
                       dtype=torch.uint8, device="cuda")

    def hierarchical():
        _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), start_block, S)
        _lib.hsa_block_topm(shape, dev["qI"], S, blk, ws_b)
        _lib.hsa_token_topk(shape, dev["qI"], dev["kI"], blk, tok, ws_t)

    hier_ms = timed(hierarchical)
    del ws_b, ws_t
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    flat_ms = timed(lambda: _lib.hsa_flat_topk(shape, dev["qI"], dev["kI"], tok, ws))
    del ws, tok, blk
    torch.cuda.empty_cache()
    return {"flat_indexer_ms": flat_ms, "hierarchical_indexer_ms": hier_ms, "speedup": flat_ms / hier_ms,
            "note": "same inputs and output form; hierarchical = hsa_block_summary (re-summarised blocks) + "
                    "hsa_block_topm + hsa_token_topk, called one after the other"}


def two_level_comparison(w: Workload, dev: dict, shape, stage_ms: dict, blk3, steps: int, hip) -> dict:
    """Time the two-level hsa_forward (every causal block scored) on the same
    inputs, m and k, against the three-level stages, and report how many of
    its kept blocks the three-level selection also keeps."""
    import torch

    from hierarchical_index_sparse_amd import _lib, pipeline
    w2 = w.with_(group=0, top_m2=0)
    out = pipeline.alloc_outputs(w2)
    ws = torch.empty(_lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_FORWARD), dtype=torch.uint8,
                     device="cuda")
    start = (w.seq_len - w.n_q) // w.block
    _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, out["S"])

    def run(lists):
        _lib.hsa_forward(shape, dev["qI"], dev["kI"], dev.get("W"), start, out["S"], dev["Q"], dev["K"], dev["V"],
                         out["blk"] if lists else None, None, out["O"], out["lse"], ws)

    run(True)
    torch.cuda.synchronize()
    blk2 = out["blk"].cpu().numpy().reshape(-1, w.top_m)
    b3 = blk3.reshape(-1, w.top_m)
    overlap = float(np.mean([np.intersect1d(x[x >= 0], y[y >= 0]).size / max(1, (x >= 0).sum())
                             for x, y in zip(blk2, b3)]))
    n = max(3, min(steps, 10))
    events = [[hip.create() for _ in range(5)] for _ in range(n)]
    for s in range(n):
        _lib.hsa_sparse_set_stage_events(events[s])
        run(False)
    torch.cuda.synchronize()
    _lib.hsa_sparse_set_stage_events(None)
    st2 = {name: float(np.mean([hip.elapsed_ms(ev[i], ev[i + 1]) for ev in events]))
           for i, name in enumerate(STAGES)}
    step2 = float(np.mean([hip.elapsed_ms(ev[0], ev[4]) for ev in events]))
    for ev in events:
        for e in ev:
            hip.destroy(e)
    del out, ws
    torch.cuda.empty_cache()
    return {"two_level_stage_ms": st2, "two_level_step_ms": step2,
            "three_level_block_stages_ms": stage_ms["block_summary"] + stage_ms["block_topm"],
            "two_level_block_stages_ms": st2["block_summary"] + st2["block_topm"],
            "block_list_overlap": overlap,
            "note": "same inputs, m and k; block stages = summaries + block selection; overlap = mean fraction "
                    "of the two-level kept blocks that the three-level selection also keeps"}


def dense_comparison(w: Workload, dev: dict, steps: int, hip, step_ms: float) -> dict:
    """Time exact attention over every causal token (the full attention the
    HiLS page measures its decode speedup against) on the same Q, K, V with
    hsa_sparse_attn and a list 0..t per query."""
    import torch

    from hierarchical_index_sparse_amd import _lib
    wd = w.with_(per_head=False, top_k=w.seq_len)
    shape = _lib.shape_of(wd)
    t = w.seq_len - w.n_q + torch.arange(w.n_q, device="cuda", dtype=torch.int32)
    s = torch.arange(w.seq_len, device="cuda", dtype=torch.int32)
    tok = torch.where(s[None, :] <= t[:, None], s[None, :], torch.full_like(s[None, :], -1))
    tok = tok[None].expand(w.batch, -1, -1).contiguous()
    O = torch.empty((w.batch, w.n_q, w.n_heads_q, w.head_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, _lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_SPARSE_ATTN)),
                     dtype=torch.uint8, device="cuda")
    _lib.hsa_sparse_attn(shape, dev["Q"], dev["K"], dev["V"], tok, O, None, ws)
    torch.cuda.synchronize()
    n = max(3, min(steps, 10))
    ev = [(hip.create(), hip.create()) for _ in range(n)]
    stream = torch.cuda.current_stream().cuda_stream
    for a, b in ev:
        hip.record(a, stream)
        _lib.hsa_sparse_attn(shape, dev["Q"], dev["K"], dev["V"], tok, O, None, ws)
        hip.record(b, stream)
    torch.cuda.synchronize()
    dense_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in ev]))
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    kv_bytes = w.batch * w.n_q * w.seq_len * w.n_heads_kv * w.head_dim * 2 * 2
    del tok, O, ws
    torch.cuda.empty_cache()
    return {"dense_attention_ms": dense_ms, "dense_hbm_frac": kv_bytes / (dense_ms / 1000.0) / 1e9 / HBM_PEAK_GBS,
            "sparse_step_ms": step_ms, "speedup": dense_ms / step_ms,
            "note": "dense = exact attention of every query over all causal tokens (hsa_sparse_attn, same Q/K/V); "
                    "sparse = the whole per-head step (landmarks of the touched chunk, selection, attention)"}


# ------------------------------------------------------------------- main


# the SURVEY configurations reported beside the headline workload
# the timed region's steps whose dominant-kernel dispatches carry events
EVENT_EVERY = 8

CONFIG_WORKLOADS = ("decode_128k", "chunked_prefill_512k", "decode_512k", "landmark_decode_1m")


def measured_peaks(hip) -> dict:
    """What this GPU reaches on a plain device copy (torch's copy kernel,
    1 GiB read + 1 GiB written) and on a large bf16 GEMM (torch.matmul,
    8192^3, hipBLASLt), best of several runs each: the measured ceilings the
    vendor peaks are set against."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    out = {}

    def best_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = hip.create(), hip.create()
            hip.record(a, stream)
            fn()
            hip.record(b, stream)
            times.append(hip.elapsed_ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        return min(times)

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = best_ms(lambda: dst.copy_(src), 10)
    out["copy_GBs"] = 2.0 * n / (ms / 1000.0) / 1e9
    del src, dst
    m = 8192
    a = torch.randn((m, m), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((m, m), device="cuda", dtype=torch.bfloat16)
    c = torch.empty((m, m), device="cuda", dtype=torch.bfloat16)
    ms = best_ms(lambda: torch.matmul(a, b, out=c), 10)
    out["bf16_gemm_TFLOPs"] = 2.0 * m ** 3 / (ms / 1000.0) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    out["vendor_hbm_GBs"] = HBM_PEAK_GBS
    out["vendor_bf16_mfma_TFLOPs"] = MFMA_BF16_PEAK_TFLOPS
    out["note"] = ("copy: 1 GiB device-to-device copy (2 GiB moved), best of 10; gemm: 8192^3 bf16 torch.matmul, "
                   "best of 10")
    return out


def roofline_entry(w: Workload, kernel: str, kernel_ms: float, n_launch: int, lens, peaks: dict | None) -> dict:
    """The roofline of one kernel: algorithmic work per launch over its
    average duration, against the roof its regime is bound by (bf16 MFMA
    for the contractions over shared, cache-resident operands; HBM for
    kernels that stream their bytes once).  kernel_ms is the kernel's time
    in one step, summed over its n_launch launches (a long prefill runs the
    attention once per query chunk); the rate is the same either way."""
    kw = kernel_work(w, kernel, lens)
    sec = kernel_ms / 1000.0
    if kw["bound"] == "mfma":
        achieved = kw["flops"] / sec / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
        if peaks:
            roof["frac_of_measured_gemm"] = achieved / peaks["bf16_gemm_TFLOPs"]
        if kw["bytes"]:
            roof["gather_rate_GBs"] = kw["bytes"] / sec / 1e9
            roof["gather_note"] = ("algorithmic bytes gathered per second; rows shared by many queries are served "
                                   "from LDS, L2 and the MALL, so this is a rate, not a fraction of HBM")
        roof["algorithmic_per_launch"] = kw["flops"] / n_launch
    else:
        achieved = kw["bytes"] / sec / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        if peaks:
            roof["frac_of_measured_copy"] = achieved / peaks["copy_GBs"]
        roof["algorithmic_per_launch"] = kw["bytes"] / n_launch
    roof["traffic"] = recorded_traffic(w.name, kernel)
    roof["traffic_note"] = ("FETCH_SIZE and WRITE_SIZE per launch, scaled by a copy of known size: bytes between "
                            "L2 and the memory fabric, MALL hits included (an upper bound on DRAM bytes)")
    if roof["traffic"] is not None:
        # the counted bytes over the launch time: the second reading of the
        # HBM fraction, an upper bound on the DRAM rate (MALL hits included)
        rate = roof["traffic"] / (kernel_ms / 1000.0 / n_launch) / 1e9
        roof["traffic_GBs"] = rate
        roof["traffic_frac_of_hbm_peak"] = rate / HBM_PEAK_GBS
    roof["kernel"] = kernel
    roof["stage"] = KERNEL_STAGE.get(kernel)
    roof["launches_per_step"] = n_launch
    roof["avg_launch_us"] = kernel_ms * 1000.0 / n_launch
    roof["kernel_ms_timed"] = kernel_ms
    roof["kernel_ms_note"] = ("the kernel's launches in one step, summed (a long prefill runs it once per query chunk), "
                              f"by HIP events on every {EVENT_EVERY}th step of the timed region; "
                              "algorithmic_per_launch is the step's work over its launches")
    return roof


def stage_rates(w: Workload, work: dict, stage_ms: dict) -> dict:
    """Per stage: time, algorithmic bytes and flops per second, and the
    fraction of a roof only where it is one: HBM for stages that stream
    their bytes once (decode, and the block summaries), bf16 MFMA for the
    stages with MFMA contractions.  Prefill stages gather rows that many
    queries share, so their byte rates are rates only."""
    out = {}
    for n in STAGES:
        sec = stage_ms[n] / 1000.0
        gbs = work[n]["bytes"] / sec / 1e9 if sec > 0 else 0.0
        tfs = work[n]["flops"] / sec / 1e12 if sec > 0 else 0.0
        e = {"ms": stage_ms[n], "algorithmic_GBs": gbs}
        streams = regime(w) == "decode" or n == "block_summary"
        e["hbm_frac"] = gbs / HBM_PEAK_GBS if streams and gbs <= HBM_PEAK_GBS else None
        if work[n]["flops"]:
            e["TFLOPs"] = tfs
            e["mfma_frac"] = tfs / MFMA_BF16_PEAK_TFLOPS
        out[n] = e
    return out


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measure(w: Workload, inp: dict, args, hip, peaks=None, ora=None, headline=True) -> dict:
    """Time K steps of the workload's whole path (after W warmup steps) and
    the breakdowns around them; check the benchmarked configuration's
    outputs against the oracle when `ora` (its summaries) is given."""
    import torch

    from hierarchical_index_sparse_amd import _lib, pipeline
    dev = pipeline.to_device(inp)
    out = pipeline.alloc_outputs(w)
    shape = _lib.shape_of(w)
    op = _lib.HSA_SPARSE_OP_FORWARD_HEADS if w.per_head else _lib.HSA_SPARSE_OP_FORWARD
    ws = torch.empty(_lib.hsa_sparse_workspace_size(shape, op), dtype=torch.uint8, device="cuda")

    # summaries of blocks before the new queries are state (built once at
    # ingest); each step re-summarises the blocks the queries' tokens touch
    start_block = (w.seq_len - w.n_q) // w.block
    if w.per_head:
        _lib.hsa_head_landmarks(shape, dev["K"], dev.get("W"), 0, out["LK"])
    else:
        _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, out["S"])

    lens = inp.get("seq_lens")

    if w.group:
        _lib.hsa_super_summary(shape, w.group, out["S"], 0, out["S2"])

    def checked_step():
        if w.per_head:
            _lib.hsa_forward_heads(shape, dev.get("W"), start_block, dev["Q"], dev["K"], dev["V"], out["LK"], None,
                                   out["O"], out["lse"], ws)
        elif w.group:
            _lib.hsa_forward_3level(shape, w.group, w.top_m2, dev["qI"], dev["kI"], dev.get("W"), start_block,
                                    out["S"], out["S2"], dev["Q"], dev["K"], dev["V"], out["sup"], None, None,
                                    out["O"], out["lse"], ws)
        elif lens is None:
            _lib.hsa_forward(shape, dev["qI"], dev["kI"], dev.get("W"), start_block, out["S"], dev["Q"], dev["K"],
                             dev["V"], None, None, out["O"], out["lse"], ws)
        else:  # one decode step over sequences of different lengths
            _lib.hsa_decode_step(shape, dev["seq_lens"], dev["qI"], dev["kI"], dev.get("W"), out["S"], dev["Q"],
                                 dev["K"], dev["V"], None, None, out["O"], out["lse"], ws)

    # After one call through the checking wrappers above, steps call the
    # entry point with its arguments marshalled once, so that the host's
    # per-call cost (tens of microseconds of Python checks) does not pace
    # the short decode steps.
    checked_step()
    torch.cuda.synchronize()
    lib = _lib.load()
    sref = ctypes.byref(shape)
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = ws.numel()

    def ptr(t):
        return None if t is None else t.data_ptr()

    if w.per_head:
        fn, call_args = lib.hsa_forward_heads, (sref, None, ptr(dev.get("W")), start_block, ptr(dev["Q"]),
                                                ptr(dev["K"]), ptr(dev["V"]), ptr(out["LK"]), None, ptr(out["O"]),
                                                ptr(out["lse"]), ptr(ws), nbytes, stream)
    elif w.group:
        fn, call_args = lib.hsa_forward_3level, (sref, None, w.group, w.top_m2, ptr(dev["qI"]), ptr(dev["kI"]),
                                                 ptr(dev.get("W")), start_block, ptr(out["S"]), ptr(out["S2"]),
                                                 ptr(dev["Q"]), ptr(dev["K"]), ptr(dev["V"]), ptr(out["sup"]), None,
                                                 None, ptr(out["O"]), ptr(out["lse"]), ptr(ws), nbytes, stream)
    elif lens is None:
        fn, call_args = lib.hsa_forward, (sref, ptr(dev["qI"]), ptr(dev["kI"]), ptr(dev.get("W")), start_block,
                                          ptr(out["S"]), ptr(dev["Q"]), ptr(dev["K"]), ptr(dev["V"]), None, None,
                                          ptr(out["O"]), ptr(out["lse"]), ptr(ws), nbytes, stream)
    else:
        fn, call_args = lib.hsa_decode_step, (sref, ptr(dev["seq_lens"]), ptr(dev["qI"]), ptr(dev["kI"]),
                                              ptr(dev.get("W")), ptr(out["S"]), ptr(dev["Q"]), ptr(dev["K"]),
                                              ptr(dev["V"]), None, None, ptr(out["O"]), ptr(out["lse"]), ptr(ws),
                                              nbytes, stream)

    def step():
        st = fn(*call_args)
        if st != 0:
            raise _lib.HsaSparseError(st, fn.__name__, lib.hsa_sparse_last_error().decode())

    if args.calibrate_copy_mib and headline:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Stage breakdown (untimed): all five stage boundaries recorded.  Every
    # recorded event costs the stream a few microseconds, so the timed region
    # below records none of them.
    n_prof = max(3, min(args.steps, 10))
    events = [[hip.create() for _ in range(5)] for _ in range(n_prof)]
    for s in range(n_prof):
        _lib.hsa_sparse_set_stage_events(events[s])
        step()
    torch.cuda.synchronize()
    _lib.hsa_sparse_set_stage_events(None)
    stage_ms = {name: float(np.mean([hip.elapsed_ms(ev[i], ev[i + 1]) for ev in events]))
                for i, name in enumerate(STAGES)}
    gpu_step_ms = float(np.mean([hip.elapsed_ms(ev[0], ev[4]) for ev in events]))
    for ev in events:
        for e in ev:
            hip.destroy(e)
    # Kernel breakdown (untimed): every kernel's dispatch carries its own
    # start/stop events (hsa_sparse_set_kernel_events), which add no work
    # to the stream.  A kernel may run several times in a step (long
    # prefills run the token stage and the attention in query chunks), so
    # times are summed per kernel name; the largest sum is the dominant
    # kernel.
    n_slots = 64
    kev = [([hip.create() for _ in range(n_slots)], [hip.create() for _ in range(n_slots)]) for _ in range(n_prof)]
    for s in range(n_prof):
        _lib.hsa_sparse_set_kernel_events(kev[s][0], kev[s][1])
        step()
    torch.cuda.synchronize()
    names = _lib.hsa_sparse_last_kernels()
    _lib.hsa_sparse_set_kernel_events(None, None)
    nk = min(len(names), n_slots)
    launch_us = [float(np.mean([hip.elapsed_ms(kev[s][0][i], kev[s][1][i]) for s in range(n_prof)])) * 1000.0
                 for i in range(nk)]
    for a, b in kev:
        for e in a + b:
            hip.destroy(e)
    order = list(dict.fromkeys(names[:nk]))
    kernel_us = [(n, sum(u for m, u in zip(names, launch_us) if m == n), names[:nk].count(n)) for n in order]
    dom = max(kernel_us, key=lambda x: x[1])[0]
    dom_idx = [i for i in range(nk) if names[i] == dom]

    # Timed region: K whole steps.  The dominant kernel's dispatches carry
    # start/stop events on every EVENT_EVERY-th step (steps 0, 8, 16, ...),
    # giving its duration in those steps; an event-carrying dispatch costs
    # the stream several microseconds (about 6 us per decode step), so events
    # on every step would slow the very steps being timed.  Event arrays are
    # built before the loop.
    sampled = list(range(0, args.steps, EVENT_EVERY))
    timed = [[(hip.create(), hip.create()) for _ in dom_idx] for _ in sampled]
    Ev = ctypes.c_void_p * (dom_idx[-1] + 1)
    ev_arrays = [None] * args.steps
    for s_i, evs in zip(sampled, timed):
        st_ev, sp_ev = Ev(), Ev()
        for i, (a, b) in zip(dom_idx, evs):
            st_ev[i], sp_ev[i] = a, b
        ev_arrays[s_i] = (st_ev, sp_ev)
    set_kev = lib.hsa_sparse_set_kernel_events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for evs in ev_arrays:
        if evs is not None:
            set_kev(evs[0], evs[1], dom_idx[-1] + 1)
            step()
            set_kev(None, None, 0)
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms = float(np.mean([sum(hip.elapsed_ms(a, b) for a, b in evs) for evs in timed]))
    for evs in timed:
        for a, b in evs:
            hip.destroy(a)
            hip.destroy(b)

    # Parity of the benchmarked configuration: one more call writes the index
    # lists too; its O must equal the timed steps' bit for bit, and a sample
    # of queries is checked against the oracle.  Per-head lists rank float
    # scores and are checked with an fp32 bound in the tests instead.
    parity = None
    if ora is not None and not w.per_head:
        ora_S, ora_S2 = ora
        chk = pipeline.alloc_outputs(w)
        if w.group:
            _lib.hsa_forward_3level(shape, w.group, w.top_m2, dev["qI"], dev["kI"], dev.get("W"), start_block,
                                    out["S"], out["S2"], dev["Q"], dev["K"], dev["V"], chk["sup"], chk["blk"],
                                    chk["tok"], chk["O"], chk["lse"], ws)
        elif lens is None:
            _lib.hsa_forward(shape, dev["qI"], dev["kI"], dev.get("W"), start_block, out["S"], dev["Q"], dev["K"],
                             dev["V"], chk["blk"], chk["tok"], chk["O"], chk["lse"], ws)
        else:
            _lib.hsa_decode_step(shape, dev["seq_lens"], dev["qI"], dev["kI"], dev.get("W"), out["S"], dev["Q"],
                                 dev["K"], dev["V"], chk["blk"], chk["tok"], chk["O"], chk["lse"], ws)
        torch.cuda.synchronize()
        same = bool(torch.equal(chk["O"], out["O"]) and torch.equal(chk["lse"], out["lse"]))
        total = w.batch * w.n_q
        flat_ids = np.unique(np.linspace(0, total - 1, min(PARITY_SAMPLE, total)).round().astype(np.int64))
        pairs = [(int(x // w.n_q), int(x % w.n_q)) for x in flat_ids]
        bs = torch.tensor([p[0] for p in pairs], device="cuda")
        qs = torch.tensor([p[1] for p in pairs], device="cuda")
        rows = {key: chk[key][bs, qs].cpu().numpy() for key in ("blk", "tok", "O", "lse")}
        del chk
        parity = parity_check(w, inp, ora_S, ora_S2, rows, pairs)
        parity["timed_outputs_identical"] = same
        parity["pass"] = parity["pass"] and same

    extras = {}
    if regime(w) == "prefill" and not (w.per_head or w.group or lens is not None):
        extras["block_score_mfma"] = block_score_mfma(w, dev, out["S"], hip, args.steps, peaks,
                                                      stage_ms["block_topm"])
    if headline:
        # the flat indexer takes one length for the batch
        if not (args.no_flat or lens is not None or w.group or w.per_head):
            extras["indexer_vs_flat"] = flat_comparison(w, dev, shape, out["S"], start_block, args.steps, hip)
        if w.group:
            blk3 = pipeline.alloc_outputs(w)["blk"]
            _lib.hsa_block_topm_3level(shape, w.group, w.top_m2, dev["qI"], out["S"], out["S2"], out["sup"], blk3)
            torch.cuda.synchronize()
            extras["three_level_vs_two_level"] = two_level_comparison(w, dev, shape, stage_ms, blk3.cpu().numpy(),
                                                                      args.steps, hip)
        if w.per_head:
            extras["per_head_vs_dense_attention"] = dense_comparison(w, dev, args.steps, hip, gpu_step_ms)
    del dev, out, ws
    torch.cuda.empty_cache()

    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    queries = w.batch * w.n_q
    work = algorithmic_work(w, lens)
    step_bytes = sum(work[n]["bytes"] for n in STAGES)
    step_flops = sum(work[n]["flops"] for n in STAGES)
    step_sec = ms_per_step / 1000.0
    step = {"algorithmic_GB": step_bytes / 1e9, "algorithmic_TFLOP": step_flops / 1e12}
    if regime(w) == "decode":
        # every byte of a decode step is read once: the whole step against HBM
        step["hbm_frac"] = step_bytes / step_sec / 1e9 / HBM_PEAK_GBS
    else:
        step["mfma_frac"] = step_flops / step_sec / 1e12 / MFMA_BF16_PEAK_TFLOPS
    return {
        "value": queries / step_sec,
        "ms_per_step": ms_per_step,
        "stage_ms": stage_ms,
        "kernel_us": [[n, round(u, 2), c] for n, u, c in kernel_us],
        "gpu_step_ms_all_stage_events": gpu_step_ms,
        "stage_rates": stage_rates(w, work, stage_ms),
        "step_roofline": step,
        "roofline": roofline_entry(w, dom, dom_ms, len(dom_idx), lens, peaks),
        "parity": parity,
        **extras,
    }


def block_score_mfma(w: Workload, dev: dict, S, hip, steps: int, peaks: dict | None, stage_ms: float) -> dict:
    """The block-score contraction on its own: hsa_block_score_max runs the
    MFMA tiling of step 2 with each query's maximum formed on chip (4 bytes
    per query leave it), so its kernel time is the contraction's.  Measured
    against the bf16 MFMA peak with the algorithmic causal flops (scored
    blocks x landmark rows x 2 d_index)."""
    import torch

    from hierarchical_index_sparse_amd import _lib
    shape = _lib.shape_of(w)
    out = torch.empty((w.batch, w.n_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, _lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_BLOCK_SCORE_MAX)),
                     dtype=torch.uint8, device="cuda")
    _lib.hsa_block_score_max(shape, dev["qI"], S, out, ws)
    torch.cuda.synchronize()
    n = max(5, min(steps, 20))
    # events around each kernel of the call (a second kernel reduces per-chunk
    # maxima when the rows are split over workgroups); the time runs from the
    # first kernel's start to the last kernel's end
    ev = [[hip.create() for _ in range(4)] for _ in range(n)]
    names = None
    for a0, a1, b0, b1 in ev:
        _lib.hsa_sparse_set_kernel_events([a0, a1], [b0, b1])
        _lib.hsa_block_score_max(shape, dev["qI"], S, out, ws)
        names = _lib.hsa_sparse_last_kernels()
    torch.cuda.synchronize()
    _lib.hsa_sparse_set_kernel_events(None, None)
    last = len(names) - 1
    us = float(np.mean([hip.elapsed_ms(e[0], e[2 + last]) for e in ev])) * 1000.0
    for e in ev:
        for x in e:
            hip.destroy(x)
    del out, ws
    sb, _, _ = per_query_counts(w)
    flops = 2.0 * w.d_index * w.n_landmarks * float(sb.sum()) * w.batch
    tfs = flops / (us / 1e6) / 1e12
    res = {"kernel": names[0], "kernels": names, "kernel_us": us, "algorithmic_GFLOP": flops / 1e9,
           "achieved_TFLOPs": tfs, "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "frac": tfs / MFMA_BF16_PEAK_TFLOPS,
           "block_topm_stage_ms": stage_ms,
           "note": "score-only build of the block-score MFMA tiling (per-query maximum on chip, 4 B per query "
                   "written); the block_topm stage (scores written, then the exact top-m select) for comparison"}
    if peaks:
        res["frac_of_measured_gemm"] = tfs / peaks["bf16_gemm_TFLOPs"]
    return res


def config_of(w: Workload, args, lens) -> dict:
    return {"workload": w.name, "batch_override": args.batch > 0,
            "summary_start_block": (w.seq_len - w.n_q) // w.block if lens is None else "each sequence's last block",
            "seq_lens": None if lens is None else f"uniform in [{w.varlen_min}, {w.seq_len}], "
                                                  f"mean {float(np.mean(lens)):.0f} (seeded)",
            "batch": w.batch, "seq_len": w.seq_len, "n_q": w.n_q,
            "d_index": w.d_index, "block": w.block, "top_m": w.top_m, "top_k": w.top_k,
            "heads_q": w.n_heads_q, "heads_kv": w.n_heads_kv, "head_dim": w.head_dim,
            "n_landmarks": w.n_landmarks,
            **({"group": w.group, "top_m2": w.top_m2} if w.group else {}),
            **({"selection": "per query head from Q and landmarks of K"} if w.per_head else {}),
            "parallelism": "single GPU"}


def oracle_state(w: Workload, inp: dict):
    """The oracle's summaries (and super-block summaries) of every sequence,
    for the parity check of a configuration (single process)."""
    from oracle import hisa_oracle as orc
    if w.per_head:
        return None
    lens = inp.get("seq_lens")
    S = [orc.block_summary(inp["kI"][b] if lens is None else inp["kI"][b, :int(lens[b])], w.block, inp.get("W"))
         for b in range(w.batch)]
    return S, ([orc.super_summary(x, w.group) for x in S] if w.group else None)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_64k", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-sample", type=int, default=1024, help="queries the CPU oracle is timed on")
    ap.add_argument("--batch", type=int, default=0,
                    help="run the workload at this batch instead of its own (a batch study: the line then says "
                         "batch_override; the workload's own batch is the measured configuration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flat", action="store_true",
                    help="skip timing the flat indexer (every causal token scored) on the same inputs")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the headline workload (default: also the other SURVEY configurations, "
                         "reported under 'configs')")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring copy bandwidth and GEMM rate")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a kernel of known "
                         "traffic, to scale hardware byte counters against)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(decode sequences and prefill queries would shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    w = WORKLOADS[args.workload]
    if args.batch > 0:
        w = dataclasses.replace(w, batch=args.batch)
    progress(f"inputs of {w.name}")
    inp = datagen.make_inputs(w)
    # the oracle is timed in forked worker processes: before the GPU is touched
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, inp, args.cpu_sample)
    ora = None if cpu is None else (cpu.pop("_S"), cpu.pop("_S2"))

    import torch  # noqa: F401
    hip = HipEvents()
    progress("measured peaks")
    peaks = None if args.no_peaks else measured_peaks(hip)
    progress(f"measuring {w.name}")
    head = measure(w, inp, args, hip, peaks, ora, headline=True)
    lens = inp.get("seq_lens")
    del inp

    configs = None
    explicit = any(a == "--workload" or a.startswith("--workload=") for a in sys.argv[1:])
    if not (args.no_configs or explicit or args.batch):
        configs = {}
        for name in CONFIG_WORKLOADS:
            wc = WORKLOADS[name]
            progress(f"inputs of {name}")
            cinp = datagen.make_inputs(wc)
            progress(f"measuring {name}")
            r = measure(wc, cinp, args, hip, peaks, oracle_state(wc, cinp), headline=False)
            del cinp
            configs[name] = {"value": r["value"], "unit": "queries/s", "ms_per_step": r["ms_per_step"],
                             "stage_ms": r["stage_ms"], "kernel_us": r["kernel_us"],
                             "stage_rates": r["stage_rates"], "step_roofline": r["step_roofline"],
                             "roofline": r["roofline"], "parity": r["parity"],
                             **({"block_score_mfma": r["block_score_mfma"]} if "block_score_mfma" in r else {}),
                             "config": config_of(wc, args, None)}

    res = {
        "metric": "queries/sec end-to-end (index+attn)",
        "value": head["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "fp32",
        "data": ("synthetic (seeded; N(0,1) bf16 Q/K/V, one planted needle chunk per sequence and kv head)"
                 if w.per_head else "synthetic (seeded; integer-valued bf16 indexer vectors, N(0,1) bf16 Q/K/V)"),
        "config": config_of(w, args, lens),
        **{k: v for k, v in head.items() if k not in ("value", "ms_per_step")},
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
