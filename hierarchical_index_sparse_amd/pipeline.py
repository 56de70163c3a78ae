"""Run the four steps on the GPU through the C ABI.

Plumbing only: allocates output tensors with torch, moves host inputs to
the device and calls the entry points of libhsa_sparse.so in order.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from .workloads import Workload


def to_device(inp: dict, device="cuda") -> dict:
    """Host arrays (bf16 as uint16 bits, W as int8) -> GPU tensors."""
    out = {}
    for key, arr in inp.items():
        if arr is None or key.endswith("needles"):
            out[key] = arr
            continue
        a = np.ascontiguousarray(arr)
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out[key] = t.to(device, non_blocking=False)
    return out


def alloc_outputs(w: Workload, device="cuda") -> dict:
    nqt = (w.batch, w.n_q)
    res = {
        "S": torch.zeros((w.batch, w.n_blocks, w.n_landmarks, w.d_index), dtype=torch.bfloat16, device=device),
        "blk": torch.full(nqt + (w.top_m,), -7, dtype=torch.int32, device=device),
        "tok": torch.full(nqt + (w.top_k,), -7, dtype=torch.int32, device=device),
        "O": torch.full(nqt + (w.n_heads_q, w.head_dim), float("nan"), dtype=torch.float32, device=device),
        "lse": torch.full(nqt + (w.n_heads_q,), float("nan"), dtype=torch.float32, device=device),
    }
    if w.per_head:
        qh = nqt + (w.n_heads_q,)
        return {
            "LK": torch.zeros((w.batch, w.n_blocks, w.n_landmarks, w.n_heads_kv, w.head_dim), dtype=torch.bfloat16,
                              device=device),
            "blk": torch.full(qh + (w.top_m,), -7, dtype=torch.int32, device=device),
            "O": res["O"],
            "lse": res["lse"],
        }
    if w.group:
        res["S2"] = torch.zeros((w.batch, w.n_super, w.n_landmarks, w.d_index), dtype=torch.bfloat16, device=device)
        res["sup"] = torch.full(nqt + (w.top_m2,), -7, dtype=torch.int32, device=device)
    return res


def run_stages(w: Workload, dev: dict, out: dict | None = None, attention: bool = True) -> dict:
    """Steps 1-4 through the four single-step entry points."""
    shape = _lib.shape_of(w)
    out = out or alloc_outputs(w, dev["qI"].device)
    _lib.hsa_block_summary(shape, dev["kI"], dev.get("W"), 0, out["S"])
    _lib.hsa_block_topm(shape, dev["qI"], out["S"], out["blk"])
    _lib.hsa_token_topk(shape, dev["qI"], dev["kI"], out["blk"], out["tok"])
    if attention:
        _lib.hsa_sparse_attn(shape, dev["Q"], dev["K"], dev["V"], out["tok"], out["O"], out["lse"])
    return out


def run_forward(w: Workload, dev: dict, out: dict | None = None, keep_lists: bool = True,
                workspace: torch.Tensor | None = None, summary_start_block: int = 0) -> dict:
    """Steps 1-4 through hsa_forward."""
    shape = _lib.shape_of(w)
    out = out or alloc_outputs(w, dev["qI"].device)
    _lib.hsa_forward(shape, dev["qI"], dev["kI"], dev.get("W"), summary_start_block, out["S"], dev["Q"],
                     dev["K"], dev["V"], out["blk"] if keep_lists else None,
                     out["tok"] if keep_lists else None, out["O"], out["lse"], workspace)
    return out


def run_forward_3level(w: Workload, dev: dict, out: dict | None = None, keep_lists: bool = True,
                       workspace: torch.Tensor | None = None, summary_start_block: int = 0,
                       seq_lens: torch.Tensor | None = None) -> dict:
    """Steps 1-4 through hsa_forward_3level (super-blocks of w.group blocks)."""
    shape = _lib.shape_of(w)
    out = out or alloc_outputs(w, dev["qI"].device)
    _lib.hsa_forward_3level(shape, w.group, w.top_m2, dev["qI"], dev["kI"], dev.get("W"), summary_start_block,
                            out["S"], out["S2"], dev["Q"], dev["K"], dev["V"], out["sup"],
                            out["blk"] if keep_lists else None, out["tok"] if keep_lists else None, out["O"],
                            out["lse"], workspace, seq_lens=seq_lens)
    return out


def run_forward_heads(w: Workload, dev: dict, out: dict | None = None, keep_lists: bool = True,
                      workspace: torch.Tensor | None = None, summary_start_block: int = 0,
                      seq_lens: torch.Tensor | None = None) -> dict:
    """Per-head chunk selection and attention through hsa_forward_heads."""
    shape = _lib.shape_of(w)
    out = out or alloc_outputs(w, dev["Q"].device)
    _lib.hsa_forward_heads(shape, dev.get("W"), summary_start_block, dev["Q"], dev["K"], dev["V"], out["LK"],
                           out["blk"] if keep_lists else None, out["O"], out["lse"], workspace, seq_lens=seq_lens)
    return out


def to_host(out: dict) -> dict:
    res = {}
    for key, t in out.items():
        if t.dtype == torch.bfloat16:
            res[key] = t.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            res[key] = t.cpu().numpy()
    return res
