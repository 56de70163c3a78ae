"""Seeded synthetic inputs, shared by the kernels' tests and the oracle's.

This module only draws random numbers and packs them as bf16 bit patterns
(numpy ``uint16``); it holds none of the method's arithmetic.

Recipe (one numpy PCG64 stream per tensor, sequence and chunk, keyed by
``SeedSequence(seed, spawn_key=(tensor_id, b, chunk))``):

* ``qI``  indexer queries: integers uniform in [-q_range, q_range].
* ``kI``  indexer keys: a per-(sequence, block) integer centre uniform in
  [-centre_range, centre_range], plus per-token integer noise uniform in
  [-noise_range, noise_range], clipped to [-q_range, q_range].  Optional
  needle blocks get the centre ``needle_gain * sign(qI of the sequence's
  first query)`` (sign(0) = +1).
* ``Q, K, V`` attention operands: N(0, 1) in fp32, rounded to bf16.
* ``W``  landmark projection: 0/1 Bernoulli(1/2), int8, shared by all blocks.

Small integers are exact in bf16, so every indexer score is an exact value.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .workloads import Workload

_TID = {"qI": 1, "kI_centre": 2, "kI_noise": 3, "Q": 4, "K": 5, "V": 6, "W": 7,
        "needles": 8, "seq_lens": 9, "head_needles": 10}
_CHUNK = 1 << 22  # elements per independent stream chunk


def _rng(seed: int, tensor: str, *key: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(_TID[tensor],) + key)))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (torch's CPU conversion, round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


_INT_LUT = f32_to_bf16_bits(np.arange(-128, 128, dtype=np.float32))


def int_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bits of small integers (|v| <= 128, all exact in bf16)."""
    v = np.asarray(v)
    assert v.min(initial=0) >= -128 and v.max(initial=0) <= 127
    return _INT_LUT[v.astype(np.int64) + 128]


def _normal_bf16(seed: int, tensor: str, b: int, n: int, pool) -> np.ndarray:
    out = np.empty(n, np.uint16)
    chunks = [(c, min(_CHUNK, n - c * _CHUNK)) for c in range((n + _CHUNK - 1) // _CHUNK)]

    def fill(ci):
        c, cnt = ci
        g = _rng(seed, tensor, b, c)
        out[c * _CHUNK:c * _CHUNK + cnt] = f32_to_bf16_bits(
            g.standard_normal(cnt, dtype=np.float32))

    list(pool.map(fill, chunks))
    return out


def gen_index_queries(w: Workload, q_range: int = 8) -> np.ndarray:
    """qI[b, n_q, d_index] bf16 bits."""
    out = np.empty((w.batch, w.n_q, w.d_index), np.uint16)
    for b in range(w.batch):
        g = _rng(w.seed, "qI", b)
        out[b] = int_to_bf16_bits(g.integers(-q_range, q_range + 1,
                                             size=(w.n_q, w.d_index), dtype=np.int16))
    return out


def gen_index_keys(w: Workload, qI_bits: np.ndarray, q_range: int = 8,
                   centre_range: int = 4, noise_range: int = 4,
                   needle_gain: int = 4) -> tuple[np.ndarray, np.ndarray]:
    """kI[b, L, d_index] bf16 bits and the planted needle blocks [b, needles]."""
    L, B, d = w.seq_len, w.block, w.d_index
    nb = w.n_blocks
    out = np.empty((w.batch, L, d), np.uint16)
    needles = np.zeros((w.batch, w.needles), np.int64)
    rows_per_chunk = max(B, (_CHUNK // d) // B * B)
    with ThreadPoolExecutor(_workers()) as pool:
        for b in range(w.batch):
            centre = _rng(w.seed, "kI_centre", b).integers(
                -centre_range, centre_range + 1, size=(nb, d), dtype=np.int16)
            if w.needles:
                assert nb - 2 >= w.needles
                g = _rng(w.seed, "needles", b)
                needles[b] = np.sort(g.choice(np.arange(1, nb - 1), size=w.needles,
                                              replace=False))
                q = qI_bits[b, 0].astype(np.uint32) << 16
                qf = q.view(np.float32)
                sgn = np.where(qf < 0, -1, 1).astype(np.int16)
                centre[needles[b]] = needle_gain * sgn

            def fill(c, b=b, centre=centre):
                r0 = c * rows_per_chunk
                r1 = min(L, r0 + rows_per_chunk)
                noise = _rng(w.seed, "kI_noise", b, c).integers(
                    -noise_range, noise_range + 1, size=(r1 - r0, d), dtype=np.int16)
                v = np.clip(centre[np.arange(r0, r1) // B] + noise, -q_range, q_range)
                out[b, r0:r1] = int_to_bf16_bits(v)

            list(pool.map(fill, range((L + rows_per_chunk - 1) // rows_per_chunk)))
    return out, needles


def gen_attention_inputs(w: Workload) -> dict[str, np.ndarray]:
    """Q[b, n_q, Hq, d], K and V[b, L, Hkv, d], all bf16 bits."""
    res = {}
    shapes = {"Q": (w.n_q, w.n_heads_q, w.head_dim),
              "K": (w.seq_len, w.n_heads_kv, w.head_dim),
              "V": (w.seq_len, w.n_heads_kv, w.head_dim)}
    with ThreadPoolExecutor(_workers()) as pool:
        for name, shp in shapes.items():
            n = int(np.prod(shp))
            arr = np.empty((w.batch,) + shp, np.uint16)
            for b in range(w.batch):
                arr[b] = _normal_bf16(w.seed, name, b, n, pool).reshape(shp)
            res[name] = arr
    return res


def gen_landmark_projection(w: Workload) -> np.ndarray | None:
    """W[n_landmarks, block] int8 in {0, 1}, or None in mean mode."""
    if w.n_landmarks == 1:
        return None
    g = _rng(w.seed, "W", 0)
    return g.integers(0, 2, size=(w.n_landmarks, w.block), dtype=np.int8)


def gen_seq_lens(w: Workload) -> np.ndarray | None:
    """Current length of each sequence, uniform in [varlen_min, seq_len], for
    workloads of different lengths (decode); None when all are seq_len."""
    if not w.varlen_min:
        return None
    g = _rng(w.seed, "seq_lens", 0)
    return g.integers(w.varlen_min, w.seq_len + 1, size=w.batch).astype(np.int32)


def plant_head_needles(w: Workload, att: dict) -> np.ndarray:
    """Per-head workloads: in every (sequence, kv head g) one chunk j in
    1 .. nb-2 gets keys K + 2 * sign(Q_h) for one query head h of g (the
    last query's), so that head h's score for chunk j stands far above the
    rest.  Modifies att["K"]; returns [b, Hkv, 2] (chunk, head)."""
    nb, B = w.n_blocks, w.block
    qpg = w.n_heads_q // w.n_heads_kv
    assert nb - 2 >= 1
    out = np.zeros((w.batch, w.n_heads_kv, 2), np.int64)
    for b in range(w.batch):
        g_rng = _rng(w.seed, "head_needles", b)
        for g in range(w.n_heads_kv):
            j = int(g_rng.integers(1, nb - 1))
            h = g * qpg + int(g_rng.integers(0, qpg))
            q = (att["Q"][b, -1, h].astype(np.uint32) << 16).view(np.float32)
            rows = slice(j * B, min(w.seq_len, j * B + B))
            k = (att["K"][b, rows, g].astype(np.uint32) << 16).view(np.float32)
            att["K"][b, rows, g] = f32_to_bf16_bits(k + np.where(q < 0, -2.0, 2.0).astype(np.float32))
            out[b, g] = (j, h)
    return out


def make_inputs(w: Workload, attention: bool = True, **kw) -> dict[str, np.ndarray]:
    """All inputs of one workload as host arrays (bf16 as uint16 bits)."""
    if w.per_head:  # no indexer vectors: the selection reads Q and K
        res = {"W": gen_landmark_projection(w), "seq_lens": gen_seq_lens(w)}
        res.update(gen_attention_inputs(w))
        if w.needles:
            res["head_needles"] = plant_head_needles(w, res)
        return res
    q_range = kw.pop("q_range", 8)
    qI = gen_index_queries(w, q_range=q_range)
    kI, needles = gen_index_keys(w, qI, q_range=q_range, **kw)
    res = {"qI": qI, "kI": kI, "needles": needles, "W": gen_landmark_projection(w), "seq_lens": gen_seq_lens(w)}
    if attention:
        res.update(gen_attention_inputs(w))
    return res
