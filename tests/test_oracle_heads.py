"""Pins of the oracle's per-head selection (chunk scores from the attention
queries against landmarks of the attention keys, per kv head).

Checked against exact rational arithmetic on float-valued bf16 keys, an
enumeration of the kept chunk sets with exact scores for every head (which
pins the query-head to kv-head mapping), dense causal attention from torch
when every chunk is kept, and the reduction to the shared-indexer path with
one head.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact_bf16 import bf16_rne_of_fraction
from oracle import hisa_oracle as orc


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def seq_of(rng, L, Hq, Hkv, d, nq=1, scale=1.0):
    return {"Q": rand_bf16(rng, (1, nq, Hq, d), scale), "K": rand_bf16(rng, (1, L, Hkv, d), scale),
            "V": rand_bf16(rng, (1, L, Hkv, d))}


@pytest.mark.parametrize("L,B,nL", [(37, 8, 1), (64, 16, 2), (50, 16, 1)])
def test_head_landmarks_exact_on_float_keys(L, B, nL):
    rng = np.random.default_rng(10 * L + B + nL)
    Hkv, d = 2, 6
    K = rand_bf16(rng, (L, Hkv, d))
    W = None if nL == 1 else rng.integers(0, 2, size=(nL, B)).astype(np.int8)
    LK = orc.head_landmarks(K, B, W)
    nb = -(-L // B)
    assert LK.shape == (nb, nL, Hkv, d)
    Kf = orc.bf16_to_f64(K)
    for j in range(nb):
        for l in range(nL):
            for g in range(Hkv):
                for e in range(d):
                    tot = sum((Fraction(float(Kf[r, g, e])) * (1 if W is None else int(W[l, r - j * B]))
                               for r in range(j * B, min(L, j * B + B))), Fraction(0))
                    assert LK[j, l, g, e] == bf16_rne_of_fraction(tot / B), (j, l, g, e)


def _certified(ids, score, count):
    good = []
    for sub in itertools.combinations(ids, count):
        rest = [j for j in ids if j not in sub]
        if all(score[a] > score[b] or (score[a] == score[b] and a < b) for a in sub for b in rest):
            good.append(sorted(sub))
    assert len(good) == 1
    return good[0]


@pytest.mark.parametrize("seed", range(12))
def test_per_head_selection_brute_force(seed):
    # every head's kept chunks by enumeration with exact scores; the kv head
    # of query head h is h // (Hq / Hkv) (a wrong mapping, e.g. h % Hkv,
    # reads another head's landmarks and fails here)
    rng = np.random.default_rng(6000 + seed)
    B, d, Hq, Hkv = int(rng.choice([2, 4])), 4, 4, 2
    L = int(rng.integers(4 * B, 14 * B))
    seq = seq_of(rng, L, Hq, Hkv, d)
    LK = orc.head_landmarks(seq["K"][0], B)
    LKf = orc.bf16_to_f64(LK)
    Qf = orc.bf16_to_f64(seq["Q"][0, 0])
    for _ in range(3):
        t = int(rng.integers(0, L))
        m = int(rng.integers(2, 6))
        got = orc.forward_query_heads(seq, 0, 0, t, B, m, 0.5, LK, attention=False)["blk"]
        c = t // B
        for h in range(Hq):
            g = h // (Hq // Hkv)
            kept = [int(x) for x in got[h] if x >= 0]
            if c + 1 <= m:
                assert kept == list(range(c + 1))
                continue
            sc = {j: sum(Fraction(float(LKf[j, 0, g, e])) * Fraction(float(Qf[h, e])) for e in range(d))
                  for j in range(c + 1)}
            assert kept == [0] + _certified(list(range(1, c)), sc, m - 2) + [c], (h, t, m)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (6, 1)])
def test_every_chunk_kept_is_dense_attention(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    L, B, d, nq = 40, 8, 16, 40
    seq = seq_of(rng, L, Hq, Hkv, d, nq=nq)
    LK = orc.head_landmarks(seq["K"][0], B)
    scale = 0.25
    q = torch.tensor(orc.bf16_to_f64(seq["Q"][0])).permute(1, 0, 2)[None]
    k = torch.tensor(orc.bf16_to_f64(seq["K"][0])).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    v = torch.tensor(orc.bf16_to_f64(seq["V"][0])).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)[0].permute(1, 0, 2)
    for i in range(nq):
        r = orc.forward_query_heads(seq, 0, i, i, B, L // B, scale, LK)
        assert np.abs(r["O"] - ref[i].numpy()).max() <= 1e-12


def test_one_head_reduces_to_the_shared_indexer_path():
    # Hq = Hkv = 1 with qI := Q and kI := K and k = m*B (every candidate token
    # kept): the same block lists, O and lse as forward_query
    rng = np.random.default_rng(77)
    L, B, d, m = 300, 16, 8, 5
    seq = seq_of(rng, L, 1, 1, d, nq=3)
    LK = orc.head_landmarks(seq["K"][0], B)
    shared = {"qI": seq["Q"][:, :, 0], "kI": seq["K"][:, :, 0], "Q": seq["Q"], "K": seq["K"], "V": seq["V"]}
    S = orc.block_summary(shared["kI"][0], B)
    assert np.array_equal(S, LK[:, :, 0])
    for i, t in enumerate([L - 3, L - 2, L - 1]):
        a = orc.forward_query_heads(seq, 0, i, t, B, m, 0.3, LK)
        b = orc.forward_query(shared, 0, i, t, B, m, m * B, 0.3, S_bits=S)
        assert np.array_equal(a["blk"][0], b["blk"])
        assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])


def test_heads_select_differently():
    # the point of per-head selection: heads of one kv group rank chunks by
    # their own queries; a chunk whose keys align with head 1 only is kept
    # by head 1 and not by head 0
    rng = np.random.default_rng(5)
    L, B, d = 256, 16, 32
    seq = seq_of(rng, L, 2, 1, d, scale=0.1)
    Q = orc.bf16_to_f64(seq["Q"][0, 0])
    Q[0] = 0.0
    Q[0, 0] = 1.0                       # head 0 looks along e_0
    Q[1] = 0.0
    Q[1, 1] = 1.0                       # head 1 looks along e_1
    seq["Q"][0, 0] = orc.f64_to_bf16_rne(Q)
    K = orc.bf16_to_f64(seq["K"][0])
    K[5 * B:6 * B, 0, 1] = 4.0          # chunk 5 aligns with head 1
    K[9 * B:10 * B, 0, 0] = 4.0         # chunk 9 aligns with head 0
    seq["K"][0] = orc.f64_to_bf16_rne(K)
    LK = orc.head_landmarks(seq["K"][0], B)
    blk = orc.forward_query_heads(seq, 0, 0, L - 1, B, 3, 0.2, LK, attention=False)["blk"]
    assert list(blk[0]) == [0, 9, 15] and list(blk[1]) == [0, 5, 15]
