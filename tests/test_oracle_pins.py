"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something other than itself: the
hand-worked example, the definition of round-to-nearest-even, brute-force
enumeration, an independent rank-count definition of top-k, closed forms,
and torch's dense attention on the CPU in float64.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import hisa_oracle as orc
from hierarchical_index_sparse_amd import datagen
from hierarchical_index_sparse_amd.workloads import Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_of_ints(a):
    return datagen.int_to_bf16_bits(np.asarray(a))


def torch_bf16_bits(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- bf16 ----


def test_bf16_rne_table():
    vals, want = [], []
    for line in open(os.path.join(GOLDEN, "bf16_rne.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v, h = line.split()
        vals.append(float(v))
        want.append(int(h, 16))
    got = orc.f64_to_bf16_rne(np.array(vals))
    assert list(got) == want
    # decoding the rounded value gives back a value within half an ulp
    dec = orc.bf16_to_f64(got)
    for v, dv in zip(vals, dec):
        if v != 0:
            assert abs(dv - v) <= 2.0 ** (math.floor(math.log2(abs(v))) - 8)


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(1)
    # random fp32 values over many binades, plus exact halfway cases
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-40, 40, 200000))).astype(np.float32)
    base = x.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    x = x[(np.abs(x) >= 2.0 ** -126) & (np.abs(x) < 2.0 ** 127)]
    assert np.array_equal(orc.f64_to_bf16_rne(x.astype(np.float64)), torch_bf16_bits(x))


def test_bf16_decode():
    assert list(orc.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x4480], np.uint16))) == [1.0, -2.0, 0.0, 1024.0]
    v = np.arange(-8, 9)
    assert np.array_equal(orc.bf16_to_f64(bits_of_ints(v)), v.astype(np.float64))


# -------------------------------------------------------- worked example --


def load_worked():
    ex = {"kI": [], "summary": [], "tokens": {}}
    for line in open(os.path.join(GOLDEN, "hisa_worked_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        if f[0] in ("kI", "summary"):
            ex[f[0]].append([int(x) for x in f[1:]])
        elif f[0] == "k":
            ex["tokens"][int(f[1])] = [int(x) for x in f[3:]]
        elif f[0] in ("q", "blocks"):
            ex[f[0]] = [int(x) for x in f[1:]]
        else:
            ex[f[0]] = int(f[1])
    return ex


def test_worked_example():
    ex = load_worked()
    kI = bits_of_ints(ex["kI"])
    q = bits_of_ints(ex["q"])
    S = orc.block_summary(kI, ex["block"])
    assert np.array_equal(orc.bf16_to_f64(S[:, 0]), np.array(ex["summary"], np.float64))
    blk = orc.select_blocks(q, S, ex["t"], ex["block"], ex["m"])
    assert list(blk) == ex["blocks"]
    for k, want in ex["tokens"].items():
        assert list(orc.select_tokens(q, kI, blk, ex["t"], ex["block"], k)) == want


# ------------------------------------------------------------- summary ----


def _exact_bf16_of_fraction(fr: Fraction) -> int:
    # the fractions here have <= 11 significant bits: exact in fp32, so
    # torch's fp32 -> bf16 conversion rounds the exact value
    f = float(fr)
    assert Fraction(f) == fr
    return int(torch_bf16_bits([f])[0])


@pytest.mark.parametrize("L,B,nL", [(37, 8, 1), (64, 16, 4), (50, 16, 2), (8, 8, 1)])
def test_summary_matches_exact_fractions(L, B, nL):
    rng = np.random.default_rng(L * 100 + B + nL)
    d = 5
    ints = rng.integers(-8, 9, size=(L, d))
    W = None if nL == 1 else rng.integers(0, 2, size=(nL, B)).astype(np.int8)
    S = orc.block_summary(bits_of_ints(ints), B, W)
    nb = (L + B - 1) // B
    assert S.shape == (nb, nL, d)
    for j in range(nb):
        for l in range(nL):
            for c in range(d):
                tot = sum(int(ints[r, c]) * (1 if W is None else int(W[l, r - j * B]))
                          for r in range(j * B, min(L, j * B + B)))
                assert S[j, l, c] == _exact_bf16_of_fraction(Fraction(tot, B))


def test_landmark_all_ones_equals_mean():
    rng = np.random.default_rng(7)
    kI = bits_of_ints(rng.integers(-8, 9, size=(300, 16)))
    mean = orc.block_summary(kI, 32)
    ones = orc.block_summary(kI, 32, np.ones((1, 32), np.int8))
    assert np.array_equal(mean, ones)


def test_summary_score_closed_form_without_rounding():
    # When no bf16 rounding happens (|block sum| <= 256 for B = 128, since
    # bf16 holds 8 significant bits), B * (q . mean) equals the sum over the
    # block of q . kI[s]: the mean-of-token-scores identity.
    rng = np.random.default_rng(3)
    B, d, nb = 128, 16, 6
    kI = rng.integers(-2, 3, size=(nb * B, d))
    kI[:, :] = np.clip(kI, -2, 2)
    assert np.abs(kI.reshape(nb, B, d).sum(1)).max() <= 256
    q = rng.integers(-8, 9, size=d)
    S = orc.block_summary(bits_of_ints(kI), B)
    sc = orc.block_scores(bits_of_ints(q), S, nb - 1)
    direct = (kI.reshape(nb, B, d) @ q).sum(1)
    assert np.array_equal(sc * B, direct.astype(np.float64))


# ------------------------------------------------------- block select -----


def _rank_select(scores, ids, count):
    """Independent top-count: an id is kept iff fewer than `count` ids beat it."""
    keep = []
    for a, sa in zip(ids, scores):
        beaten = sum(1 for b, sb in zip(ids, scores) if sb > sa or (sb == sa and b < a))
        if beaten < count:
            keep.append(a)
    return sorted(keep)


def _tiny_case(seed, L, B, d, nL=1, vr=2):
    rng = np.random.default_rng(seed)
    kI = rng.integers(-vr, vr + 1, size=(L, d))
    W = None if nL == 1 else rng.integers(0, 2, size=(nL, B)).astype(np.int8)
    return rng, kI, W


@pytest.mark.parametrize("seed", range(40))
def test_block_select_brute_force(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 4, 8]))
    L = int(rng.integers(B, 96))
    d = 4
    nL = int(rng.choice([1, 2]))
    _, kI, W = _tiny_case(seed, L, B, d, nL)
    kb = bits_of_ints(kI)
    S = orc.block_summary(kb, B, W)
    Sf = orc.bf16_to_f64(S)
    for _ in range(4):
        m = int(rng.integers(2, 6))
        t = int(rng.integers(0, L))
        qi = rng.integers(-2, 3, size=d)
        blk = orc.select_blocks(bits_of_ints(qi), S, t, B, m)
        c = t // B
        assert blk.shape == (m,)
        kept = [int(x) for x in blk if x >= 0]
        assert kept == sorted(kept)
        assert all(x == -1 for x in blk[len(kept):])
        if c + 1 <= m:
            assert kept == list(range(c + 1))
            continue
        assert kept[0] == 0 and kept[-1] == c and len(kept) == m
        # exact block scores with Fractions
        sc = [max(sum(Fraction(float(Sf[j, l, e])) * int(qi[e]) for e in range(d)) for l in range(Sf.shape[1]))
              for j in range(c + 1)]
        mid = list(range(1, c))
        # brute force: exactly one (m-2)-subset satisfies the certificate
        # "every kept block beats every dropped block under (score desc, id asc)"
        good = []
        for sub in itertools.combinations(mid, m - 2):
            rest = [j for j in mid if j not in sub]
            if all(sc[a] > sc[b] or (sc[a] == sc[b] and a < b) for a in sub for b in rest):
                good.append(sorted(sub))
        assert len(good) == 1
        assert kept[1:-1] == good[0]
        assert kept[1:-1] == _rank_select([sc[j] for j in mid], mid, m - 2)


# ------------------------------------------------------- token select -----


@pytest.mark.parametrize("seed", range(40))
def test_token_select_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.choice([1, 2, 4, 8]))
    L = int(rng.integers(B, 96))
    d = 4
    _, kI, _ = _tiny_case(1000 + seed, L, B, d)
    kb = bits_of_ints(kI)
    S = orc.block_summary(kb, B)
    for _ in range(4):
        m = int(rng.integers(2, 6))
        k = int(rng.integers(1, 41))
        t = int(rng.integers(0, L))
        qi = rng.integers(-2, 3, size=d)
        qb = bits_of_ints(qi)
        blk = orc.select_blocks(qb, S, t, B, m)
        tok = orc.select_tokens(qb, kb, blk, t, B, k)
        cand = [s for s in range(t + 1) if s // B in set(int(x) for x in blk if x >= 0)]
        kept = [int(x) for x in tok if x >= 0]
        assert all(x == -1 for x in tok[len(kept):])
        if len(cand) <= k:
            assert kept == cand
            continue
        assert len(kept) == k
        sc = [int(np.dot(kI[s], qi)) for s in cand]
        assert kept == _rank_select(sc, cand, k)
        if math.comb(len(cand), k) <= 3000:
            good = []
            for sub in itertools.combinations(range(len(cand)), k):
                rest = [i for i in range(len(cand)) if i not in sub]
                if all(sc[a] > sc[b] or (sc[a] == sc[b] and a < b) for a in sub for b in rest):
                    good.append(sorted(cand[i] for i in sub))
            assert good == [kept]


@pytest.mark.parametrize("seed", range(12))
def test_degrades_to_flat_indexer(seed):
    # HISA page: on short inputs the hierarchical indexer gives exactly the
    # original flat indexer's selection.  With m >= number of causal blocks
    # every block is kept, so the token set must equal the flat top-k, here
    # defined independently by rank counting.
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.choice([2, 4, 8, 16]))
    L = int(rng.integers(B, 200))
    d = 6
    kI = rng.integers(-3, 4, size=(L, d))
    kb = bits_of_ints(kI)
    S = orc.block_summary(kb, B)
    nb = (L + B - 1) // B
    for _ in range(5):
        t = int(rng.integers(0, L))
        k = int(rng.integers(1, 60))
        qi = rng.integers(-3, 4, size=d)
        qb = bits_of_ints(qi)
        blk = orc.select_blocks(qb, S, t, B, max(2, nb))
        tok = orc.select_tokens(qb, kb, blk, t, B, k)
        flat = orc.flat_topk(qb, kb, t, k)
        assert np.array_equal(tok, flat)
        kept = [int(x) for x in tok if x >= 0]
        sc = [int(np.dot(kI[s], qi)) for s in range(t + 1)]
        assert kept == _rank_select(sc, list(range(t + 1)), k)


def test_work_count_bound():
    # HISA page, complexity: per query at most ceil((t+1)/B) summaries plus
    # m*B tokens are scored (O(L^2/B + L*m*B) per layer).
    for B, m, k in [(64, 8, 256), (128, 64, 2048), (128, 128, 4096), (16, 3, 5)]:
        for t in list(range(0, 3 * B * m, 7)) + [65535, 524287]:
            n = orc.scored_items(t, B, m, k)
            assert n <= -(-(t + 1) // B) + m * B


def test_scored_items_counts_what_the_selects_rank(monkeypatch):
    # scored_items is a closed form: check it against what select_blocks and
    # select_tokens actually rank (the sizes they hand to top_by_score) on
    # small random inputs, over every query position of several shapes, so an
    # off-by-one block or token in the formula fails
    sizes = []
    real = orc.top_by_score

    def counting(scores, ids, count):
        sizes.append(len(scores))
        return real(scores, ids, count)

    monkeypatch.setattr(orc, "top_by_score", counting)
    rng = np.random.default_rng(11)
    for B, m, k, L in [(8, 2, 5, 100), (8, 3, 20, 150), (16, 4, 40, 300), (4, 6, 7, 97), (16, 5, 100, 333)]:
        d = 4
        kI = rng.integers(-2, 3, size=(L, d))
        kb = bits_of_ints(kI)
        S = orc.block_summary(kb, B)
        for t in range(L):
            qb = bits_of_ints(rng.integers(-2, 3, size=d))
            sizes.clear()
            blk = orc.select_blocks(qb, S, t, B, m)
            orc.select_tokens(qb, kb, blk, t, B, k)
            assert sum(sizes) == orc.scored_items(t, B, m, k), (B, m, k, t, sizes)


def test_prefill_64k_work_totals():
    # the algorithmic totals the roofline figures of the 64K prefill rest on
    # (L = n_q = 65536, B = 128, m = 64, k = 2048): summed over every query
    # from the oracle's own candidate enumeration and its scored_items
    B, m, k, L = 128, 64, 2048, 65536
    cand_total = kept_total = scored_total = 0
    for t in range(L):
        c = t // B
        blk = np.arange(c + 1) if c + 1 <= m else np.concatenate([np.arange(m - 1), [c]])
        n = orc.candidate_tokens(blk, t, B).size
        cand_total += n
        kept_total += min(n, k)
        scored_total += orc.scored_items(t, B, m, k)
    assert kept_total == 132_121_600           # kept (query, token) pairs
    assert cand_total == 499_679_232           # candidate tokens (499.7 M)
    # scored = causal blocks beyond the forced ones + candidates of the
    # queries with more than k of them
    assert scored_total == 16_429_056 + 497_581_056


# ------------------------------------------------------------ attention ---


def _rand_bf16(rng, shape):
    return datagen.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (16, 1), (8, 8)])
def test_dense_equivalence_sdpa(Hq, Hkv):
    # When k covers every causal token and m every causal block, the output is
    # dense causal softmax attention: compare with torch's SDPA (float64, CPU).
    rng = np.random.default_rng(Hq * 10 + Hkv)
    L, d, B = 40, 128, 4
    Q = _rand_bf16(rng, (L, Hq, d))
    K = _rand_bf16(rng, (L, Hkv, d))
    V = _rand_bf16(rng, (L, Hkv, d))
    kI = bits_of_ints(rng.integers(-8, 9, size=(L, 8)))
    qI = bits_of_ints(rng.integers(-8, 9, size=(L, 8)))
    scale = 1 / math.sqrt(d)
    seq = {"qI": qI[None], "kI": kI[None], "Q": Q[None], "K": K[None], "V": V[None]}
    q = torch.tensor(orc.bf16_to_f64(Q)).permute(1, 0, 2)[None]
    kk = torch.tensor(orc.bf16_to_f64(K)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    vv = torch.tensor(orc.bf16_to_f64(V)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True, scale=scale)[0]
    logits = torch.einsum("hqd,hkd->hqk", q[0], kk[0]) * scale
    logits = logits.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    ref_lse = torch.logsumexp(logits, -1)
    for t in range(L):
        r = orc.forward_query(seq, 0, t, t, B, m=L // B + 1, k=L, scale=scale)
        assert list(r["tok"][:t + 1]) == list(range(t + 1))
        np.testing.assert_allclose(r["O"], ref[:, t].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["lse"], ref_lse[:, t].numpy(), rtol=0, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    L, Hq, Hkv, d = 30, 4, 2, 128
    Q = _rand_bf16(rng, (Hq, d))
    K = _rand_bf16(rng, (L, Hkv, d))
    V = _rand_bf16(rng, (L, Hkv, d))
    Vf = orc.bf16_to_f64(V)
    Kf = orc.bf16_to_f64(K)
    # one token: the output is that token's value row, lse its logit
    O, lse = orc.sparse_attention(Q, K, V, np.array([7, -1, -1], np.int32), 0.1)
    for h in range(Hq):
        np.testing.assert_array_equal(O[h], Vf[7, h // 2])
        assert abs(lse[h] - 0.1 * orc.bf16_to_f64(Q)[h] @ Kf[7, h // 2]) < 1e-12
    # zero query: uniform weights -> mean of the kept value rows, lse = log n
    tok = np.array([1, 4, 9, 22], np.int32)
    O, lse = orc.sparse_attention(np.zeros_like(Q), K, V, tok, 0.1)
    for h in range(Hq):
        np.testing.assert_allclose(O[h], Vf[tok, h // 2].mean(0), atol=1e-14)
        assert abs(lse[h] - math.log(4)) < 1e-14
    # two tokens: logistic closed form
    tok = np.array([3, 11], np.int32)
    O, _ = orc.sparse_attention(Q, K, V, tok, 0.3)
    qf = orc.bf16_to_f64(Q)
    for h in range(Hq):
        g = h // 2
        dz = 0.3 * (qf[h] @ Kf[3, g] - qf[h] @ Kf[11, g])
        w = 1 / (1 + math.exp(-dz))
        np.testing.assert_allclose(O[h], w * Vf[3, g] + (1 - w) * Vf[11, g], atol=1e-13)
    # permutation invariance and convex hull
    tok = np.array([0, 5, 6, 13, 29], np.int32)
    O1, l1 = orc.sparse_attention(Q, K, V, tok, 0.2)
    O2, l2 = orc.sparse_attention(Q, K, V, tok[::-1].copy(), 0.2)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    for h in range(Hq):
        rows = Vf[tok, h // 2]
        assert np.all(O1[h] <= rows.max(0) + 1e-12) and np.all(O1[h] >= rows.min(0) - 1e-12)


# ------------------------------------------------------ workload checks ---


def test_forced_blocks_and_needles():
    # Forced first and last blocks (HISA page), and the planted needle blocks
    # of the decode workload are found by the block stage.
    w = Workload(name="mini_decode", batch=3, seq_len=128 * 200, n_q=1, d_index=128, block=128,
                 top_m=16, top_k=512, n_heads_q=2, n_heads_kv=1, needles=4)
    inp = datagen.make_inputs(w, attention=False)
    for b in range(w.batch):
        S = orc.block_summary(inp["kI"][b], w.block)
        t = w.query_pos(0)
        blk = orc.select_blocks(inp["qI"][b, 0], S, t, w.block, w.top_m)
        assert blk[0] == 0 and blk[-1] == t // w.block
        assert set(inp["needles"][b].tolist()) <= set(blk.tolist())


def test_datagen_deterministic_and_shaped():
    w = Workload(name="mini", batch=2, seq_len=300, n_q=5, d_index=16, block=32, top_m=3,
                 top_k=20, n_heads_q=4, n_heads_kv=2, n_landmarks=4)
    a = datagen.make_inputs(w)
    b = datagen.make_inputs(w)
    for key in ("qI", "kI", "Q", "K", "V", "W"):
        assert np.array_equal(a[key], b[key])
    assert a["qI"].shape == (2, 5, 16) and a["kI"].shape == (2, 300, 16)
    assert a["Q"].shape == (2, 5, 4, 128) and a["K"].shape == (2, 300, 2, 128)
    assert a["W"].shape == (4, 32) and set(np.unique(a["W"])) <= {0, 1}
    kv = orc.bf16_to_f64(a["kI"])
    assert kv.min() >= -8 and kv.max() <= 8 and np.all(kv == np.round(kv))
    # noise is bounded by 4 around a per-block centre: within a block the
    # spread of any column is at most 8 (before clipping)
    spread = np.ptp(kv[0, :288].reshape(9, 32, 16), axis=1)
    assert spread.max() <= 8
    c = datagen.make_inputs(w.with_(seed=1))
    assert not np.array_equal(a["kI"], c["kI"])


def test_datagen_matches_stored_hashes():
    # every generated tensor of every named workload (shrunk) hashes as when
    # tests/golden/datagen_sha256.txt was written: inputs are the same on
    # every machine and across library versions
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_datagen_hashes.py")
    spec = importlib.util.spec_from_file_location("make_datagen_hashes", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    stored = [ln.rstrip("\n") for ln in open(mod.OUT) if not ln.startswith("#")]
    fresh = list(mod.lines())
    assert [ln.rsplit(" ", 1)[0] for ln in fresh] == [ln.rsplit(" ", 1)[0] for ln in stored]
    changed = [a for a, b in zip(fresh, stored) if a != b]
    assert not changed, f"generated inputs changed: {changed[:5]}"
