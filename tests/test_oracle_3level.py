"""Pins of the oracle's three-level selection (super-blocks -> blocks -> tokens).

The super-block summary is checked against exact rational arithmetic with a
round-to-nearest-even written here from its definition; the selection is
checked against its reductions to the two-level selection (every super-block
kept; super-blocks of one block) and against brute-force enumeration of the
kept sets at both levels with exact scores.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import hisa_oracle as orc
from hierarchical_index_sparse_amd import datagen
from exact_bf16 import bf16_rne_of_fraction as _bf16_rne_of_fraction


def bits_of_ints(a):
    return datagen.int_to_bf16_bits(np.asarray(a))


def test_fraction_rounding_helper():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even neighbour 1
    assert _bf16_rne_of_fraction(Fraction(1) + Fraction(1, 256)) == 0x3F80
    assert _bf16_rne_of_fraction(Fraction(1) + Fraction(3, 256)) == 0x3F82
    assert _bf16_rne_of_fraction(Fraction(-255, 1)) == 0xC37F  # 8 significant bits: exact
    assert _bf16_rne_of_fraction(Fraction(-511, 1)) == 0xC400  # tie between 510 and 512
    assert _bf16_rne_of_fraction(Fraction(257, 1)) == 0x4380
    assert _bf16_rne_of_fraction(Fraction(259, 1)) == 0x4382


@pytest.mark.parametrize("L,B,G,nL", [(37, 4, 2, 1), (100, 4, 4, 2), (64, 8, 8, 1), (9, 2, 4, 1), (130, 1, 16, 3)])
def test_super_summary_exact_fractions(L, B, G, nL):
    rng = np.random.default_rng(L + 10 * B + 100 * G + nL)
    d = 5
    ints = rng.integers(-8, 9, size=(L, d))
    W = None if nL == 1 else rng.integers(0, 2, size=(nL, B)).astype(np.int8)
    S = orc.block_summary(bits_of_ints(ints), B, W)
    S2 = orc.super_summary(S, G)
    nb = S.shape[0]
    nsb = -(-nb // G)
    assert S2.shape == (nsb, nL, d)
    Sf = orc.bf16_to_f64(S)
    for J in range(nsb):
        for l in range(nL):
            for e in range(d):
                tot = sum((Fraction(float(Sf[j, l, e])) for j in range(J * G, min(nb, J * G + G))), Fraction(0))
                assert S2[J, l, e] == _bf16_rne_of_fraction(tot / G), (J, l, e)


def test_super_summary_rounds_once():
    # summaries 1 + 2^-7 and 1: their mean 1 + 2^-8 is a tie, rounded to the
    # even neighbour 1.0; two equal summaries average to themselves
    one, up = 0x3F80, 0x3F81
    S = np.array([up, one, up, up], np.uint16).reshape(4, 1, 1)
    S2 = orc.super_summary(S, 2)
    assert S2[0, 0, 0] == 0x3F80 and S2[1, 0, 0] == 0x3F81
    # 256, 1, 1, 0: the exact mean 64.5 is a bf16 value; a sum rounded to
    # bf16 after each addition would lose both ones (256 + 1 ties to 256)
    S = np.array([0x4380, one, one, 0], np.uint16).reshape(4, 1, 1)
    assert orc.super_summary(S, 4)[0, 0, 0] == 0x4281
    # a missing block past the end counts as zero: (2 + 0 + 0 + 0) / 4
    S = np.array([0x4000], np.uint16).reshape(1, 1, 1)
    assert orc.super_summary(S, 4)[0, 0, 0] == 0x3F00


@pytest.mark.parametrize("seed", range(16))
def test_three_level_reduces_when_every_super_block_is_kept(seed):
    # m2 at least the number of causal super-blocks: level 1 keeps them all,
    # so the block list must be the two-level one
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([2, 4, 8]))
    L = int(rng.integers(B, 160))
    d = 4
    kb = bits_of_ints(rng.integers(-2, 3, size=(L, d)))
    S = orc.block_summary(kb, B)
    S2 = orc.super_summary(S, G)
    for _ in range(6):
        t = int(rng.integers(0, L))
        m = int(rng.integers(2, 9))
        C = t // (B * G)
        m2 = max(2, C + 1 + int(rng.integers(0, 3)))
        qb = bits_of_ints(rng.integers(-2, 3, size=d))
        got = orc.select_blocks_3level(qb, S, S2, t, B, G, m2, m)
        assert np.array_equal(got, orc.select_blocks(qb, S, t, B, m)), (t, m, m2)


@pytest.mark.parametrize("seed", range(16))
def test_three_level_with_single_block_groups_is_two_level(seed):
    # G = 1, m2 = m: the super-blocks are the blocks, level 1 keeps exactly the
    # two-level list and level 2 keeps all of it
    rng = np.random.default_rng(4000 + seed)
    B = int(rng.choice([1, 2, 4, 8]))
    L = int(rng.integers(B, 200))
    d = 5
    kb = bits_of_ints(rng.integers(-3, 4, size=(L, d)))
    S = orc.block_summary(kb, B)
    S2 = orc.super_summary(S, 1)
    assert np.array_equal(S2, S)
    for _ in range(6):
        t = int(rng.integers(0, L))
        m = int(rng.integers(2, 7))
        qb = bits_of_ints(rng.integers(-3, 4, size=d))
        got = orc.select_blocks_3level(qb, S, S2, t, B, 1, m, m)
        assert np.array_equal(got, orc.select_blocks(qb, S, t, B, m))


def _certified_subset(ids, score, count):
    """The one subset of `count` ids such that every kept id beats every dropped
    id under (score descending, id ascending), found by enumeration."""
    good = []
    for sub in itertools.combinations(ids, count):
        rest = [j for j in ids if j not in sub]
        if all(score[a] > score[b] or (score[a] == score[b] and a < b) for a in sub for b in rest):
            good.append(sorted(sub))
    assert len(good) == 1
    return good[0]


@pytest.mark.parametrize("seed", range(30))
def test_three_level_brute_force(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([2, 3, 4]))
    nL = int(rng.choice([1, 2]))
    L = int(rng.integers(B * G, 120))
    d = 3
    kI = rng.integers(-2, 3, size=(L, d))
    W = None if nL == 1 else rng.integers(0, 2, size=(nL, B)).astype(np.int8)
    S = orc.block_summary(bits_of_ints(kI), B, W)
    S2 = orc.super_summary(S, G)
    Sf, S2f = orc.bf16_to_f64(S), orc.bf16_to_f64(S2)

    def exact_score(Xf, j, qi):
        return max(sum(Fraction(float(Xf[j, l, e])) * int(qi[e]) for e in range(d)) for l in range(Xf.shape[1]))

    for _ in range(4):
        t = int(rng.integers(0, L))
        m2 = int(rng.integers(2, 5))
        m = int(rng.integers(2, 7))
        qi = rng.integers(-2, 3, size=d)
        got = orc.select_blocks_3level(bits_of_ints(qi), S, S2, t, B, G, m2, m)
        c, C = t // B, t // (B * G)
        # level 1 by enumeration
        if C + 1 <= m2:
            sup = list(range(C + 1))
        else:
            s2 = {J: exact_score(S2f, J, qi) for J in range(C + 1)}
            sup = [0] + _certified_subset(list(range(1, C)), s2, m2 - 2) + [C]
        cand = sorted(j for J in sup for j in range(J * G, J * G + G) if j <= c)
        assert 0 in cand and c in cand
        if len(cand) <= m:
            want = cand
        else:
            s1 = {j: exact_score(Sf, j, qi) for j in cand}
            mid = [j for j in cand if j not in (0, c)]
            want = [0] + _certified_subset(mid, s1, m - 2) + [c]
        assert [int(x) for x in got if x >= 0] == sorted(want), (t, m2, m)
        assert all(x == -1 for x in got[len(want):]) and got.shape == (m,)
