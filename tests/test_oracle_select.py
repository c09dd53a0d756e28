"""Pins for the oracle's group-limited selection (page section "Mixture of
Experts": sigmoid scores, groups ranked by the sum of their two best scores,
best groups kept, top experts chosen inside them, weights normalised and
scaled).

The oracle sorts; these checks use independent formulations:
  * brute force over every subset, with the defining dominance condition
    (every chosen item beats every unchosen one, ties to the lower index);
  * for tie-free scores, the max-sum characterisation of a top-m set;
  * heapq.nlargest when every group is kept (plain top-k);
  * hand-worked examples in tests/golden/hand_selection.json.
"""
import heapq
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import group_limited_topk, group_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_selection.json")


def beats(a_val, a_idx, b_val, b_idx):
    """a ranks above b: larger value, or equal value and lower index."""
    return a_val > b_val or (a_val == b_val and a_idx < b_idx)


def brute_force_top(values, m):
    """The unique m-subset dominating its complement, by enumeration."""
    n = len(values)
    found = []
    for sub in itertools.combinations(range(n), m):
        inside = set(sub)
        ok = all(beats(values[a], a, values[b], b)
                 for a in inside for b in range(n) if b not in inside)
        if ok:
            found.append(sub)
    assert len(found) == 1, found
    return set(found[0])


def brute_force_select(s_row, groups, topk_groups, k):
    E = len(s_row)
    gsz = E // groups
    gsc = []
    for g in range(groups):
        mem = s_row[g * gsz:(g + 1) * gsz]
        gsc.append(max(mem[i] + mem[j] for i in range(gsz) for j in range(gsz) if i != j))
    kept = brute_force_top(gsc, topk_groups)
    elig = [e for e in range(E) if e // gsz in kept]
    vals = [s_row[e] for e in elig]
    chosen_local = brute_force_top(vals, k)
    return {elig[i] for i in chosen_local}, kept


SHAPES = [  # (E, groups, topk_groups, k)
    (16, 4, 2, 3),
    (32, 8, 3, 4),
    (64, 8, 4, 8),
    (12, 3, 2, 5),
]


@pytest.mark.parametrize("E,G,KG,k", SHAPES)
def test_brute_force_random(E, G, KG, k):
    rng = np.random.default_rng(1000 + E + G + KG + k)
    s = rng.random((24, E))
    ids, w, m_g, m_e = group_limited_topk(s, G, KG, k, 2.5)
    for t in range(s.shape[0]):
        # brute force over k-subsets of the eligible experts is expensive for
        # (64, 8, 4, 8) (C(32, 8) = 10.5M); restrict the exhaustive level to
        # smaller cases and use the max-sum characterisation otherwise.
        if math.comb(KG * (E // G), k) <= 20000:
            exp_ids, _ = brute_force_select(list(s[t]), G, KG, k)
            assert set(ids[t].tolist()) == exp_ids
        else:
            gsz = E // G
            gsc = [max(a + b for a, b in itertools.combinations(s[t, g*gsz:(g+1)*gsz], 2))
                   for g in range(G)]
            best = max(itertools.combinations(range(G), KG), key=lambda c: sum(gsc[i] for i in c))
            elig = [e for e in range(E) if e // gsz in best]
            # top-k by value of a tie-free set = the k-subset of maximum sum;
            # the maximum-sum k-subset of a set is its k largest: verify by
            # checking that no swap of a chosen and an unchosen expert increases the sum
            chosen = set(ids[t].tolist())
            assert chosen <= set(elig)
            for a in chosen:
                for b in set(elig) - chosen:
                    assert s[t, a] > s[t, b]
        # ids are distinct and ordered by decreasing score
        assert len(set(ids[t].tolist())) == k
        sc = s[t, ids[t]]
        assert np.all(np.diff(sc) <= 0)


@pytest.mark.parametrize("E,G,KG,k", [(16, 4, 2, 3), (32, 8, 3, 4)])
def test_brute_force_with_ties(E, G, KG, k):
    """Scores on a coarse dyadic grid so exact ties are frequent."""
    rng = np.random.default_rng(77 + E)
    s = rng.integers(1, 6, size=(40, E)).astype(np.float64) / 8.0
    ids, w, m_g, m_e = group_limited_topk(s, G, KG, k, 2.5)
    for t in range(s.shape[0]):
        exp_ids, _ = brute_force_select(list(s[t]), G, KG, k)
        assert set(ids[t].tolist()) == exp_ids


def test_beam_group_level_enumerated():
    """Beam shape (256 experts, 8 groups of 32, keep 4, top-8): all C(8,4)=70
    group subsets enumerated; expert level checked by dominance."""
    rng = np.random.default_rng(5)
    s = 1.0 / (1.0 + np.exp(-rng.normal(0, 1.43, size=(64, 256))))
    ids, w, m_g, m_e = group_limited_topk(s, 8, 4, 8, 2.5)
    gs = group_scores(s, 8)
    for t in range(s.shape[0]):
        gsc = [max(a + b for a, b in itertools.combinations(s[t, g*32:(g+1)*32], 2)) for g in range(8)]
        assert np.allclose(gsc, gs[t], rtol=0, atol=1e-15)
        kept = brute_force_top(gsc, 4)
        elig = [e for e in range(256) if e // 32 in kept]
        chosen = set(ids[t].tolist())
        assert chosen <= set(elig)
        for a in chosen:
            for b in set(elig) - chosen:
                assert beats(s[t, a], a, s[t, b], b)
        assert math.isclose(w[t].sum(), 2.5, rel_tol=0, abs_tol=1e-12)


def test_all_groups_kept_is_plain_topk():
    """topk_groups == groups reduces to ordinary top-k (heapq.nlargest)."""
    rng = np.random.default_rng(9)
    s = rng.random((50, 256))
    ids, w, _, m_e = group_limited_topk(s, 8, 8, 8, 1.0)
    for t in range(s.shape[0]):
        ref = heapq.nlargest(8, range(256), key=lambda e: (s[t, e], -e))
        assert ids[t].tolist() == ref


def test_hand_examples():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        s = np.array([c["scores"]], dtype=np.float64)
        ids, w, m_g, m_e = group_limited_topk(s, c["groups"], c["topk_groups"], c["k"], c["scale"])
        assert ids[0].tolist() == c["ids"], c["name"]
        exp_w = np.array(c["weights_num"]) / c["weights_den"]
        np.testing.assert_allclose(w[0], exp_w, rtol=1e-13, err_msg=c["name"])
        assert math.isclose(m_g[0], c["group_margin"], abs_tol=1e-12), c["name"]
        em = c["expert_margin"]
        if em == "inf":
            assert math.isinf(m_e[0])
        else:
            assert math.isclose(m_e[0], em, abs_tol=1e-12), c["name"]


def test_group_scores_pairwise():
    rng = np.random.default_rng(3)
    s = rng.random((10, 64))
    gs = group_scores(s, 8)
    for t in range(10):
        for g in range(8):
            m = s[t, g*8:(g+1)*8]
            assert gs[t, g] == max(m[i] + m[j] for i in range(8) for j in range(i + 1, 8))


def test_margin_detects_ties():
    s = np.full((1, 16), 0.25)
    _, _, m_g, m_e = group_limited_topk(s, 4, 2, 3, 2.5)
    assert m_g[0] == 0.0 and m_e[0] == 0.0


def test_k1_weight_is_scale():
    rng = np.random.default_rng(2)
    s = rng.random((20, 64))
    _, w, _, _ = group_limited_topk(s, 4, 2, 1, 2.5)
    assert np.all(w[:, 0] == 2.5)
