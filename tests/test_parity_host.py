"""Pins of the parity helper that accepts near-tie selections (CPU only).

For a token whose selection margin is below 1e-6 several selections are
correct; tests/parity.py accepts the GPU's if `selection_valid` says it is a
group-limited top-k of the oracle's scores under some resolution of the
near-ties.  These tests pin that helper against the oracle's own selection
rule (page "Willkommen Beam", section "Mixture of Experts"):

  * soundness: for every subset it accepts at delta = 0, a tiny perturbation
    of the scores makes the oracle choose exactly that subset;
  * completeness: every subset the oracle chooses under random tiny
    perturbations of tied scores is accepted;
  * with distinct scores exactly one subset of all C(E, k) is accepted, the
    oracle's;
  * far-from-boundary swaps are rejected; a boundary gap is accepted once
    delta covers it.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from parity import selection_valid

SMALL = dict(E=16, groups=4, topk_groups=2, k=3)


def oracle_ids(s, groups, topk_groups, k):
    ids, _, _, _ = O.group_limited_topk(s[None, :], groups, topk_groups, k, 2.5)
    return frozenset(ids[0].tolist())


def accepted_subsets(s, E, groups, topk_groups, k, delta=0.0):
    return {frozenset(c) for c in itertools.combinations(range(E), k)
            if selection_valid(c, s, groups, topk_groups, k, delta)}


def test_distinct_scores_accept_only_the_oracle_selection():
    rng = np.random.default_rng(1)
    for _ in range(20):
        s = rng.uniform(0.05, 0.95, SMALL["E"])
        acc = accepted_subsets(s, **SMALL)
        assert acc == {oracle_ids(s, SMALL["groups"], SMALL["topk_groups"], SMALL["k"])}


def test_tied_scores_sound_and_complete():
    rng = np.random.default_rng(2)
    E, G, KG, k = SMALL["E"], SMALL["groups"], SMALL["topk_groups"], SMALL["k"]
    gsz = E // G
    for trial in range(25):
        s = rng.choice([0.2, 0.5, 0.7], size=E)          # many exact ties
        acc = accepted_subsets(s, E, G, KG, k)
        assert acc, "the oracle's own selection is always accepted"
        assert oracle_ids(s, G, KG, k) in acc
        # soundness: lift the subset (and its groups) a hair above the ties
        for sub in acc:
            groups = {e // gsz for e in sub}
            chosen = None
            for extra in itertools.combinations([g for g in range(G) if g not in groups],
                                                KG - len(groups)):
                kept = groups | set(extra)
                bump = np.where(np.isin(np.arange(E) // gsz, list(kept)), 0.5, 0.0)
                bump[list(sub)] = 1.0
                if oracle_ids(s + 1e-9 * bump, G, KG, k) == sub:
                    chosen = kept
                    break
            assert chosen is not None, f"trial {trial}: accepted {sorted(sub)} is not achievable"
        # completeness: random tie resolutions land in the accepted set
        for _ in range(200):
            got = oracle_ids(s + 1e-9 * rng.uniform(size=E), G, KG, k)
            assert got in acc, f"trial {trial}: oracle choice {sorted(got)} rejected"


def test_beam_group_shape_oracle_selection_valid():
    rng = np.random.default_rng(3)
    for _ in range(50):
        s = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, 256)))
        ids = oracle_ids(s, 8, 4, 8)
        assert selection_valid(sorted(ids), s, 8, 4, 8, 0.0)


def test_far_swaps_rejected_and_delta_covers_a_gap():
    E, G, KG, k = 256, 8, 4, 8
    rng = np.random.default_rng(4)
    s = rng.uniform(0.1, 0.9, E)
    ids = sorted(oracle_ids(s, G, KG, k))
    gsz = E // G
    gs = np.sort(s.reshape(G, gsz), axis=1)[:, -2:].sum(axis=1)
    kept = set(np.argsort(-gs, kind="stable")[:KG].tolist())
    # an expert of a dropped group in place of the weakest selected one
    weakest = min(ids, key=lambda e: s[e])
    dropped_e = max((e for e in range(E) if e // gsz not in kept), key=lambda e: s[e])
    swap = [e for e in ids if e != weakest] + [dropped_e]
    if (dropped_e // gsz) not in {e // gsz for e in ids}:
        assert not selection_valid(swap, s, G, KG, k, 1e-6)
    # the next eligible expert in place of the weakest: valid exactly when
    # delta covers their score gap
    elig = [e for e in range(E) if e // gsz in kept and e not in ids]
    nxt = max(elig, key=lambda e: s[e])
    swap = [e for e in ids if e != weakest] + [nxt]
    gap = s[weakest] - s[nxt]
    assert gap > 0
    assert not selection_valid(swap, s, G, KG, k, 0.5 * gap)
    assert selection_valid(swap, s, G, KG, k, 1.01 * gap)


@pytest.mark.parametrize("bad", [[0, 1], [0, 0, 1], [0, 1, 99]])
def test_malformed_selections_rejected(bad):
    s = np.linspace(0.1, 0.9, 16)
    assert not selection_valid(bad, s, 4, 2, 3, 1.0)
