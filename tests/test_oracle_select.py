"""Pins of the oracle's vocabulary selection (VocabTrim page, Step 2: top-K
by count, both maps, coverage; FR-Spec notes, key design: top-|V_high| by
frequency) against brute force, invariants, a hand-worked example and the
Zipf closed form for coverage."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN


def brute_rank(c):
    return sorted(range(len(c)), key=lambda v: (-int(c[v]), v))


def check_invariants(c, V_high, t2f, f2t, sel, tot):
    V = c.size
    assert t2f.shape == (V_high,) and f2t.shape == (V,)
    assert t2f.min() >= 0 and t2f.max() < V
    assert np.unique(t2f).size == V_high                  # injective
    ct = c[t2f].astype(np.int64)
    assert np.all(np.diff(ct) <= 0)                        # non-increasing counts
    same = np.diff(ct) == 0
    assert np.all(np.diff(t2f.astype(np.int64))[same] > 0)  # ids ascend in ties
    # f2t is the inverse on kept ids and -1 elsewhere
    np.testing.assert_array_equal(f2t[t2f], np.arange(V_high))
    mask = np.ones(V, bool)
    mask[t2f] = False
    assert np.all(f2t[mask] == -1)
    # cut condition: every dropped id ranks below the last kept one
    last_c, last_id = int(c[t2f[-1]]), int(t2f[-1])
    dropped = np.nonzero(mask)[0]
    dc = c[dropped].astype(np.int64)
    assert np.all((dc < last_c) | ((dc == last_c) & (dropped > last_id)))
    assert sel == int(ct.sum())
    assert tot == int(c.astype(np.int64).sum())


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_select.json")))
    counts = np.array(g["counts"], np.uint32)
    for case in g["cases"]:
        t2f, f2t, sel, tot = oracle.select(counts, case["V_high"])
        assert t2f.tolist() == case["t2f"]
        assert f2t.tolist() == case["f2t"]
        assert (sel, tot) == (case["sel"], case["tot"])
        assert sel * case["coverage_den"] == tot * case["coverage_num"]
    t2f, _, _, _ = oracle.select(counts, g["V"])
    assert t2f.tolist() == g["rank_order"]


def test_brute_force_tiny():
    w = synth.WORKLOADS["tiny"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, f2t, sel, tot = oracle.select(c, w.V_high)
    assert t2f.tolist() == brute_rank(c)[: w.V_high]
    check_invariants(c, w.V_high, t2f, f2t, sel, tot)
    # the cut falls inside a run of tied counts, so the tie rule decides
    last = c[t2f[-1]]
    assert np.sum(c == last) > np.sum(c[t2f] == last)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_brute_force_many_ties(seed):
    rng = np.random.default_rng(seed)
    V = 700
    c = rng.integers(0, 6, size=V).astype(np.uint32)   # heavy ties, zeros
    for V_high in (1, 5, 123, 699, 700):
        t2f, f2t, sel, tot = oracle.select(c, V_high)
        assert t2f.tolist() == brute_rank(c)[:V_high]
        check_invariants(c, V_high, t2f, f2t, sel, tot)


def test_uniform_counts_give_identity():
    c = np.full(500, 7, np.uint32)
    t2f, f2t, sel, tot = oracle.select(c, 500)
    np.testing.assert_array_equal(t2f, np.arange(500))
    np.testing.assert_array_equal(f2t, np.arange(500))
    assert sel == tot == 3500
    t2f, _, _, _ = oracle.select(np.zeros(9, np.uint32), 4)   # all unseen
    assert t2f.tolist() == [0, 1, 2, 3]


def test_full_vocab_is_permutation_and_prefix_property():
    rng = np.random.default_rng(9)
    c = rng.zipf(1.3, size=3000).clip(max=10**6).astype(np.uint32)
    full, f2t_full, sel, tot = oracle.select(c, c.size)
    assert sorted(full.tolist()) == list(range(c.size))
    assert sel == tot
    for V_high in (1, 10, 1000, 2999):
        t2f, _, _, _ = oracle.select(c, V_high)
        np.testing.assert_array_equal(t2f, full[:V_high])


def test_counts_near_uint32_max_and_large_sums():
    c = np.array([2**32 - 1, 5, 2**32 - 1, 2**31], np.uint32)
    t2f, _, sel, tot = oracle.select(c, 3)
    assert t2f.tolist() == [0, 2, 3]
    assert sel == 2 * (2**32 - 1) + 2**31
    assert tot == sel + 5


def _harmonic(n, s):
    return math.fsum(np.arange(1, n + 1, dtype=np.float64) ** (-s))


def _rank_coverage(c, perm, V_high):
    """Coverage of the V_high most probable ranks (not the selected ids)."""
    top = np.arange(V_high) if perm is None else perm[:V_high]
    return c[top].astype(np.int64).sum() / c.astype(np.int64).sum()


@pytest.mark.parametrize("name,n", [("tiny", None), ("llama3_8b", 10_000_000)])
def test_coverage_closed_form(name, n):
    # The kept set maximises the kept count over all V_high-subsets, so its
    # coverage is at least that of the V_high most probable ranks, whose
    # expectation is H_{V_high,s} / H_{V,s} with binomial spread.
    w = synth.WORKLOADS[name]
    ids = synth.make_ids(w, n)
    c, _ = oracle.count(ids, w.V)
    perm = synth.permutation(w)
    t2f, f2t, sel, tot = oracle.select(c, w.V_high)
    check_invariants(c, w.V_high, t2f, f2t, sel, tot)
    cov = sel / tot
    rank_cov = _rank_coverage(c, perm, w.V_high)
    assert cov >= rank_cov
    q = _harmonic(w.V_high, w.zipf_s) / _harmonic(w.V, w.zipf_s)
    sd = math.sqrt(q * (1 - q) / tot)
    assert abs(rank_cov - q) < 6 * sd
    assert cov - q < 0.015
    if name == "llama3_8b":
        assert abs(q - 0.8894) < 1e-4


def test_coverage_inside_pages_guidance():
    # Practical Guidance table: 85-95 % coverage for a 25K-50K vocabulary.
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["coverage_guidance"]
    w = synth.WORKLOADS["llama3_8b"]
    c, _ = oracle.count(synth.make_ids(w, 10_000_000), w.V)
    _, _, sel, tot = oracle.select(c, w.V_high)
    assert g["vocab_low"] <= w.V_high <= g["vocab_high"]
    assert g["low"] <= sel / tot <= g["high"]


def test_rejects_bad_sizes():
    c = np.ones(10, np.uint32)
    with pytest.raises(ValueError):
        oracle.select(c, 11)
    with pytest.raises(ValueError):
        oracle.select(c, 0)
