"""Pins of the oracle's histogram (VocabTrim page, Step 1; FR-Spec notes,
key design: corpus token frequencies) against library routines, the page's
own dict semantics, a hand-worked example and the Zipf closed form."""
import collections
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN


def test_hand_worked_stream():
    g = json.load(open(os.path.join(GOLDEN, "hand_select.json")))
    c, inv = oracle.count(g["ids"], g["V"])
    assert c.tolist() == g["counts"]
    assert inv == g["n_invalid"]


def test_matches_bincount_tiny():
    w = synth.WORKLOADS["tiny"]
    ids = synth.make_ids(w)
    c, inv = oracle.count(ids, w.V)
    assert inv == 0
    np.testing.assert_array_equal(c, np.bincount(ids, minlength=w.V))


def test_matches_page_dict_semantics():
    # The page counts with token_counts[id] = token_counts.get(id, 0) + 1.
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 300, size=5000).astype(np.int32)
    d = collections.Counter(ids.tolist())
    c, inv = oracle.count(ids, 300)
    assert inv == 0
    for v in range(300):
        assert c[v] == d.get(v, 0)


@pytest.mark.parametrize("V", [1000, 128256])
def test_invalid_ids_are_tallied_not_counted(V):
    rng = np.random.default_rng(1)
    ids = rng.integers(-50, V + 50, size=20000).astype(np.int32)
    ids[:3] = [np.iinfo(np.int32).min, np.iinfo(np.int32).max, V]
    c, inv = oracle.count(ids, V)
    ok = (ids >= 0) & (ids < V)
    np.testing.assert_array_equal(c, np.bincount(ids[ok], minlength=V))
    assert inv == int((~ok).sum())
    assert int(c.sum()) + inv == ids.size


def test_accumulate_equals_concatenation():
    rng = np.random.default_rng(2)
    V = 777
    a = rng.integers(-3, V, size=4000).astype(np.int32)
    b = rng.integers(0, V + 3, size=6000).astype(np.int32)
    c1, i1 = oracle.count(a, V)
    c2, i2 = oracle.count(b, V, counts=c1, n_invalid=i1)
    c3, i3 = oracle.count(np.concatenate([a, b]), V)
    np.testing.assert_array_equal(c2, c3)
    assert i2 == i3


def test_empty_stream():
    c, inv = oracle.count(np.zeros(0, np.int32), 17)
    assert c.tolist() == [0] * 17 and inv == 0


def _harmonic(n, s):
    r = np.arange(1, n + 1, dtype=np.float64)
    return math.fsum(r ** (-s))


def test_zipf_closed_form_llama_shape():
    # Finite Zipf: E[count of rank r] = n r^-s / H_{V,s}; each count is
    # binomial, so a 6-sigma band holds for every one of the top ranks.
    w = synth.WORKLOADS["llama3_8b"]
    n = 10_000_000
    ids = synth.make_ids(w, n)
    c, inv = oracle.count(ids, w.V)
    assert inv == 0
    perm = synth.permutation(w)
    H = _harmonic(w.V, w.zipf_s)
    for r in (1, 2, 3, 10, 100, 1000):
        p = r ** (-w.zipf_s) / H
        mean, sd = n * p, math.sqrt(n * p * (1 - p))
        assert abs(int(c[perm[r - 1]]) - mean) < 6 * sd, r
    # rank 1 is about 8.1 % of the stream at s = 1, V = 128256
    assert abs(1 / H - 0.08104) < 1e-4
