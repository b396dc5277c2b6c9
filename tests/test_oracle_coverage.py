"""Pins of the oracle's coverage curve (VocabTrim page, Step 2's coverage
for every vocabulary size at once; the guidance table's 85-95 % coverage
threshold; Step 5's share of tokens outside the trimmed vocabulary)."""
import numpy as np
import pytest

import oracle
import synth


def test_hand_example():
    counts = np.array([5, 1, 3, 0], np.uint32)
    order = np.array([0, 2, 1, 3], np.int32)
    cum, tot, vh = oracle.coverage_curve(counts, order, 0.9)
    assert cum.tolist() == [5, 8, 9, 9] and tot == 9 and vh == 3   # 8/9 < 0.9 <= 9/9
    assert oracle.coverage_curve(counts, order, 0.5)[2] == 1        # 5/9 >= 0.5
    assert oracle.coverage_curve(counts, order, 1.0)[2] == 3
    assert oracle.coverage_curve(counts, order, 1.01)[2] == -1      # unreachable
    # a partial ranking: coverage is still relative to every counted token
    cum, tot, vh = oracle.coverage_curve(counts, order[:2], 0.95)
    assert cum.tolist() == [5, 8] and tot == 9 and vh == -1


def test_curve_agrees_with_selection_sums():
    # cum[V_high - 1] is the selection's kept-count sum for every V_high and
    # the last entry its total (the selection is pinned on its own).
    w = synth.WORKLOADS["tiny"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    order, _, _, tot_s = oracle.select(c, w.V)
    cum, tot, _ = oracle.coverage_curve(c, order)
    assert tot == tot_s and int(cum[-1]) == tot
    assert np.all(np.diff(cum.astype(np.int64)) >= 0)
    for vh in (1, 7, 100, 1024, 3000, w.V):
        assert int(cum[vh - 1]) == oracle.select(c, vh)[2]


def test_zipf_closed_form_coverage():
    # finite Zipf(s): expected coverage of the top n ranks = H(n, s) / H(V, s);
    # the empirical top-n draws lucky counts near the cut, so it sits slightly
    # above (0 <= delta <= 1e-2 at 1e5 ids).
    w = synth.WORKLOADS["tiny"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    order, _, _, _ = oracle.select(c, w.V)
    cum, tot, _ = oracle.coverage_curve(c, order)
    r = np.arange(1, w.V + 1, dtype=np.float64)
    H = np.cumsum(r ** -w.zipf_s)
    for n in (64, 256, 1024, 2048):
        delta = cum[n - 1] / tot - H[n - 1] / H[-1]
        assert 0.0 <= delta <= 1e-2, (n, delta)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_threshold_is_the_smallest_prefix(seed):
    rng = np.random.default_rng(seed)
    V = 5000
    c = rng.integers(0, 50, V).astype(np.uint32)
    order = rng.permutation(V).astype(np.int32)
    for thr in rng.uniform(0.0, 1.0, 20):
        cum, tot, vh = oracle.coverage_curve(c, order, thr)
        x = thr * tot
        assert 1 <= vh <= V and cum[vh - 1] >= x
        assert vh == 1 or cum[vh - 2] < x


def test_evaluation_stream_miss_rate():
    # counts of a second (evaluation) stream against the calibration
    # ranking: 1 - cum[n-1]/tot is the share of evaluation tokens whose id is
    # not among the first n calibration ids (brute force).
    w = synth.WORKLOADS["tiny"]
    c_cal, _ = oracle.count(synth.make_ids(w), w.V)
    order, _, _, _ = oracle.select(c_cal, w.V)
    rng = np.random.default_rng(11)
    ev = rng.integers(0, w.V, 20000).astype(np.int32)
    c_ev, _ = oracle.count(ev, w.V)
    cum, tot, _ = oracle.coverage_curve(c_ev, order)
    for n in (10, 500, 1024):
        kept = set(order[:n].tolist())
        miss = sum(1 for t in ev.tolist() if t not in kept) / ev.size
        assert abs((1 - cum[n - 1] / tot) - miss) < 1e-12


def test_ids_outside_the_vocabulary_count_zero():
    counts = np.array([4, 4, 4], np.uint32)
    cum, tot, _ = oracle.coverage_curve(counts, np.array([2, -1, 7], np.int32))
    assert cum.tolist() == [4, 4, 4] and tot == 12
