"""GPU parity of the coverage curve (vt_coverage_curve) against the oracle:
exact integer sums and the same double-precision threshold decision
(VocabTrim page, Step 2 coverage for every V_high; guidance table's
coverage threshold; Step 5's share of tokens outside the vocabulary)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import DEV, to_dev_i32, to_dev_u32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


def run(dlh, counts, order, thr):
    cum, tot, vh = dlh.vt_coverage_curve(to_dev_u32(counts), to_dev_i32(order), thr)
    torch.cuda.synchronize()
    return (cum.view(torch.int64).cpu().numpy().view(np.uint64), int(tot.view(torch.int64).item()),
            int(vh.item()))


def check(dlh, counts, order, thresholds):
    for thr in thresholds:
        cum_g, tot_g, vh_g = run(dlh, counts, order, thr)
        cum_o, tot_o, vh_o = oracle.coverage_curve(counts, order, thr)
        assert np.array_equal(cum_g, cum_o) and tot_g == tot_o and vh_g == vh_o, (thr, vh_g, vh_o)


def test_tiny_ranking(dlh):
    w = synth.WORKLOADS["tiny"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    order, _, _, _ = oracle.select(c, w.V)
    check(dlh, c, order, [0.0, 0.5, 0.85, 0.8962, 0.9, 0.95, 0.99, 1.0, 1.5])
    check(dlh, c, order[:1024], [0.85, 0.9])       # partial ranking


@pytest.mark.parametrize("V,L", [(1, 1), (5, 3), (4096, 4096), (4097, 4097), (10000, 8193),
                                 (262144, 131072)])
def test_random_counts_and_ragged_sizes(dlh, V, L):
    rng = np.random.default_rng(V + L)
    c = rng.integers(0, 1000, V).astype(np.uint32)
    order = rng.permutation(V)[:L].astype(np.int32)
    if L > 2:
        order[1] = -5          # ids outside [0, V) add nothing
        order[-1] = V + 3
    thr = [0.0, 0.3, 0.7, 0.999, 1.0, 2.0]
    cum_o, tot_o, _ = oracle.coverage_curve(c, order)
    if tot_o:                  # thresholds that land exactly on a step
        thr += [float(cum_o[L // 2]) / tot_o]
    check(dlh, c, order, thr)


def test_counts_near_uint32_max_sum_exactly(dlh):
    c = np.full(9000, 0xFFFFFFF0, np.uint32)
    order = np.arange(9000, dtype=np.int32)[::-1].copy()
    check(dlh, c, order, [0.5, 1.0])


def test_llama_calibration_curve(dlh):
    w = synth.WORKLOADS["llama3_8b"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    order, _, _, _ = oracle.select(c, w.V)
    check(dlh, c, order, [0.85, 0.8894, 0.9, 0.95])
    cum, tot, vh = run(dlh, c, order, 0.0)
    # the point the draft head uses: 32768 kept ids cover about 88.9 %
    assert abs(float(cum[32767]) / tot - 0.8894) < 1e-3
