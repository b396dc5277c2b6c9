"""Pins of the oracle's multinomial draw (VocabTrim page, Step 4: the draft
loop samples one token from the subset softmax and remaps it): the
counter-based generator against its published known answers, the Gumbel
variates against their distribution, and the Gumbel-max draw against the
softmax probabilities it must reproduce."""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from conftest import GOLDEN


def test_philox_known_answers():
    kat = json.load(open(os.path.join(GOLDEN, "philox_kat.json")))
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        out = [int(x, 16) for x in v["out"]]
        assert oracle.philox4x32_10(ctr, key).tolist() == out


def test_philox_counter_and_key_sensitivity():
    # One flipped counter or key bit changes about half of the 128 output bits.
    base = oracle.philox4x32_10([1, 2, 3, 4], [5, 6])
    flips = []
    for word in range(6):
        for bit in (0, 13, 31):
            c, k = [1, 2, 3, 4], [5, 6]
            if word < 4:
                c[word] ^= 1 << bit
            else:
                k[word - 4] ^= 1 << bit
            o = oracle.philox4x32_10(c, k)
            flips.append(sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(o, base)))
    assert 48 <= np.mean(flips) <= 80 and min(flips) >= 32


def test_gumbel_variates_follow_the_standard_gumbel_law():
    g = oracle.gumbel(seed=12345, offset=7, M=8, n=25000).ravel()
    # mean = Euler-Mascheroni constant, variance = pi^2 / 6; then a
    # Kolmogorov-Smirnov test against the CDF exp(-exp(-x)).
    n = g.size
    assert abs(g.mean() - np.euler_gamma) < 5 * math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    assert stats.kstest(g, lambda x: np.exp(-np.exp(-x))).pvalue > 1e-4
    # the uniforms are (x + 1/2) / 2^24: the extreme variates are bounded
    assert g.max() < -math.log(-math.log1p(-0.5 / 2 ** 24)) + 1e-9
    assert g.min() > -math.log(-math.log(0.5 / 2 ** 24)) - 1e-9


def _exact_logit_head(z):
    """h, W with z[0, j] = z[j] exactly: h = e_0 and W[j, 0] = z[j] (bf16)."""
    zb = synth.bf16_bits_from_f32(np.asarray(z, np.float32))
    W = np.zeros((len(z), 8), np.uint16)
    W[:, 0] = zb
    h = np.zeros((1, 8), np.uint16)
    h[0, 0] = synth.bf16_bits_from_f32(np.array([1.0], np.float32))[0]
    return h, W, synth.f32_from_bf16_bits(zb).astype(np.float64)


def test_gumbel_max_draw_reproduces_the_softmax():
    # 24000 draws (4000 rows x 6 offsets) from a 6-token subset: the
    # histogram matches softmax(z) (chi-square), and each draw reports the
    # softmax probability of the drawn token.
    h1, W, z = _exact_logit_head([1.5, 0.25, -0.5, 2.0, 0.0, -3.0])
    p = np.exp(z - z.max())
    p /= p.sum()
    rows = 4000
    h = np.repeat(h1, rows, axis=0)
    t2f = np.array([40, 7, 19, 3, 88, 61], np.int32)
    counts = np.zeros(6)
    inv = {int(f): j for j, f in enumerate(t2f)}
    for off in range(6):
        ids, probs, ti = oracle.draft_sample(h, W, t2f, seed=2024, offset=off)
        assert [inv[int(i)] for i in ids] == ti.tolist()
        np.testing.assert_allclose(probs, p[ti].astype(np.float32), rtol=1e-6)
        counts += np.bincount(ti, minlength=6)
    chi2, pv = stats.chisquare(counts, counts.sum() * p)
    assert pv > 1e-4, (counts, counts.sum() * p)


def test_draws_depend_on_seed_offset_and_row_only():
    w = synth.WORKLOADS["tiny"]
    rng = np.random.default_rng(3)
    h = synth.bf16_bits_from_f32(rng.standard_normal((4, w.d)).astype(np.float32))
    W = synth.make_weights(w)[:w.V_high]
    t2f = np.arange(w.V_high, dtype=np.int32)
    a = oracle.draft_sample(h, W, t2f, seed=9, offset=100)[0]
    assert np.array_equal(a, oracle.draft_sample(h, W, t2f, seed=9, offset=100)[0])
    # other seeds or offsets give (almost surely) different draws somewhere
    assert not np.array_equal(a, oracle.draft_sample(h, W, t2f, seed=10, offset=100)[0]) or \
        not np.array_equal(a, oracle.draft_sample(h, W, t2f, seed=9, offset=101)[0])
    # a row's draw does not depend on the other rows (its counter carries m)
    b = oracle.draft_sample(h[:2], W, t2f, seed=9, offset=100)[0]
    assert np.array_equal(a[:2], b)


def test_peaked_logits_draw_the_argmax():
    # one logit 40 above the rest: every draw is that token (p > 1 - 1e-15)
    z = np.zeros(50)
    z[17] = 40.0
    h1, W, zz = _exact_logit_head(z)
    h = np.repeat(h1, 64, axis=0)
    t2f = np.arange(100, 150, dtype=np.int32)
    ids, probs, ti = oracle.draft_sample(h, W, t2f, seed=1, offset=0)
    assert (ti == 17).all() and (ids == 117).all()
    assert np.allclose(probs, 1.0)


def test_rows_sharing_a_generator_call_are_independent():
    # Rows 4b .. 4b + 3 take the four words of one Philox call: their
    # variates must be uncorrelated (a row reading another row's word would
    # give correlation 1), and rows of different blocks too.
    n = 40000
    g = oracle.gumbel(seed=77, offset=3, M=8, n=n)
    bound = 5.0 / math.sqrt(n)
    for r1, r2 in [(0, 1), (0, 2), (0, 3), (1, 2), (2, 3), (3, 4), (4, 7)]:
        assert abs(stats.spearmanr(g[r1], g[r2]).statistic) < bound, (r1, r2)
    # row m of block b is word m % 4 of the call with counter (j, b, offset)
    j = 12345
    x = oracle.philox4x32_10([j, 1, 3, 0], [77, 0])
    u = ((x >> 8).astype(np.float64) + 0.5) / 2 ** 24
    np.testing.assert_allclose(g[4:8, j], -np.log(-np.log(u)), rtol=0, atol=0)


def test_biased_draw_follows_the_bias_softmax():
    # W = 0 and bias = z: the draw histogram is softmax(bias) (chi-square).
    from scipy.special import softmax as sp_softmax
    bvals = np.array([1.0, -0.5, 2.25, 0.0, -2.0, 0.75], np.float32)
    bias = synth.bf16_bits_from_f32(bvals)
    p = sp_softmax(synth.f32_from_bf16_bits(bias).astype(np.float64))
    W = np.zeros((6, 8), np.uint16)
    h = np.zeros((3000, 8), np.uint16)
    t2f = np.array([5, 50, 500, 5000, 6, 60], np.int32)
    counts = np.zeros(6)
    for off in range(8):
        ids, probs, ti = oracle.draft_sample(h, W, t2f, seed=11, offset=off, bias=bias)
        np.testing.assert_allclose(probs, p[ti].astype(np.float32), rtol=1e-6)
        counts += np.bincount(ti, minlength=6)
    assert stats.chisquare(counts, counts.sum() * p).pvalue > 1e-4
