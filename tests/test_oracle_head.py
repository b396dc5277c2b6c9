"""Pins of the oracle's gather (VocabTrim page, Step 3), trimmed logits
(Step 4; FR-Spec notes, key design), subset softmax and top-k remap against
exact integer arithmetic, library routines, brute force, closed forms and a
hand-worked example."""
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax as sp_softmax

import oracle
import synth
from conftest import GOLDEN

bf = synth.bf16_bits_from_f32
f32 = synth.f32_from_bf16_bits


def rand_bf16(rng, shape, std=1.0):
    return bf(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


# ---------------------------------------------------------------- gather
def test_gather_is_row_copy():
    rng = np.random.default_rng(0)
    W = rng.integers(0, 2**16, size=(300, 24), dtype=np.uint16)
    t2f = rng.permutation(300)[:77].astype(np.int32)
    out = oracle.gather(W, t2f)
    assert out.tobytes() == W[t2f].tobytes()
    np.testing.assert_array_equal(oracle.gather(W, np.arange(300, dtype=np.int32)), W)


def test_gather_rejects_out_of_range():
    W = np.zeros((5, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.gather(W, np.array([0, 5], np.int32))
    with pytest.raises(ValueError):
        oracle.gather(W, np.array([-1], np.int32))


# ---------------------------------------------------------------- logits
def test_logits_exact_integers():
    # Small integers are exact in bf16; their dot products are exact
    # integers, so the oracle must reproduce Python's integer arithmetic.
    rng = np.random.default_rng(1)
    M, d, rows = 3, 40, 29
    hi = rng.integers(-8, 9, size=(M, d))
    Wi = rng.integers(-8, 9, size=(rows, d))
    z = oracle.logits(bf(hi.astype(np.float32)), bf(Wi.astype(np.float32)))
    for m in range(M):
        for j in range(rows):
            assert z[m, j] == sum(int(hi[m, t]) * int(Wi[j, t]) for t in range(d))


def test_logits_one_hot_reads_a_column():
    rng = np.random.default_rng(2)
    W = rand_bf16(rng, (50, 16), 0.02)
    for t in (0, 7, 15):
        h = np.zeros((1, 16), np.float32)
        h[0, t] = 1.0
        z = oracle.logits(bf(h), W)
        np.testing.assert_array_equal(z[0], f32(W[:, t]).astype(np.float64))


def test_logits_match_numpy_float64():
    rng = np.random.default_rng(3)
    h = rand_bf16(rng, (4, 256))
    W = rand_bf16(rng, (333, 256), 0.02)
    z = oracle.logits(h, W)
    hf, Wf = f32(h).astype(np.float64), f32(W).astype(np.float64)
    ref = hf @ Wf.T
    scale = np.abs(hf) @ np.abs(Wf).T
    assert np.all(np.abs(z - ref) <= 1e-13 * scale)


def test_trimmed_logits_equal_full_logits_at_kept_rows():
    # Trimming only drops rows: the kept logits are the full head's logits.
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w)
    h = synth.make_hidden(w, M=2)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    z_full = oracle.logits(h, W)
    z_trim = oracle.logits(h, oracle.gather(W, t2f))
    np.testing.assert_array_equal(z_trim, z_full[:, t2f])


def test_trimmed_equals_full_on_llama_slice():
    w = synth.WORKLOADS["llama3_8b"]
    rng = np.random.default_rng(4)
    W = rand_bf16(rng, (2048, w.d), 0.02)
    h = rand_bf16(rng, (1, w.d))
    t2f = rng.permutation(2048)[:512].astype(np.int32)
    np.testing.assert_array_equal(oracle.logits(h, oracle.gather(W, t2f)),
                                  oracle.logits(h, W)[:, t2f])


# ---------------------------------------------------------------- softmax
def test_softmax_matches_scipy_and_sums_to_one():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((3, 5000)) * 3
    p, mu, S = oracle.softmax(z)
    np.testing.assert_allclose(p, sp_softmax(z, axis=1), rtol=1e-13, atol=0)
    assert np.all(np.abs(p.sum(axis=1) - 1) < 1e-12)
    np.testing.assert_array_equal(mu, z.max(axis=1))
    np.testing.assert_allclose(np.log(S) + mu, logsumexp(z, axis=1), rtol=1e-14)


def test_softmax_shift_invariance_and_uniform():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((1, 1000))
    p1, _, _ = oracle.softmax(z)
    p2, _, _ = oracle.softmax(z + 37.5)
    np.testing.assert_allclose(p1, p2, rtol=1e-12)
    p, mu, S = oracle.softmax(np.full((1, 1024), 0.25))
    assert mu[0] == 0.25 and S[0] == 1024.0
    assert np.all(p == 1.0 / 1024)


def test_softmax_designed_case():
    # W rows alpha_j e_0 and h = e_0 give z_j = alpha_j exactly; the oracle's
    # probabilities must be the textbook softmax of alpha.
    alpha = np.array([0.5, -1.0, 2.0, 2.0, 0.0, -3.0], np.float32)
    W = np.zeros((6, 8), np.float32)
    W[:, 0] = alpha
    h = np.zeros((1, 8), np.float32)
    h[0, 0] = 1.0
    z = oracle.logits(bf(h), bf(W))
    np.testing.assert_array_equal(z[0], alpha.astype(np.float64))
    e = np.exp(alpha.astype(np.float64) - 2.0)
    p, _, _ = oracle.softmax(z)
    np.testing.assert_allclose(p[0], e / e.sum(), rtol=1e-15)


# ---------------------------------------------------------------- top-k
def brute_topk(z, t2f, k):
    out = []
    for m in range(z.shape[0]):
        order = np.lexsort((t2f, -z[m]))     # z desc, then full id asc
        out.append(t2f[order[:k]])
    return np.array(out, np.int32)


def test_topk_brute_force_and_full_sort():
    rng = np.random.default_rng(7)
    z = np.round(rng.standard_normal((4, 600)) * 4) / 4   # many exact ties
    t2f = rng.permutation(5000)[:600].astype(np.int32)
    for k in (1, 10, 64, 600):
        ids, ti = oracle.topk(z, t2f, k)
        np.testing.assert_array_equal(ids, brute_topk(z, t2f, k))
        np.testing.assert_array_equal(t2f[ti], ids)


def test_topk_all_ties_take_lowest_full_ids():
    t2f = np.array([9, 3, 7, 1, 8, 0], np.int32)
    ids, ti = oracle.topk(np.zeros((1, 6)), t2f, 4)
    assert ids.tolist() == [[0, 1, 3, 7]]
    assert ti.tolist() == [[5, 3, 1, 2]]


# ---------------------------------------------------------------- draft head
def test_hand_worked_draft_head():
    g = json.load(open(os.path.join(GOLDEN, "hand_head.json")))
    h = bf(np.array(g["h"], np.float32))
    W = bf(np.array(g["W_trim"], np.float32))
    t2f = np.array(g["t2f"], np.int32)
    ids, probs, (z, mu, S) = oracle.draft_head(h, W, t2f, g["k"], want_logits=True)
    np.testing.assert_array_equal(z, np.array(g["z"], np.float64))
    np.testing.assert_array_equal(mu, np.array(g["row_max"], np.float64))
    np.testing.assert_allclose(S, g["row_sum"], rtol=1e-15)
    assert ids.tolist() == g["full_ids"]
    np.testing.assert_allclose(probs, np.array(g["probs"], np.float32), rtol=0, atol=0)


def test_draft_head_is_composition():
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w)
    h = synth.make_hidden(w, M=3)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    Wt = oracle.gather(W, t2f)
    ids, probs, (z, mu, S) = oracle.draft_head(h, Wt, t2f, w.k, want_logits=True)
    np.testing.assert_array_equal(z, oracle.logits(h, Wt))
    p, mu2, S2 = oracle.softmax(z)
    np.testing.assert_array_equal(mu, mu2)
    ids2, ti = oracle.topk(z, t2f, w.k)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(probs, np.take_along_axis(p, ti, 1).astype(np.float32))
    np.testing.assert_array_equal(ids, brute_topk(z, t2f, w.k))


def test_full_vocab_reproduces_untrimmed_head():
    # V_high = V: the frequency-ranked permutation of the whole head must give
    # the same picks as the untrimmed head (identity map); only the order of
    # the fp64 softmax sum differs.
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w)
    h = synth.make_hidden(w, M=2)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V)
    assert not np.array_equal(t2f, np.arange(w.V))
    ids_t, p_t = oracle.draft_head(h, oracle.gather(W, t2f), t2f, 16)
    ids_u, p_u = oracle.draft_head(h, W, np.arange(w.V, dtype=np.int32), 16)
    np.testing.assert_array_equal(ids_t, ids_u)
    np.testing.assert_allclose(p_t, p_u, rtol=1e-6)


def test_peaked_variant_is_peaked():
    # h x 16 (exact in bf16) sharpens the subset softmax so that the absolute
    # probability tolerance is meaningful.
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w)
    h16 = synth.make_hidden(w, scale=16.0)
    h1 = synth.make_hidden(w)
    np.testing.assert_array_equal(f32(h16), f32(h1) * 16)
    t2f = np.arange(w.V, dtype=np.int32)
    _, p1 = oracle.draft_head(h1, W, t2f, 1)
    _, p16 = oracle.draft_head(h16, W, t2f, 1)
    assert p1[0, 0] < 0.05 and p16[0, 0] > 0.2


def test_head_shrink_figure():
    # FR-Spec notes: the head goes from d x 128k to d x 32k, a 75 % cut.
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["head_shrink"]
    assert 1 - g["trimmed_vocab_k"] / g["full_vocab_k"] == g["compute_cut"]
    w = synth.WORKLOADS["llama3_8b"]
    assert abs((1 - w.V_high / w.V) - g["compute_cut"]) < 0.01


# ------------------------------------------------------------------ bias
# A head that carries a bias keeps the bias of the kept ids (VocabTrim page,
# Step 3); the trimmed head is then a linear layer with that bias.
def test_bias_gather_is_a_copy_of_the_kept_entries():
    rng = np.random.default_rng(40)
    b = rng.integers(0, 2**16, size=500, dtype=np.uint16)
    t2f = rng.permutation(500)[:123].astype(np.int32)
    out = oracle.gather(b[:, None], t2f)[:, 0]
    assert out.tobytes() == b[t2f].tobytes()


def test_zero_weights_pick_the_largest_bias():
    # With W = 0 every logit is its bias: the picks are the k largest bias
    # values (equal values: lower full id) and the probabilities their softmax.
    rng = np.random.default_rng(41)
    V_high, d, k = 300, 16, 12
    bias_f = np.round(rng.standard_normal(V_high) * 4) / 4   # many exact ties
    bias = bf(bias_f.astype(np.float32))
    bv = f32(bias).astype(np.float64)
    W = np.zeros((V_high, d), np.uint16)
    h = rand_bf16(rng, (3, d))
    t2f = rng.permutation(10_000)[:V_high].astype(np.int32)
    ids, probs, (z, mu, S) = oracle.draft_head(h, W, t2f, k, want_logits=True, bias=bias)
    order = sorted(range(V_high), key=lambda j: (-bv[j], t2f[j]))[:k]
    p = np.exp(bv - logsumexp(bv))
    for m in range(3):
        np.testing.assert_array_equal(z[m], bv)
        assert ids[m].tolist() == [int(t2f[j]) for j in order]
        np.testing.assert_allclose(probs[m], p[order], rtol=1e-6)


def test_bias_shifts_every_logit_by_its_entry():
    rng = np.random.default_rng(42)
    V_high, d = 200, 64
    W = rand_bf16(rng, (V_high, d), 0.1)
    h = rand_bf16(rng, (2, d))
    bias = rand_bf16(rng, V_high, 2.0)
    t2f = np.arange(V_high, dtype=np.int32)
    _, _, (z0, _, _) = oracle.draft_head(h, W, t2f, 5, want_logits=True)
    _, _, (z1, _, _) = oracle.draft_head(h, W, t2f, 5, want_logits=True, bias=bias)
    np.testing.assert_allclose(z1 - z0, np.broadcast_to(f32(bias), z0.shape), rtol=0,
                               atol=1e-12)
    # a constant bias leaves the softmax unchanged
    c = bf(np.full(V_high, 3.5, np.float32))
    i0, p0 = oracle.draft_head(h, W, t2f, 7)
    i1, p1 = oracle.draft_head(h, W, t2f, 7, bias=c)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_allclose(p0, p1, rtol=1e-6)
