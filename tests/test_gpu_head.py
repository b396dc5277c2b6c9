"""GPU parity of the draft head through the C ABI (VocabTrim page,
Implementation, Step 4; FR-Spec notes, key design): trimmed logits, subset
softmax, per-row top-k and the trimmed -> full remap, against the fp64 CPU
oracle under the acceptance rule in tests/parity.py."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import (DEV, check_picks, logit_bound, to_dev_bf16, to_dev_i32)


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


def rand_case(seed, M, d, V_high, V=None, hscale=1.0):
    rng = np.random.default_rng(seed)
    V = V or max(V_high, 2 * V_high)
    W = synth.bf16_bits_from_f32(rng.standard_normal((V_high, d), dtype=np.float32) * np.float32(0.02))
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32) * np.float32(hscale))
    t2f = rng.permutation(V)[:V_high].astype(np.int32)
    return h, W, t2f


def run_head(dlh, h, W, t2f, k):
    ids, probs = dlh.vt_draft_head(to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), probs.cpu().numpy()


def check_case(dlh, h, W, t2f, k):
    ids_g, probs_g = run_head(dlh, h, W, t2f, k)
    ids_o, probs_o, (z_o, _, _) = oracle.draft_head(h, W, t2f, k, want_logits=True)
    return check_picks(ids_g, probs_g, z_o, t2f, k, ids_o)


def test_tiny_pipeline_matches_oracle(dlh):
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    Wt = oracle.gather(W, t2f)
    for scale in (1.0, 16.0):       # flat and peaked subset softmax
        h = synth.make_hidden(w, scale=scale)
        check_case(dlh, h, Wt, t2f, w.k)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16])
def test_draft_rows(dlh, M):
    h, W, t2f = rand_case(M, M, 512, 3000)
    check_case(dlh, h, W, t2f, 10)


@pytest.mark.parametrize("M", [17, 33, 60, 64, 65, 100, 128, 192, 257, 320, 321, 448, 449,
                               512])
def test_draft_tree_rows(dlh, M):
    # On this small head (too few tile pairs for the GEMM tiling) up to 32
    # rows run the 64-row MFMA kernel, past 32 the GEMM tiling (one more
    # 16-row block per wave for every 64 rows: full blocks at 64, 128, 192,
    # 320, 448, 512, one row past them at 257, 321, 449); then one merge
    # workgroup per row.
    h, W, t2f = rand_case(200 + M, M, 1024, 2500)
    check_case(dlh, h, W, t2f, 10)


@pytest.mark.parametrize("V_high,d,k,M", [(1, 256, 1, 60), (70, 520, 10, 60), (129, 8, 64, 60),
                                           (3000, 3584, 64, 60), (4097, 64, 10, 60),
                                           (8193, 128, 64, 60), (12288, 64, 33, 60),
                                           (4097, 520, 33, 130), (65, 8, 64, 193),
                                           (777, 8192, 10, 64), (300, 8192, 16, 200),
                                           (300, 8, 8, 40), (200, 8192, 10, 512),
                                           (4097, 520, 10, 300), (1000, 72, 10, 400),
                                           (65, 8, 64, 385)])
def test_draft_tree_edges(dlh, V_high, d, k, M):
    # Ragged tiles and row groups: a last tile of one row, a last group of
    # two (M = 130) or one (M = 193) draft rows; the longest rows (d = 8192)
    # on the GEMM tiling's single-tile and tile-pair workgroups, and one
    # 16-byte chunk per row (d = 8). Past 256 rows (two ring stages, the
    # draft-row loads issued halfway through each step) an odd number of K
    # steps with a partial last one (d = 520), a single partial step (72)
    # and a single chunk (8).
    h, W, t2f = rand_case(300 + V_high, M, d, V_high, hscale=2.0)
    check_case(dlh, h, W, t2f, min(k, V_high))


@pytest.mark.parametrize("V_high,d,M", [(32641, 72, 3), (32768, 1000, 37), (33000, 520, 64),
                                         (40000, 8, 17), (32768, 8192, 5)])
def test_gemm_tiling_small_trees(dlh, V_high, d, M):
    # Up to 64 draft rows a head of at least 256 tile pairs runs the GEMM
    # tiling: hidden sizes that leave a partial last K step (72, 1000, 520)
    # or a single chunk per row (8), a ragged last tile pair (33000, 40000),
    # and the longest rows, whose staggered K loops wrap around d.
    h, W, t2f = rand_case(900 + M, M, d, V_high, hscale=2.0)
    check_case(dlh, h, W, t2f, 10)


@pytest.mark.parametrize("V_high", [1, 10, 63, 64, 65, 1000, 4097])
def test_ragged_vocab(dlh, V_high):
    h, W, t2f = rand_case(V_high, 2, 256, V_high)
    check_case(dlh, h, W, t2f, min(10, V_high))


@pytest.mark.parametrize("d", [8, 72, 256, 520, 1000, 2048, 3584, 4096, 6144, 8192])
def test_hidden_sizes(dlh, d):
    h, W, t2f = rand_case(d, 1, d, 777)
    check_case(dlh, h, W, t2f, 10)


@pytest.mark.parametrize("d,V_high", [(6144, 777), (8192, 1000), (8192, 65), (4096, 4097)])
def test_two_rows_long_hidden(dlh, d, V_high):
    # Two draft rows with long rows: the register budget gives 8-wave
    # workgroups of one tile (d > 4096) or 16-wave ones of two tiles.
    h, W, t2f = rand_case(400 + d + V_high, 2, d, V_high)
    check_case(dlh, h, W, t2f, min(10, V_high))


@pytest.mark.parametrize("V_high,d,M", [(32768, 4096, 1), (32833, 4096, 2), (40000, 2048, 1),
                                         (32800, 2048, 2), (65536, 1024, 1)])
def test_large_vocab_tail_rows(dlh, V_high, d, M):
    # From 512 tiles on, one or two draft rows run two-tile 16-wave
    # workgroups (ragged last blocks of one tile or a partial one, two-row
    # units at d = 2048, four-row units at d = 1024).
    h, W, t2f = rand_case(500 + V_high + d, M, d, V_high, V=V_high + 1000, hscale=2.0)
    check_case(dlh, h, W, t2f, 10)


@pytest.mark.parametrize("M", [1, 2])
def test_large_vocab_repeatable(dlh, M):
    # Which wave computes a row changes from call to call (rows are taken
    # from a counter), and with two rows which workgroups merge them; the
    # results must not, and the counters must be back at zero.
    h, W, t2f = rand_case(77, M, 4096, 32768)
    hd, Wd, td = to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)
    n = dlh.vt_draft_head_workspace_size(M, 32768, 4096, 10)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref = None
    for _ in range(30):
        ids, probs = dlh.vt_draft_head(hd, Wd, td, 10, ws=ws)
        cur = (ids.cpu().numpy().tobytes(), probs.cpu().numpy().tobytes())
        ref = ref or cur
        assert cur == ref
    torch.cuda.synchronize()
    assert int(ws[:256 + 2 * 2 * 64 * 8].to(torch.int64).sum().item()) == 0


@pytest.mark.parametrize("V_high", [1, 37, 64, 65, 128, 200])
def test_two_rows_few_workgroups(dlh, V_high):
    # One workgroup merges both rows; from two workgroups on the last two
    # merge one row each.
    h, W, t2f = rand_case(300 + V_high, 2, 512, V_high, hscale=3.0)
    check_case(dlh, h, W, t2f, min(10, V_high))


@pytest.mark.parametrize("k", [1, 2, 31, 32, 63, 64])
def test_k_range(dlh, k):
    h, W, t2f = rand_case(100 + k, 2, 256, 5000, hscale=4.0)
    check_case(dlh, h, W, t2f, k)


@pytest.mark.parametrize("M,V_high", [(2, 700), (2, 5000), (6, 700), (6, 5000)])
def test_exact_ties_break_to_lower_full_id(dlh, M, V_high):
    # All rows equal: every logit ties, so the picks are the k smallest full ids.
    # With M > 2 and V_high = 5000 the candidate tiles hold 5000 tied logits,
    # more than the survivor buffer: the exact max-round fallback runs.
    rng = np.random.default_rng(5)
    d, k = 64, 12
    row = synth.bf16_bits_from_f32(rng.standard_normal(d, dtype=np.float32))
    W = np.tile(row, (V_high, 1))
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32))
    t2f = rng.permutation(100_000)[:V_high].astype(np.int32)
    ids_g, probs_g = run_head(dlh, h, W, t2f, k)
    want = np.sort(t2f)[:k]
    for m in range(M):
        np.testing.assert_array_equal(ids_g[m], want)
        np.testing.assert_allclose(probs_g[m], 1.0 / V_high, rtol=1e-5)


@pytest.mark.parametrize("k,M", [(10, 64), (64, 64), (10, 128)])
def test_draft_tree_max_vocab(dlh, k, M):
    # The largest kept vocabulary (4096 tiles per row) with full trees; with
    # k = 64 many tiles reach the merge's bound.
    from drafter_lm_head_amd import VT_VHIGH_MAX
    h, W, t2f = rand_case(11 + k + M, M, 64, VT_VHIGH_MAX, hscale=3.0)
    check_case(dlh, h, W, t2f, k)


def test_widest_tree_full_size_sampled_rows(dlh):
    # VT_M_MAX draft rows on the LLaMA-3-8B head shape (a seeded random head):
    # rows are independent, so a sample of them is checked against the oracle
    # run on those rows alone (the first and last of several row groups).
    from drafter_lm_head_amd import VT_M_MAX
    w = synth.WORKLOADS["llama3_8b"]
    rng = np.random.default_rng(512)
    Wt = synth.bf16_bits_from_f32(rng.standard_normal((w.V_high, w.d), dtype=np.float32) * np.float32(0.02))
    t2f = rng.permutation(w.V)[: w.V_high].astype(np.int32)
    h = synth.make_hidden(w, M=VT_M_MAX)
    ids_g, probs_g = run_head(dlh, h, Wt, t2f, w.k)
    rows = [0, 1, 63, 64, 200, 447, 448, VT_M_MAX - 1]
    ids_o, _, (z_o, _, _) = oracle.draft_head(h[rows], Wt, t2f, w.k, want_logits=True)
    check_picks(ids_g[rows], probs_g[rows], z_o, t2f, w.k, ids_o)


def test_hand_worked_example(dlh):
    import json, os
    from conftest import GOLDEN
    g = json.load(open(os.path.join(GOLDEN, "hand_head.json")))
    # d = 4 is below the 8-element vector width: pad with zero columns.
    h = np.zeros((2, 8), np.float32)
    h[:, :4] = g["h"]
    W = np.zeros((5, 8), np.float32)
    W[:, :4] = g["W_trim"]
    ids_g, probs_g = run_head(dlh, synth.bf16_bits_from_f32(h), synth.bf16_bits_from_f32(W),
                              np.array(g["t2f"], np.int32), g["k"])
    assert ids_g.tolist() == g["full_ids"]
    np.testing.assert_allclose(probs_g, np.array(g["probs"]), rtol=2e-6)


@pytest.mark.parametrize("M", [1, 2, 3, 20, 200])
def test_determinism_and_counter_reset(dlh, M):
    h, W, t2f = rand_case(7, M, 1024, 20000)
    hd, Wd, td = to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)
    M, d = h.shape
    n = dlh.vt_draft_head_workspace_size(M, 20000, d, 10)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref = None
    for _ in range(50):
        ids, probs = dlh.vt_draft_head(hd, Wd, td, 10, ws=ws)
        cur = (ids.cpu().numpy().tobytes(), probs.cpu().numpy().tobytes())
        if ref is None:
            ref = cur
        assert cur == ref
    torch.cuda.synchronize()
    # the ticket counter and the GEMV path's group maxima (a fixed
    # 256 + 2*2*64*8-byte prefix) are back at zero for the next call
    assert int(ws[:256 + 2 * 2 * 64 * 8].to(torch.int64).sum().item()) == 0


def test_full_vocab_equals_untrimmed_head(dlh):
    # V_high = V with the frequency-ranked permutation gives the same picks as
    # the untrimmed head with the identity map.
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w)
    h = synth.make_hidden(w, M=2, scale=4.0)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V)
    ident = np.arange(w.V, dtype=np.int32)
    ids_t, p_t = run_head(dlh, h, oracle.gather(W, t2f), t2f, 16)
    ids_u, p_u = run_head(dlh, h, W, ident, 16)
    np.testing.assert_array_equal(ids_t, ids_u)
    np.testing.assert_allclose(p_t, p_u, rtol=1e-5)


def test_logits_within_fp32_bound(dlh):
    h, W, t2f = rand_case(9, 2, 4096, 2000)
    z_g = dlh.vt_head_logits(to_dev_bf16(h), to_dev_bf16(W)).cpu().numpy().astype(np.float64)
    z_o = oracle.logits(h, W)
    assert np.all(np.abs(z_g - z_o) <= logit_bound(h, W))


@pytest.fixture(scope="module")
def llama(dlh):
    # The LLaMA-3-8B drafter head as the method builds it: 1e8 Zipf ids,
    # counted and ranked by the oracle, rows gathered from a seeded W.
    w = synth.WORKLOADS["llama3_8b"]
    W = synth.make_weights(w)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    Wt = oracle.gather(W, t2f)
    del W
    return w, Wt, t2f


@pytest.mark.parametrize("M,scale", [(1, 1.0), (1, 16.0), (4, 1.0)])
def test_llama_head_full_size(dlh, llama, M, scale):
    w, Wt, t2f = llama
    h = synth.make_hidden(w, M=M, scale=scale)
    worst = check_case(dlh, h, Wt, t2f, w.k)
    print("worst", worst)


def test_eagle2_tree_full_size(dlh, llama):
    # EAGLE-2-style draft tree: 60 rows per step on the LLaMA-3-8B head.
    w, Wt, t2f = llama
    h = synth.make_hidden(w, M=60)
    print("worst", check_case(dlh, h, Wt, t2f, w.k))


@pytest.mark.parametrize("M", [16, 64])
def test_qwen_head_full_size(dlh, M):
    w = synth.WORKLOADS["qwen2_7b"]
    rng = np.random.default_rng(77)
    Wt = synth.bf16_bits_from_f32(rng.standard_normal((w.V_high, w.d), dtype=np.float32) * np.float32(0.02))
    t2f = rng.permutation(w.V)[: w.V_high].astype(np.int32)
    h = synth.make_hidden(w, M=M)
    print("worst", check_case(dlh, h, Wt, t2f, w.k))


def test_llama_logits_bound(dlh, llama):
    w, Wt, t2f = llama
    h = synth.make_hidden(w)
    z_g = dlh.vt_head_logits(to_dev_bf16(h), to_dev_bf16(Wt)).cpu().numpy().astype(np.float64)
    z_o = oracle.logits(h, Wt)
    err = np.abs(z_g - z_o)
    assert np.all(err <= logit_bound(h, Wt))
    print("max |dz|", err.max())
