"""GPU parity of heads that carry a bias (VocabTrim page, Implementation,
Step 3: the trimmed head keeps the bias entries of the kept ids and is a
linear layer with that bias): the bias gather, and the draft head and the
draw with z = h . W_trim^T + bias, against the fp64 CPU oracle under the
acceptance rule in tests/parity.py."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import (DEV, bf16_host, check_draws, check_picks, to_dev_bf16, to_dev_i32,
                    u32_host)


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


def biased_case(seed, M, d, V_high, bias_std=1.0):
    rng = np.random.default_rng(seed)
    W = synth.bf16_bits_from_f32(rng.standard_normal((V_high, d), dtype=np.float32) * np.float32(0.02))
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32))
    b = synth.bf16_bits_from_f32(rng.standard_normal(V_high, dtype=np.float32) * np.float32(bias_std))
    t2f = rng.permutation(2 * V_high)[:V_high].astype(np.int32)
    return h, W, b, t2f


def test_gather_bias_copies_kept_entries_and_counts_bad_ones(dlh):
    rng = np.random.default_rng(1)
    V, V_high = 128256, 32768
    b = rng.integers(0, 2**16, size=V, dtype=np.uint16)
    t2f = rng.permutation(V)[:V_high].astype(np.int32)
    t2f[[5, 999, V_high - 1]] = [-1, V, V + 7]
    n_bad = torch.zeros(1, dtype=torch.int32, device=DEV).view(torch.uint32)
    out = dlh.vt_gather_bias(to_dev_bf16(b), to_dev_i32(t2f), n_bad=n_bad)
    got = bf16_host(out)
    good = (t2f >= 0) & (t2f < V)
    want = np.zeros(V_high, np.uint16)
    want[good] = b[t2f[good]]
    assert got.tobytes() == want.tobytes()
    assert int(u32_host(n_bad)[0]) == 3
    # the oracle's row gather with d = 1 is the same copy
    assert oracle.gather(b[:, None], t2f[good])[:, 0].tobytes() == got[good].tobytes()


@pytest.mark.parametrize("M", [1, 3, 4, 5, 20, 60, 130, 192, 300, 448])
def test_biased_head_matches_oracle(dlh, M):
    # GEMV path up to 2 rows, the MFMA path beyond (past 128 rows the GEMM
    # tiling's 3-, 5- and 7-block shapes); V_high is ragged.
    h, W, b, t2f = biased_case(100 + M, M, 512, 3001)
    k = 10
    ids, probs = dlh.vt_draft_head_bias(to_dev_bf16(h), to_dev_bf16(W), to_dev_bf16(b),
                                        to_dev_i32(t2f), k)
    torch.cuda.synchronize()
    ids_o, _, (z_o, _, _) = oracle.draft_head(h, W, t2f, k, want_logits=True, bias=b)
    check_picks(ids.cpu().numpy(), probs.cpu().numpy(), z_o, t2f, k, ids_o)


@pytest.mark.parametrize("M", [2, 12])
def test_zero_weights_pick_the_largest_bias(dlh, M):
    # W = 0: each logit is its bias exactly (0 + b in fp32), so the picks
    # and probabilities must be the oracle's with no near-tie allowance.
    rng = np.random.default_rng(7)
    V_high, d, k = 1500, 64, 16
    b = synth.bf16_bits_from_f32((np.round(rng.standard_normal(V_high) * 8) / 8).astype(np.float32))
    W = np.zeros((V_high, d), np.uint16)
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32))
    t2f = rng.permutation(100_000)[:V_high].astype(np.int32)
    ids, probs = dlh.vt_draft_head_bias(to_dev_bf16(h), to_dev_bf16(W), to_dev_bf16(b),
                                        to_dev_i32(t2f), k)
    torch.cuda.synchronize()
    ids_o, probs_o = oracle.draft_head(h, W, t2f, k, bias=b)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_allclose(probs.cpu().numpy(), probs_o, rtol=1e-5)


@pytest.mark.parametrize("M", [1, 60])
def test_biased_head_full_size(dlh, M):
    # The LLaMA-3-8B head shape (d = 4096, V = 128256 trimmed to 32768) with a
    # seeded random head and bias, gathered on the GPU.
    w = synth.WORKLOADS["llama3_8b"]
    rng = np.random.default_rng(M)
    Wt = synth.bf16_bits_from_f32(rng.standard_normal((w.V_high, w.d), dtype=np.float32) * np.float32(0.02))
    t2f = rng.permutation(w.V)[: w.V_high].astype(np.int32)
    b = synth.bf16_bits_from_f32(rng.standard_normal(w.V, dtype=np.float32) * np.float32(0.5))
    bt = dlh.vt_gather_bias(to_dev_bf16(b), to_dev_i32(t2f))
    h = synth.make_hidden(w, M=M)
    ids, probs = dlh.vt_draft_head_bias(to_dev_bf16(h), to_dev_bf16(Wt), bt, to_dev_i32(t2f),
                                        w.k)
    torch.cuda.synchronize()
    ids_o, _, (z_o, _, _) = oracle.draft_head(h, Wt, t2f, w.k, want_logits=True, bias=b[t2f])
    check_picks(ids.cpu().numpy(), probs.cpu().numpy(), z_o, t2f, w.k, ids_o)


@pytest.mark.parametrize("M,V_high", [(2, 2000), (9, 2000), (70, 2000), (2, 33000), (40, 33000),
                                      (180, 2000), (300, 2000)])
def test_biased_draws_match_oracle(dlh, M, V_high):
    # Small heads: GEMV (two rows), 64-row kernel, GEMM tiling (3 and 5
    # blocks per wave past 128 rows); heads of 256 or more tile pairs: the
    # GEMM tiling with its variates drawn before the K loop, here with a
    # ragged last tile pair.
    h, W, b, t2f = biased_case(300 + M, M, 256, V_high, bias_std=2.0)
    near = 0
    for off in range(4):
        ids, probs = dlh.vt_draft_sample_bias(to_dev_bf16(h), to_dev_bf16(W), to_dev_bf16(b),
                                              to_dev_i32(t2f), 99, off)
        torch.cuda.synchronize()
        near += check_draws(ids.cpu().numpy(), probs.cpu().numpy(), h, W, t2f, 99, off, bias=b)
    assert near <= 1
