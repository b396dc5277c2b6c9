"""GPU parity of the fused multinomial draw (vt_draft_sample) against the
oracle's Gumbel-max draw with the same Philox4x32-10 stream (VocabTrim page,
Step 4: sample one token from the subset softmax, remap to its full id)."""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
from parity import DEV, check_draws, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


def rand_case(seed, M, d, V_high, hscale=1.0):
    rng = np.random.default_rng(seed)
    W = synth.bf16_bits_from_f32(rng.standard_normal((V_high, d), dtype=np.float32) * np.float32(0.02))
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32) * np.float32(hscale))
    t2f = rng.permutation(2 * V_high)[:V_high].astype(np.int32)
    return h, W, t2f


def draw(dlh, h, W, t2f, seed, offset):
    ids, probs = dlh.vt_draft_sample(to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f), seed, offset)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), probs.cpu().numpy()


def test_tiny_pipeline_draws_match_oracle(dlh):
    w = synth.WORKLOADS["tiny"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    Wt = oracle.gather(synth.make_weights(w), t2f)
    h = synth.make_hidden(w, M=4, scale=8.0)
    near = 0
    for off in range(6):
        ids, probs = draw(dlh, h, Wt, t2f, 77, off)
        near += check_draws(ids, probs, h, Wt, t2f, 77, off)
    assert near <= 1


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 33, 60, 64, 65, 130, 300, 384, 385, 512])
def test_draws_match_oracle_gemv_and_mfma(dlh, M):
    # Past 256 rows the draw runs on 80- and 96-row blocks up to 384 rows,
    # on two groups of 256 rows beyond.
    h, W, t2f = rand_case(100 + M, M, 512, 3000, hscale=6.0)   # ragged V_high
    for off in (0, 1, 2**40 + 5):
        ids, probs = draw(dlh, h, W, t2f, 0xDEADBEEF12345, off)
        assert check_draws(ids, probs, h, W, t2f, 0xDEADBEEF12345, off) <= max(1, M // 64)


@pytest.mark.parametrize("M,d,V_high", [(300, 520, 4097), (384, 72, 1000)])
def test_two_stage_draws_with_ragged_hidden_size(dlh, M, d, V_high):
    # Draws on the 80- and 96-row blocks (two ring stages, draft-row loads
    # halfway through each K step) with a partial last K step and an odd
    # number of steps (d = 520), or one partial step (d = 72).
    h, W, t2f = rand_case(700 + M, M, d, V_high, hscale=4.0)
    for off in (0, 3):
        ids, probs = draw(dlh, h, W, t2f, 0x5EED, off)
        assert check_draws(ids, probs, h, W, t2f, 0x5EED, off) <= max(1, M // 64)


@pytest.mark.parametrize("M,d,V_high", [(150, 72, 1000), (200, 520, 4097), (256, 4096, 700),
                                         (450, 8, 700)])
def test_draws_on_3_and_4_blocks_with_few_k_steps(dlh, M, d, V_high):
    # Draws on 3 and 4 blocks per wave (and past 384 rows on two groups of
    # 256) with hidden sizes of 2 K steps (d = 72), 9 (520), 1 (8) and 64
    # (4096): the variates drawn in the epilogue whatever the step count.
    h, W, t2f = rand_case(800 + M, M, d, V_high, hscale=4.0)
    for off in (0, 5):
        ids, probs = draw(dlh, h, W, t2f, 0xC0FFEE, off)
        assert check_draws(ids, probs, h, W, t2f, 0xC0FFEE, off) <= max(1, M // 64)


@pytest.mark.parametrize("V_high", [1, 64, 65, 200, 40000])
def test_two_row_draws_few_and_many_workgroups(dlh, V_high):
    # Two rows: one merging workgroup (one tile) or two in parallel; the
    # counters must be back at zero after every call.
    h, W, t2f = rand_case(700 + V_high, 2, 256, V_high, hscale=4.0)
    hd, Wd, td = to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)
    ws = torch.zeros(dlh.vt_draft_head_workspace_size(2, V_high, 256, 1), dtype=torch.uint8,
                     device=DEV)
    for off in (0, 1, 2):
        ids, probs = dlh.vt_draft_sample(hd, Wd, td, 99, off, ws=ws)
        torch.cuda.synchronize()
        assert check_draws(ids.cpu().numpy(), probs.cpu().numpy(), h, W, t2f, 99, off) <= 1
        assert int(ws[:256].to(torch.int64).sum().item()) == 0


def test_draws_are_reproducible_and_move_with_offset(dlh):
    h, W, t2f = rand_case(5, 4, 256, 2048, hscale=2.0)
    a = draw(dlh, h, W, t2f, 1, 10)
    for _ in range(5):
        b = draw(dlh, h, W, t2f, 1, 10)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    others = [draw(dlh, h, W, t2f, 1, 11 + i)[0] for i in range(4)]
    assert any(not np.array_equal(a[0], o) for o in others)


def _exact_head(z, rows):
    zb = synth.bf16_bits_from_f32(np.asarray(z, np.float32))
    W = np.zeros((len(z), 8), np.uint16)
    W[:, 0] = zb
    h = np.zeros((rows, 8), np.uint16)
    h[:, 0] = synth.bf16_bits_from_f32(np.array([1.0], np.float32))[0]
    return h, W, synth.f32_from_bf16_bits(zb).astype(np.float64)


@pytest.mark.parametrize("M", [4, 64, 256])
def test_gpu_draws_follow_the_softmax(dlh, M):
    # Draws from a 6-token subset with exactly known logits: the histogram
    # over many (row, offset) draws matches softmax(z) (chi-square).
    h, W, z = _exact_head([1.5, 0.25, -0.5, 2.0, 0.0, -3.0], M)
    p = np.exp(z - z.max())
    p /= p.sum()
    t2f = np.array([40, 7, 19, 3, 88, 61], np.int32)
    inv = {int(f): j for j, f in enumerate(t2f)}
    hd, Wd, td = to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)
    counts = np.zeros(6)
    n_off = 12000 // M
    out = torch.empty((n_off, M), dtype=torch.int32, device=DEV)
    for off in range(n_off):
        dlh.vt_draft_sample(hd, Wd, td, 4242, off, full_ids=out[off])
    ids = out.cpu().numpy().ravel()
    counts = np.bincount([inv[int(i)] for i in ids], minlength=6)
    chi2, pv = stats.chisquare(counts, counts.sum() * p)
    assert pv > 1e-4, (counts, counts.sum() * p)


def test_peaked_row_always_draws_its_argmax(dlh):
    z = np.zeros(300)
    z[123] = 40.0
    h, W, _ = _exact_head(z, 3)
    t2f = np.arange(1000, 1300, dtype=np.int32)
    for off in range(5):
        ids, probs = draw(dlh, h, W, t2f, 9, off)
        assert (ids == 1123).all() and np.allclose(probs, 1.0)


@pytest.fixture(scope="module")
def llama(dlh):
    w = synth.WORKLOADS["llama3_8b"]
    W = synth.make_weights(w)
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    Wt = oracle.gather(W, t2f)
    del W
    return w, Wt, t2f


@pytest.mark.parametrize("M", [1, 60])
def test_llama_full_size_draws(dlh, llama, M):
    w, Wt, t2f = llama
    h = synth.make_hidden(w, M=M, scale=4.0)
    for off in (0, 1):
        ids, probs = draw(dlh, h, Wt, t2f, 2025, off)
        assert check_draws(ids, probs, h, Wt, t2f, 2025, off) <= max(1, M // 20)
