"""GPU checks of the boundary's auxiliary calls through the C ABI:

* vt_head_logits' per-row softmax statistics (max and sum of exp over the
  kept subset; FR-Spec notes, key design: the softmax covers the subset only)
  against the fp64 oracle;
* vt_draft_head_trimmed, the draft step without the remap (VocabTrim page,
  Practical Guidance: remapping overhead), against the oracle run with the
  identity map, which ranks equal logits by the lower trimmed index;
* the bounded wait of the two-row merge made to give up from the host (the
  workspace's hold and spin-limit words): affected outputs are -1 / NaN, the
  status query reports it once, and the next call is exact again;
* the streaming-read ceiling kernel runs over a buffer.
"""
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import DEV, check_picks, to_dev_bf16, to_dev_i32


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
    t2f = rng.permutation(3 * V_high)[:V_high].astype(np.int32)
    return h, W, t2f


@pytest.mark.parametrize("M,d,V_high,scale", [(1, 4096, 32768, 1.0), (3, 512, 1000, 16.0),
                                               (2, 256, 65, 4.0)])
def test_row_statistics(dlh, M, d, V_high, scale):
    h, W, _ = rand_case(31 + M, M, d, V_high, scale)
    _, rmax, rsum = dlh.vt_head_logits(to_dev_bf16(h), to_dev_bf16(W), stats=True)
    torch.cuda.synchronize()
    z = oracle.logits(h, W)
    mu_o = z.max(axis=1)
    s_o = np.exp(z - mu_o[:, None]).sum(axis=1)
    from parity import logit_bound
    bound = logit_bound(h, W)
    rmax = rmax.cpu().numpy().astype(np.float64)
    rsum = rsum.cpu().numpy().astype(np.float64)
    # max: within the fp32 logit bound of the row; sum: each term exp(z - mu)
    # moves by at most a factor exp(2 * bound), plus fp32 summation error.
    assert np.all(np.abs(rmax - mu_o) <= bound.max(axis=1))
    tol = np.expm1(2 * bound.max(axis=1)) + V_high * 2.0 ** -23
    assert np.all(np.abs(rsum - s_o) <= tol * s_o), (rsum, s_o)


@pytest.mark.parametrize("M,d,V_high,k", [(1, 4096, 32768, 10), (2, 512, 3000, 16),
                                           (60, 1024, 2500, 10), (100, 256, 700, 8)])
def test_trimmed_ids_match_identity_map_oracle(dlh, M, d, V_high, k):
    h, W, t2f = rand_case(57 + M, M, d, V_high, 3.0)
    ids, probs = dlh.vt_draft_head_trimmed(to_dev_bf16(h), to_dev_bf16(W), k)
    torch.cuda.synchronize()
    ident = np.arange(V_high, dtype=np.int32)
    ids_o, _, (z_o, _, _) = oracle.draft_head(h, W, ident, k, want_logits=True)
    check_picks(ids.cpu().numpy(), probs.cpu().numpy(), z_o, ident, k, ids_o)
    # with the remap the same picks come back as t2f[j] (no exact ties here)
    full, p_full = dlh.vt_draft_head(to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t2f[ids.cpu().numpy()], full.cpu().numpy())
    np.testing.assert_array_equal(probs.cpu().numpy(), p_full.cpu().numpy())


@pytest.mark.parametrize("sample", [False, True])
def test_bounded_wait_gives_up_observably(dlh, sample):
    # Two draft rows over 79 tiles: the last two workgroups merge one row
    # each, the earlier of them after waiting for every arrival. The hold
    # word asks it to wait for one arrival more than exist; the spin limit
    # makes it give up after 1000 sleeps.
    M, d, V_high, k = 2, 512, 5000, 10
    h, W, t2f = rand_case(91, M, d, V_high, 3.0)
    hd, Wd, td = to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)
    kk = 1 if sample else k
    ws = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, kk), dtype=torch.uint8,
                     device=DEV)

    def run():
        if sample:
            return dlh.vt_draft_sample(hd, Wd, td, 5, 6, ws=ws)
        return dlh.vt_draft_head(hd, Wd, td, k, ws=ws)

    ref_ids, ref_p = [t.cpu().numpy() for t in run()]
    dlh.vt_draft_head_status(ws)                                   # nothing to report
    words = ws[dlh.VT_WS_HOLD_OFFSET:dlh.VT_WS_SPIN_LIMIT_OFFSET + 4].view(torch.int32)
    words.copy_(torch.tensor([1, 1000], dtype=torch.int32))
    ids, p = [t.cpu().numpy().reshape(M, -1) for t in run()]
    with pytest.raises(dlh.VtError) as e:
        dlh.vt_draft_head_status(ws)
    assert e.value.status == dlh.VT_ERR_TIMEOUT
    dlh.vt_draft_head_status(ws)                                   # cleared by the query
    # the earlier merger takes row 1; row 0 is merged by the last arrival
    assert np.all(ids[1] == -1) and np.all(np.isnan(p[1]))
    np.testing.assert_array_equal(ids[0], ref_ids.reshape(M, -1)[0])
    words.zero_()
    ids2, p2 = [t.cpu().numpy() for t in run()]
    dlh.vt_draft_head_status(ws)
    np.testing.assert_array_equal(ids2, ref_ids)
    np.testing.assert_array_equal(p2, ref_p)
    assert int(ws[:256].to(torch.int64).sum().item()) == 0


def test_stream_read_runs(dlh):
    buf = torch.zeros(1 << 24, dtype=torch.uint8, device=DEV)
    sink = dlh.vt_stream_read(buf)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0          # zeros fold to zero: the store never fires
    with pytest.raises(dlh.VtError):
        dlh.vt_stream_read(buf[:1000])
