"""vt_draft_head_noalloc, the draft step for callers that cannot allocate:
through the C ABI, its results equal vt_draft_head's (same kernels, scratch
inside the library instead of a caller's workspace), on two calls in a row
whose second is smaller (the scratch keeps the first call's contents), and a
request larger than the fixed scratch is refused before any launch."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import DEV, to_dev_bf16, to_dev_i32


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


def case(seed, M, d, V_high, scale=1.0):
    rng = np.random.default_rng(seed)
    W = synth.bf16_bits_from_f32(rng.standard_normal((V_high, d), dtype=np.float32) * np.float32(0.02))
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32) * np.float32(scale))
    t2f = rng.permutation(4 * V_high)[:V_high].astype(np.int32)
    return to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)


def host(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("shapes", [
    [(60, 4096, 32768, 10), (1, 512, 5000, 8)],      # tree, then one row
    [(2, 4096, 32768, 10), (2, 256, 700, 4)],        # two-row GEMV merge, twice
    [(200, 1024, 8000, 16), (5, 520, 3001, 10)],     # GEMM-tiled, then small tree
])
def test_noalloc_matches_workspace_call(dlh, shapes):
    for i, (M, d, V_high, k) in enumerate(shapes):
        h, W, t2f = case(100 * i + M, M, d, V_high, scale=2.0)
        ws = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, k), dtype=torch.uint8,
                         device=DEV)
        ref_ids, ref_p = dlh.vt_draft_head(h, W, t2f, k, ws=ws)
        ids = torch.full((M, k), -7, dtype=torch.int32, device=DEV)
        probs = torch.full((M, k), -7.0, dtype=torch.float32, device=DEV)
        dlh.vt_draft_head_noalloc(h, W, t2f, k, full_ids=ids, probs=probs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(ids), host(ref_ids))
        np.testing.assert_array_equal(host(probs), host(ref_p))
        dlh.vt_draft_head_status(None, DEV)   # no bounded wait gave up


def test_noalloc_refuses_requests_beyond_its_scratch(dlh):
    M, d, V_high, k = 512, 64, 262144, 10
    assert dlh.vt_draft_head_workspace_size(M, V_high, d, k) > dlh.VT_NOALLOC_WS_BYTES
    h, W, t2f = case(1, 2, d, 64)
    hb = torch.zeros((M, d), dtype=torch.int16, device=DEV)
    Wb = torch.zeros((V_high, d), dtype=torch.int16, device=DEV)
    tb = torch.arange(V_high, dtype=torch.int32, device=DEV)
    ids = torch.full((M, k), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(dlh.VtError) as e:
        dlh.vt_draft_head_noalloc(hb, Wb, tb, k, full_ids=ids)
    assert e.value.status == dlh.VT_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert int((ids == -7).all().item()) == 1      # nothing was launched


@pytest.mark.parametrize("M", [1, 60])
def test_noalloc_graph_replays_match_eager(dlh, M):
    # The caller it exists for: a captured serving loop. After a first eager
    # call (which sets the scratch up), the call is captured in a HIP graph
    # with preallocated outputs; every replay, with an unrelated eager call
    # on the same scratch between some of them, gives the eager result.
    V_high, d, k = 5000, 512, 10
    h, W, t2f = case(300 + M, M, d, V_high, scale=2.0)
    h2, _, _ = case(400 + M, M, d, V_high, scale=2.0)
    ids = torch.empty((M, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((M, k), dtype=torch.float32, device=DEV)
    run = lambda: dlh.vt_draft_head_noalloc(h, W, t2f, k, full_ids=ids, probs=probs)
    run()
    torch.cuda.synchronize()
    ref = (host(ids).tobytes(), host(probs).tobytes())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    other_ids = torch.empty_like(ids)
    other_probs = torch.empty_like(probs)
    for rep in range(5):
        ids.fill_(-1)
        probs.fill_(-1.0)
        if rep % 2:
            dlh.vt_draft_head_noalloc(h2, W, t2f, k, full_ids=other_ids, probs=other_probs)
        g.replay()
        torch.cuda.synchronize()
        assert (host(ids).tobytes(), host(probs).tobytes()) == ref, rep
    dlh.vt_draft_head_status(None, DEV)
