"""The draft step under HIP graph capture (torch.cuda.CUDAGraph), as a serving
loop would run it: every call only launches kernels on the caller's stream
(no allocation, no memset, no host synchronisation), so it can be captured.
Each replay, with eager work and an unrelated eager call on the same
workspace in between, must give the eager call's results bit for bit."""
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


def case(seed, M, d, V_high):
    rng = np.random.default_rng(seed)
    W = synth.bf16_bits_from_f32(rng.standard_normal((V_high, d), dtype=np.float32) * np.float32(0.05))
    h = synth.bf16_bits_from_f32(rng.standard_normal((M, d), dtype=np.float32))
    t2f = rng.permutation(3 * V_high)[:V_high].astype(np.int32)
    return to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(t2f)


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture (loads the library's kernels)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("M,V_high,d", [(1, 5000, 512), (8, 5000, 512), (60, 5000, 512),
                                         (2, 32768, 256), (60, 32768, 256)])
def test_draft_head_graph_replays_match_eager(dlh, M, V_high, d):
    # Small heads: the GEMV and the 64-row kernel; 256 tile pairs: the GEMM
    # tiling on its LDS ring.
    k = 10
    h, W, t2f = case(M, M, d, V_high)
    h2, _, _ = case(M + 100, M, d, V_high)
    ws = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, k), dtype=torch.uint8,
                     device=DEV)
    ids = torch.empty((M, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((M, k), dtype=torch.float32, device=DEV)
    run = lambda: dlh.vt_draft_head(h, W, t2f, k, full_ids=ids, probs=probs, ws=ws)
    run()
    torch.cuda.synchronize()
    ref = (ids.cpu().numpy().tobytes(), probs.cpu().numpy().tobytes())
    g = capture(run)
    other_ids = torch.empty_like(ids)
    other_probs = torch.empty_like(probs)
    for rep in range(5):
        ids.fill_(-1)
        probs.fill_(-1.0)
        if rep % 2:  # an unrelated eager call on the same workspace
            dlh.vt_draft_head(h2, W, t2f, k, full_ids=other_ids, probs=other_probs, ws=ws)
        g.replay()
        torch.cuda.synchronize()
        assert (ids.cpu().numpy().tobytes(), probs.cpu().numpy().tobytes()) == ref, rep


@pytest.mark.parametrize("M,V_high", [(1, 3000), (9, 3000), (40, 32768)])
def test_draft_sample_graph_replays_match_eager(dlh, M, V_high):
    d = 256
    h, W, t2f = case(7 + M, M, d, V_high)
    ws = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, 1), dtype=torch.uint8,
                     device=DEV)
    ids = torch.empty(M, dtype=torch.int32, device=DEV)
    probs = torch.empty(M, dtype=torch.float32, device=DEV)
    run = lambda: dlh.vt_draft_sample(h, W, t2f, 1234, 5, full_ids=ids, probs=probs, ws=ws)
    run()
    torch.cuda.synchronize()
    ref = (ids.cpu().numpy().tobytes(), probs.cpu().numpy().tobytes())
    g = capture(run)
    for rep in range(4):
        ids.fill_(-1)
        probs.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert (ids.cpu().numpy().tobytes(), probs.cpu().numpy().tobytes()) == ref, rep
