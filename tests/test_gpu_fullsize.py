"""GPU parity at the workloads' full sizes, on the launch shapes the
benchmark times, against the fp64 CPU oracle (VocabTrim page, Implementation,
Steps 1-5; FR-Spec notes, key design and key experimental data):

* the Qwen-2-7B-shaped head (d = 3584, V = 152064 cut to 32768 kept rows, one
  draft row), built the way the method builds it (1e8 Zipf ids counted and
  ranked, rows gathered), with top-10 picks and with the multinomial draw;
* the untrimmed LLaMA-3-8B head (all 128256 rows, identity map), the
  baseline of the wall-time reduction that trimming buys.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import check_draws, check_picks, to_dev_bf16, to_dev_i32


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


@pytest.fixture(scope="module")
def qwen():
    w = synth.WORKLOADS["qwen2_7b"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    t2f, _, _, _ = oracle.select(c, w.V_high)
    W = synth.make_weights(w)
    Wt = oracle.gather(W, t2f)
    del W
    return w, Wt, t2f


@pytest.mark.parametrize("scale", [1.0, 16.0])
def test_qwen_head_one_row_full_size(dlh, qwen, scale):
    # d = 3584 gives 448 16-byte chunks per row (7 per lane) and 512 tiles:
    # the one-row GEMV in two-tile 16-wave workgroups.
    w, Wt, t2f = qwen
    h = synth.make_hidden(w, M=1, scale=scale)
    ids, probs = dlh.vt_draft_head(to_dev_bf16(h), to_dev_bf16(Wt), to_dev_i32(t2f), w.k)
    torch.cuda.synchronize()
    ids_o, _, (z_o, _, _) = oracle.draft_head(h, Wt, t2f, w.k, want_logits=True)
    print("worst", check_picks(ids.cpu().numpy(), probs.cpu().numpy(), z_o, t2f, w.k, ids_o))


def test_qwen_draw_one_row_full_size(dlh, qwen):
    w, Wt, t2f = qwen
    h = synth.make_hidden(w, M=1, scale=4.0)
    hd, Wd, td = to_dev_bf16(h), to_dev_bf16(Wt), to_dev_i32(t2f)
    near = 0
    for off in range(4):
        ids, probs = dlh.vt_draft_sample(hd, Wd, td, 0x5EED, off)
        torch.cuda.synchronize()
        near += check_draws(ids.cpu().numpy(), probs.cpu().numpy(), h, Wt, t2f, 0x5EED, off)
    assert near <= 1


def test_untrimmed_llama_head_identity_map(dlh):
    # V_high = V = 128256 with the identity map: 2004 tiles, the full head the
    # trimmed one is compared with.
    w = synth.WORKLOADS["llama3_8b"]
    W = synth.make_weights(w)
    ident = np.arange(w.V, dtype=np.int32)
    for scale in (1.0, 16.0):
        h = synth.make_hidden(w, M=1, scale=scale)
        ids, probs = dlh.vt_draft_head(to_dev_bf16(h), to_dev_bf16(W), to_dev_i32(ident), w.k)
        torch.cuda.synchronize()
        ids_o, _, (z_o, _, _) = oracle.draft_head(h, W, ident, w.k, want_logits=True)
        print("worst", check_picks(ids.cpu().numpy(), probs.cpu().numpy(), z_o, ident, w.k,
                                   ids_o))
