"""GPU parity of the preparation steps through the C ABI: histogram,
top-V_high selection and row gather must equal the CPU oracle bit for bit
(VocabTrim page, Implementation, Steps 1-3; FR-Spec notes, key design)."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dlh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import drafter_lm_head_amd as m
    return m


from parity import (bf16_host, to_dev_bf16, to_dev_i32, to_dev_u32, u32_host,
                    u64_scalar)


def run_count(dlh, ids, V):
    c, inv = dlh.vt_count_freq(to_dev_i32(ids), V)
    torch.cuda.synchronize()
    return u32_host(c), u64_scalar(inv)


@pytest.mark.parametrize("case", ["tiny", "invalid", "ragged_n", "small_V", "empty"])
def test_count_small(dlh, case):
    rng = np.random.default_rng(11)
    if case == "tiny":
        w = synth.WORKLOADS["tiny"]
        ids, V = synth.make_ids(w), w.V
    elif case == "invalid":
        V = 5000
        ids = rng.integers(-100, V + 100, size=300_001).astype(np.int32)
        ids[:2] = [np.iinfo(np.int32).min, np.iinfo(np.int32).max]
    elif case == "ragged_n":
        V = 777
        ids = rng.integers(0, V, size=4 * 1024 * 5 + 3).astype(np.int32)
    elif case == "small_V":
        V = 1
        ids = rng.integers(-1, 2, size=1001).astype(np.int32)
    else:
        V = 300
        ids = np.zeros(0, np.int32)
    c, inv = run_count(dlh, ids, V)
    c_o, inv_o = oracle.count(ids, V)
    np.testing.assert_array_equal(c, c_o)
    assert inv == inv_o


def test_count_accumulate(dlh):
    rng = np.random.default_rng(12)
    V = 40000          # one range of 16-bit bins
    a = rng.integers(-5, V + 5, size=123_457).astype(np.int32)
    b = rng.integers(0, V, size=70_001).astype(np.int32)
    c, inv = dlh.vt_count_freq(to_dev_i32(a), V)
    c, inv = dlh.vt_count_freq(to_dev_i32(b), V, counts=c, n_invalid=inv, accumulate=True)
    torch.cuda.synchronize()
    c_o, inv_o = oracle.count(np.concatenate([a, b]), V)
    np.testing.assert_array_equal(u32_host(c), c_o)
    assert u64_scalar(inv) == inv_o


@pytest.mark.parametrize("name", ["llama3_8b", "qwen2_7b"])
def test_count_full_size(dlh, name):
    # 1e8 Zipf ids over 128256 / 152064 ids: two ranges of 16-bit bins, hot bins.
    w = synth.WORKLOADS[name]
    ids = synth.make_ids(w)
    c, inv = run_count(dlh, ids, w.V)
    c_o, inv_o = oracle.count(ids, w.V)
    np.testing.assert_array_equal(c, c_o)
    assert inv == inv_o == 0


@pytest.mark.parametrize("V,n,hot", [(100_000, 20_000_000, 0.9), (152_064, 3_000_001, 0.5),
                                     (38_913, 1_000_003, 1.0)])
def test_count_16bit_bins_overflow(dlh, V, n, hot):
    # Past 38912 ids the counts live in 16-bit LDS bins: a hot id crosses 2^15
    # many times in every workgroup, so its overflow records carry most of its
    # count; an odd V puts the hot id next to the padding bin.
    rng = np.random.default_rng(V)
    ids = rng.integers(-3, V + 3, size=n).astype(np.int32)
    ids[rng.random(n) < hot] = V - 1 if V % 2 else V // 2
    c, inv = run_count(dlh, ids, V)
    c_o, inv_o = oracle.count(ids, V)
    np.testing.assert_array_equal(c, c_o)
    assert inv == inv_o


def run_select(dlh, counts, V_high):
    t2f, f2t, sel, tot = dlh.vt_select_vocab(to_dev_u32(counts), V_high)
    torch.cuda.synchronize()
    return t2f.cpu().numpy(), f2t.cpu().numpy(), u64_scalar(sel), u64_scalar(tot)


def check_select(dlh, counts, V_high):
    got = run_select(dlh, counts, V_high)
    want = oracle.select(counts, V_high)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    assert got[2:] == want[2:]


def test_select_tiny(dlh):
    w = synth.WORKLOADS["tiny"]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    for V_high in (1, 8, w.V_high, 1025, w.V):
        check_select(dlh, c, V_high)


@pytest.mark.parametrize("seed", [0, 1])
def test_select_heavy_ties(dlh, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 4, size=70_000).astype(np.uint32)
    for V_high in (1, 1000, 34_999, 69_999, 70_000):
        check_select(dlh, c, V_high)


def test_select_edge_counts(dlh):
    check_select(dlh, np.zeros(5000, np.uint32), 17)          # nothing counted
    check_select(dlh, np.full(3000, 9, np.uint32), 3000)      # uniform -> identity
    big = np.array([2**32 - 1, 0, 2**32 - 1, 2**31, 5, 2**31 + 1], np.uint32)
    for V_high in range(1, 7):
        check_select(dlh, big, V_high)


@pytest.mark.parametrize("V", [16384, 16387, 50001])
def test_select_many_workgroups_edges(dlh, V):
    # From 16384 ids on the selection runs over many workgroups: all-zero and
    # uniform counts (pure id order), full-range 32-bit counts, a few maximal
    # counts over a sea of ties; cuts at and around the 2048-key sort blocks.
    rng = np.random.default_rng(V)
    cases = [np.zeros(V, np.uint32), np.full(V, 7, np.uint32),
             rng.integers(0, 2**32, size=V, dtype=np.uint64).astype(np.uint32),
             np.where(rng.random(V) < 0.01, 2**32 - 1, rng.integers(0, 3, size=V)).astype(np.uint32)]
    for c in cases:
        for V_high in (1, 2, 2047, 2048, 2049, V - 1, V):
            check_select(dlh, c, V_high)


@pytest.mark.parametrize("name", ["llama3_8b", "qwen2_7b"])
def test_select_full_size(dlh, name):
    w = synth.WORKLOADS[name]
    c, _ = oracle.count(synth.make_ids(w), w.V)
    for V_high in (8192, 32768, 65536, w.V):
        check_select(dlh, c, V_high)


def test_gather_small_and_bad_rows(dlh):
    rng = np.random.default_rng(13)
    for V, d, V_high in ((300, 8, 300), (4096, 256, 1024), (1000, 520, 7), (50, 8192, 3)):
        W = rng.integers(0, 2**16, size=(V, d), dtype=np.uint16)
        t2f = rng.permutation(V)[:V_high].astype(np.int32)
        out = dlh.vt_gather_head(to_dev_bf16(W), to_dev_i32(t2f))
        torch.cuda.synchronize()
        assert bf16_host(out).tobytes() == oracle.gather(W, t2f).tobytes()
    # ids outside [0, V) are not read through: zero rows, counted
    W = rng.integers(0, 2**16, size=(64, 16), dtype=np.uint16)
    t2f = np.array([3, -1, 64, 2**31 - 1, 5], np.int32)
    n_bad = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    out = bf16_host(dlh.vt_gather_head(to_dev_bf16(W), to_dev_i32(t2f), n_bad=n_bad))
    assert int(n_bad.item()) == 3
    np.testing.assert_array_equal(out[0], W[3])
    np.testing.assert_array_equal(out[4], W[5])
    assert not out[1:4].any()


def test_prep_pipeline_llama(dlh):
    # The whole preparation at the LLaMA-3-8B shape: count 1e8 ids, keep 32768,
    # gather the [128256, 4096] head; every byte equals the oracle's.
    w = synth.WORKLOADS["llama3_8b"]
    ids = synth.make_ids(w)
    W = synth.make_weights(w)
    c, inv = dlh.vt_count_freq(to_dev_i32(ids), w.V)
    t2f, f2t, sel, tot = dlh.vt_select_vocab(c, w.V_high)
    Wt = dlh.vt_gather_head(to_dev_bf16(W), t2f)
    cov = dlh.coverage(sel, tot)
    c_o, _ = oracle.count(ids, w.V)
    t2f_o, f2t_o, sel_o, tot_o = oracle.select(c_o, w.V_high)
    np.testing.assert_array_equal(t2f.cpu().numpy(), t2f_o)
    np.testing.assert_array_equal(f2t.cpu().numpy(), f2t_o)
    assert cov == sel_o / tot_o
    assert bf16_host(Wt).tobytes() == oracle.gather(W, t2f_o).tobytes()


def test_mapping_saved_from_device_round_trips(dlh, tmp_path):
    # The device's counts and maps, saved with their checksums and the
    # stream's seed, load back bit for bit; the reloaded t2f gathers the same
    # head as the device's own.
    from drafter_lm_head_amd.mapping import load_mapping, save_mapping
    rng = np.random.default_rng(23)
    V, V_high, d = 128256, 32768, 64
    ids = synth.zipf_ids(2_000_000, V, 1.1, rng)
    c, _ = dlh.vt_count_freq(to_dev_i32(ids), V)
    t2f, f2t, sel, tot = dlh.vt_select_vocab(c, V_high)
    save_mapping(str(tmp_path), c, t2f, f2t, seed=23)
    m = load_mapping(str(tmp_path))
    np.testing.assert_array_equal(m.counts, u32_host(c))
    np.testing.assert_array_equal(m.t2f, t2f.cpu().numpy())
    np.testing.assert_array_equal(m.f2t, f2t.cpu().numpy())
    assert m.sums() == (u64_scalar(sel), u64_scalar(tot)) and m.seed == 23
    c_o, _ = oracle.count(ids, V)
    np.testing.assert_array_equal(m.t2f, oracle.select(c_o, V_high)[0])
    W = synth.head_weights(V, d, rng)
    Wd = to_dev_bf16(W)
    a = dlh.vt_gather_head(Wd, t2f)
    b = dlh.vt_gather_head(Wd, to_dev_i32(m.t2f))
    torch.cuda.synchronize()
    assert bf16_host(a).tobytes() == bf16_host(b).tobytes()
