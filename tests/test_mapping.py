"""Saving and loading the vocabulary mapping (counts, t2f, f2t with sha256
and the calibration seed): round trip, tamper and consistency checks. The
maps come from the oracle's selection over a seeded Zipf stream."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from drafter_lm_head_amd.mapping import MappingError, load_mapping, save_mapping


def make(seed=5, V=3000, V_high=700, n=200000):
    rng = np.random.default_rng(seed)
    ids = synth.zipf_ids(n, V, 1.1, rng)
    counts, _ = oracle.count(ids, V)
    t2f, f2t, sel, tot = oracle.select(counts, V_high)
    return counts, t2f, f2t, sel, tot


def test_round_trip(tmp_path):
    counts, t2f, f2t, sel, tot = make()
    man = save_mapping(str(tmp_path), counts, t2f, f2t, seed=5, notes={"stream": "zipf 1.1"})
    assert man["sel_sum"] == sel and man["tot_sum"] == tot
    m = load_mapping(str(tmp_path))
    np.testing.assert_array_equal(m.counts, counts)
    np.testing.assert_array_equal(m.t2f, t2f)
    np.testing.assert_array_equal(m.f2t, f2t)
    assert m.seed == 5 and m.notes == {"stream": "zipf 1.1"}
    assert (m.V, m.V_high) == (3000, 700) and m.sums() == (sel, tot)
    # a second save of the same mapping writes the same bytes
    man2 = save_mapping(str(tmp_path / "again"), m.counts, m.t2f, m.f2t, seed=5,
                        notes=m.notes)
    assert man2["sha256"] == man["sha256"]


def test_torch_tensors_and_int32_counts(tmp_path):
    torch = pytest.importorskip("torch")
    counts, t2f, f2t, _, _ = make(seed=6, V=500, V_high=500, n=5000)
    save_mapping(str(tmp_path), torch.from_numpy(counts.view(np.int32)),
                 torch.from_numpy(t2f), torch.from_numpy(f2t))
    m = load_mapping(str(tmp_path))
    np.testing.assert_array_equal(m.counts, counts)
    assert m.seed is None and m.V_high == m.V == 500


def test_tampered_file_is_refused(tmp_path):
    counts, t2f, f2t, _, _ = make()
    save_mapping(str(tmp_path), counts, t2f, f2t, seed=1)
    p = tmp_path / "t2f.npy"
    b = bytearray(p.read_bytes())
    b[-1] ^= 1
    p.write_bytes(bytes(b))
    with pytest.raises(MappingError, match="checksum"):
        load_mapping(str(tmp_path))


def test_manifest_must_agree(tmp_path):
    counts, t2f, f2t, _, _ = make()
    save_mapping(str(tmp_path), counts, t2f, f2t)
    mp = tmp_path / "mapping.json"
    man = json.loads(mp.read_text())
    man["sel_sum"] += 1
    mp.write_text(json.dumps(man))
    with pytest.raises(MappingError, match="sums"):
        load_mapping(str(tmp_path))
    man["sel_sum"] -= 1
    man["format"] = "something-else"
    mp.write_text(json.dumps(man))
    with pytest.raises(MappingError, match="format"):
        load_mapping(str(tmp_path))
    os.remove(mp)
    with pytest.raises(MappingError):
        load_mapping(str(tmp_path))


def test_inconsistent_maps_are_refused(tmp_path):
    counts, t2f, f2t, _, _ = make(V=100, V_high=10, n=1000)
    bad = f2t.copy()
    bad[t2f[3]] = 4
    with pytest.raises(MappingError, match="inverse"):
        save_mapping(str(tmp_path), counts, t2f, bad)
    dup = t2f.copy()
    dup[1] = dup[0]
    with pytest.raises(MappingError, match="repeats"):
        save_mapping(str(tmp_path), counts, dup, f2t)
    out = t2f.copy()
    out[0] = 100
    with pytest.raises(MappingError, match="outside"):
        save_mapping(str(tmp_path), counts, out, f2t)
    with pytest.raises(MappingError):
        save_mapping(str(tmp_path), counts, t2f, f2t[:-1])
