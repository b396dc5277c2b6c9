"""Saving and loading the vocabulary mapping, the method's one-time artefact.

The frequency statistics are gathered once, offline, and the kept set is
fixed from them (FR-Spec paper notes, key design: frequency-ranked
vocabulary compression; VocabTrim skill page, Implementation, Step 2, which
returns the two maps and the coverage). This module stores that result so a
serving process loads it instead of recounting:

* ``counts.npy``  uint32[V]       the calibration counts (vt_count_freq)
* ``t2f.npy``     int32[V_high]   trimmed index -> full id (vt_select_vocab)
* ``f2t.npy``     int32[V]        full id -> trimmed index, -1 if not kept
* ``mapping.json``                format tag, V, V_high, the kept and total
  counts, the calibration seed, the sha256 of each array file, and free-form
  notes from the caller

Arrays are plain ``.npy`` files written and read with pickling disabled.
``load_mapping`` checks every checksum and the maps' structure (t2f a set of
distinct ids in range, f2t its inverse, -1 elsewhere) and raises
``MappingError`` on any mismatch. Host code only: no step of the draft path
runs here.
"""
from __future__ import annotations

import hashlib
import json
import os
from dataclasses import dataclass, field

import numpy as np

FORMAT = "vocabtrim-mapping/1"
MANIFEST = "mapping.json"
_FILES = {"counts": ("counts.npy", np.uint32), "t2f": ("t2f.npy", np.int32),
          "f2t": ("f2t.npy", np.int32)}


class MappingError(ValueError):
    """A stored mapping is missing, corrupted or inconsistent."""


@dataclass
class VocabMapping:
    counts: np.ndarray          # uint32[V]
    t2f: np.ndarray             # int32[V_high]
    f2t: np.ndarray             # int32[V]
    seed: int | None = None     # seed of the calibration stream, if synthetic
    notes: dict = field(default_factory=dict)

    @property
    def V(self) -> int:
        return int(self.counts.shape[0])

    @property
    def V_high(self) -> int:
        return int(self.t2f.shape[0])

    def sums(self) -> tuple[int, int]:
        """(kept count, total count) as exact integers."""
        c = self.counts.astype(np.uint64)
        return int(c[self.t2f].sum()), int(c.sum())


def _host(a, dtype) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor on any device
        import torch
        a = a.detach()
        if a.dtype == torch.uint32:
            a = a.view(torch.int32)
        a = a.cpu().numpy()
    a = np.ascontiguousarray(a)
    if a.ndim != 1:
        raise MappingError(f"expected a 1-d array, got shape {a.shape}")
    if a.dtype != dtype:
        if a.dtype.itemsize != np.dtype(dtype).itemsize or a.dtype.kind not in "iu":
            raise MappingError(f"expected {np.dtype(dtype)}, got {a.dtype}")
        a = a.view(dtype)
    return a


def _sha256(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for block in iter(lambda: f.read(1 << 20), b""):
            h.update(block)
    return h.hexdigest()


def check_structure(counts: np.ndarray, t2f: np.ndarray, f2t: np.ndarray) -> None:
    """Raises MappingError unless t2f holds distinct ids in [0, V) and f2t is
    its inverse (f2t[t2f[i]] == i, -1 for every id that is not kept)."""
    V, V_high = counts.shape[0], t2f.shape[0]
    if f2t.shape[0] != V:
        raise MappingError(f"f2t has {f2t.shape[0]} entries, counts {V}")
    if not 1 <= V_high <= V:
        raise MappingError(f"V_high = {V_high} outside [1, V = {V}]")
    if t2f.min() < 0 or t2f.max() >= V:
        raise MappingError("t2f holds ids outside [0, V)")
    expect = np.full(V, -1, dtype=np.int32)
    expect[t2f] = np.arange(V_high, dtype=np.int32)
    if np.count_nonzero(expect >= 0) != V_high:
        raise MappingError("t2f repeats an id")
    if not np.array_equal(expect, f2t):
        raise MappingError("f2t is not the inverse of t2f")


def save_mapping(path: str, counts, t2f, f2t, seed: int | None = None,
                 notes: dict | None = None) -> dict:
    """Writes the mapping to directory ``path`` (created if needed) and
    returns the manifest. Accepts numpy arrays or torch tensors (copied to the
    host); uint32 counts may come as int32 bit patterns."""
    m = VocabMapping(_host(counts, np.uint32), _host(t2f, np.int32), _host(f2t, np.int32),
                     seed, dict(notes or {}))
    check_structure(m.counts, m.t2f, m.f2t)
    os.makedirs(path, exist_ok=True)
    sel, tot = m.sums()
    manifest = {"format": FORMAT, "V": m.V, "V_high": m.V_high, "sel_sum": sel,
                "tot_sum": tot, "seed": seed, "notes": m.notes, "sha256": {}}
    for key, (name, _) in _FILES.items():
        p = os.path.join(path, name)
        tmp = p + ".tmp"
        with open(tmp, "wb") as f:
            np.save(f, getattr(m, key), allow_pickle=False)
        os.replace(tmp, p)
        manifest["sha256"][name] = _sha256(p)
    tmp = os.path.join(path, MANIFEST + ".tmp")
    with open(tmp, "w") as f:
        json.dump(manifest, f, indent=1, sort_keys=True)
    os.replace(tmp, os.path.join(path, MANIFEST))
    return manifest


def load_mapping(path: str) -> VocabMapping:
    """Reads a mapping written by save_mapping, verifying the checksums, the
    shapes and dtypes, the stored sums and the maps' structure."""
    mp = os.path.join(path, MANIFEST)
    try:
        with open(mp) as f:
            manifest = json.load(f)
    except (OSError, ValueError) as e:
        raise MappingError(f"cannot read {mp}: {e}") from e
    if manifest.get("format") != FORMAT:
        raise MappingError(f"unknown format {manifest.get('format')!r}")
    arrays = {}
    for key, (name, dtype) in _FILES.items():
        p = os.path.join(path, name)
        if not os.path.exists(p):
            raise MappingError(f"missing {name}")
        want = manifest.get("sha256", {}).get(name)
        if _sha256(p) != want:
            raise MappingError(f"checksum mismatch for {name}")
        a = np.load(p, allow_pickle=False)
        if a.dtype != dtype or a.ndim != 1:
            raise MappingError(f"{name}: expected 1-d {np.dtype(dtype)}, got {a.dtype} {a.shape}")
        arrays[key] = a
    m = VocabMapping(arrays["counts"], arrays["t2f"], arrays["f2t"], manifest.get("seed"),
                     manifest.get("notes", {}))
    if m.V != manifest.get("V") or m.V_high != manifest.get("V_high"):
        raise MappingError("array sizes disagree with the manifest")
    check_structure(m.counts, m.t2f, m.f2t)
    if m.sums() != (manifest.get("sel_sum"), manifest.get("tot_sum")):
        raise MappingError("stored sums disagree with the counts")
    return m
