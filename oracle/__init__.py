"""CPU oracle of the frequency-ranked drafter LM head (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does. It wraps ``oracle.c`` (plain C, fp64), which shares no code with the
GPU library, through ctypes.

Each function cites the passage it follows; see ``oracle.c`` for the
definitions and the readings of points the pages leave open. All functions
are pinned by the CPU tests (``tests/test_oracle_*.py``); none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = C.CDLL(_LIB)
            P = C.c_void_p
            i32, u64 = C.c_int32, C.c_uint64
            lib.or_count.argtypes = [P, u64, i32, P, C.c_int, P]
            lib.or_select.argtypes = [P, i32, i32, P, P, P, P]
            lib.or_gather.argtypes = [P, i32, i32, P, i32, P]
            lib.or_logits.argtypes = [P, i32, i32, P, i32, P]
            lib.or_softmax.argtypes = [P, i32, i32, P, P, P]
            lib.or_topk.argtypes = [P, P, i32, i32, i32, P, P]
            lib.or_draft_head.argtypes = [P, i32, i32, P, P, i32, P, i32, P, P, P, P, P]
            lib.or_draft_sample.argtypes = [P, i32, i32, P, P, i32, P, u64, u64, P, P, P, P]
            lib.or_philox4x32_10.argtypes = [P, P, P]
            lib.or_philox4x32_10.restype = None
            lib.or_gumbel.argtypes = [u64, u64, i32, i32]
            lib.or_gumbel.restype = C.c_double
            lib.or_gumbel_block.argtypes = [u64, u64, i32, i32, P]
            lib.or_gumbel_block.restype = C.c_int
            lib.or_coverage_curve.argtypes = [P, i32, P, i32, C.c_double, P, P, P]
            lib.or_threads.argtypes = []
            lib.or_set_threads.argtypes = [C.c_int]
            lib.or_set_threads.restype = C.c_int
            for f in (lib.or_threads, lib.or_count, lib.or_select, lib.or_gather, lib.or_logits,
                      lib.or_softmax, lib.or_topk, lib.or_draft_head, lib.or_draft_sample,
                      lib.or_coverage_curve):
                f.restype = C.c_int
            _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().or_threads())


def set_threads(n: int) -> int:
    """Sets the OpenMP thread count of later calls (results do not depend on
    it); returns the count now in effect."""
    return int(_load().or_set_threads(int(n)))


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dtype, ndim=None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    if ndim is not None and a.ndim != ndim:
        raise ValueError(f"expected {ndim}-d array, got shape {a.shape}")
    return a


def _ok(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def count(ids, V: int, counts=None, n_invalid: int = 0):
    """Token-id histogram (VocabTrim page, Step 1; FR-Spec notes, key design).

    Returns ``(counts uint32[V], n_invalid)``. When ``counts`` is given the new
    ids are added to a copy of it and to ``n_invalid`` (batched streams).
    """
    ids = _arr(ids, np.int32, 1)
    acc = counts is not None
    c = np.zeros(V, np.uint32) if not acc else _arr(counts, np.uint32, 1).copy()
    if c.shape[0] != V:
        raise ValueError("counts must have V entries")
    inv = np.array([n_invalid if acc else 0], dtype=np.uint64)
    _ok(_load().or_count(_p(ids), ids.size, V, _p(c), int(acc), _p(inv)), "count")
    return c, int(inv[0])


def select(counts, V_high: int):
    """Top-V_high by count, ties to the lower id (VocabTrim page, Step 2).

    Returns ``(t2f int32[V_high], f2t int32[V], sel, tot)``; coverage is
    ``sel / tot``.
    """
    c = _arr(counts, np.uint32, 1)
    V = c.shape[0]
    t2f = np.empty(V_high, np.int32)
    f2t = np.empty(V, np.int32)
    sel = np.zeros(1, np.uint64)
    tot = np.zeros(1, np.uint64)
    _ok(_load().or_select(_p(c), V, V_high, _p(t2f), _p(f2t), _p(sel), _p(tot)), "select")
    return t2f, f2t, int(sel[0]), int(tot[0])


def gather(W, t2f):
    """Row gather W_trim = W[t2f] (VocabTrim page, Step 3)."""
    W = _arr(W, np.uint16, 2)
    t2f = _arr(t2f, np.int32, 1)
    out = np.empty((t2f.size, W.shape[1]), np.uint16)
    _ok(_load().or_gather(_p(W), W.shape[0], W.shape[1], _p(t2f), t2f.size, _p(out)), "gather")
    return out


def logits(h, W):
    """fp64 logits z[M, rows] = h . W^T (VocabTrim page, Step 4; FR-Spec)."""
    h = _arr(h, np.uint16, 2)
    W = _arr(W, np.uint16, 2)
    if h.shape[1] != W.shape[1]:
        raise ValueError("h and W must have the same d")
    z = np.empty((h.shape[0], W.shape[0]), np.float64)
    _ok(_load().or_logits(_p(h), h.shape[0], h.shape[1], _p(W), W.shape[0], _p(z)), "logits")
    return z


def softmax(z):
    """Subset softmax in fp64 (FR-Spec notes, key design).

    Returns ``(p[M, n], mu[M], S[M])``.
    """
    z = _arr(z, np.float64, 2)
    M, n = z.shape
    p = np.empty_like(z)
    mu = np.empty(M, np.float64)
    S = np.empty(M, np.float64)
    _ok(_load().or_softmax(_p(z), M, n, _p(p), _p(mu), _p(S)), "softmax")
    return p, mu, S


def topk(z, t2f, k: int):
    """Per-row top-k by (logit desc, full id asc), remapped through t2f.

    Returns ``(full_ids int32[M, k], trimmed index int32[M, k])``.
    """
    z = _arr(z, np.float64, 2)
    t2f = _arr(t2f, np.int32, 1)
    M, n = z.shape
    if t2f.size != n:
        raise ValueError("t2f must have one entry per logit column")
    ids = np.empty((M, k), np.int32)
    ti = np.empty((M, k), np.int32)
    _ok(_load().or_topk(_p(z), _p(t2f), M, n, k, _p(ids), _p(ti)), "topk")
    return ids, ti


def _bias(bias, V_high):
    if bias is None:
        return None
    b = _arr(bias, np.uint16, 1)
    if b.size != V_high:
        raise ValueError("bias must have V_high entries")
    return b


def draft_head(h, W_trim, t2f, k: int, want_logits: bool = False, bias=None):
    """One draft-head call: logits (plus the head's bf16 bias when given; VocabTrim
    page, Step 3 keeps it), subset softmax, top-k, remap.

    Returns ``(full_ids int32[M, k], probs float32[M, k])`` and, with
    ``want_logits``, also ``(z fp64[M, V_high], mu[M], S[M])``.
    """
    h = _arr(h, np.uint16, 2)
    W_trim = _arr(W_trim, np.uint16, 2)
    t2f = _arr(t2f, np.int32, 1)
    M, d = h.shape
    V_high = W_trim.shape[0]
    if W_trim.shape[1] != d or t2f.size != V_high:
        raise ValueError("shape mismatch")
    b = _bias(bias, V_high)
    ids = np.empty((M, k), np.int32)
    probs = np.empty((M, k), np.float32)
    z = np.empty((M, V_high), np.float64) if want_logits else None
    mu = np.empty(M, np.float64)
    S = np.empty(M, np.float64)
    _ok(_load().or_draft_head(_p(h), M, d, _p(W_trim), _p(b), V_high, _p(t2f), k,
                              _p(ids), _p(probs), _p(z), _p(mu), _p(S)), "draft_head")
    if want_logits:
        return ids, probs, (z, mu, S)
    return ids, probs


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon et al., SC 2011) of one counter and key."""
    c = np.asarray(ctr, np.uint32).reshape(4).copy()
    k = np.asarray(key, np.uint32).reshape(2).copy()
    out = np.empty(4, np.uint32)
    _load().or_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def gumbel(seed: int, offset: int, M: int, n: int):
    """The Gumbel variates G[m, j] of a draw keyed by (seed, offset)."""
    g = np.empty((M, n), np.float64)
    _ok(_load().or_gumbel_block(C.c_uint64(seed), C.c_uint64(offset), M, n, _p(g)), "gumbel")
    return g


def draft_sample(h, W_trim, t2f, seed: int, offset: int, want_logits: bool = False, bias=None):
    """One multinomial draw per row from the subset softmax (Gumbel-max with
    Philox uniforms), remapped through t2f (VocabTrim page, Step 4).

    Returns ``(full_ids int32[M], probs float32[M], trimmed index int32[M])``
    and, with ``want_logits``, also ``z fp64[M, V_high]``.
    """
    h = _arr(h, np.uint16, 2)
    W_trim = _arr(W_trim, np.uint16, 2)
    t2f = _arr(t2f, np.int32, 1)
    M, d = h.shape
    V_high = W_trim.shape[0]
    if W_trim.shape[1] != d or t2f.size != V_high:
        raise ValueError("shape mismatch")
    b = _bias(bias, V_high)
    ids = np.empty(M, np.int32)
    probs = np.empty(M, np.float32)
    ti = np.empty(M, np.int32)
    z = np.empty((M, V_high), np.float64) if want_logits else None
    _ok(_load().or_draft_sample(_p(h), M, d, _p(W_trim), _p(b), V_high, _p(t2f), C.c_uint64(seed),
                                C.c_uint64(offset), _p(ids), _p(probs), _p(ti), _p(z)),
        "draft_sample")
    if want_logits:
        return ids, probs, ti, z
    return ids, probs, ti


def coverage_curve(counts, order, min_coverage: float = 1.0):
    """Cumulative counts along a ranking (VocabTrim page, Step 2's coverage
    for every V_high; the guidance table's coverage threshold).

    Returns ``(cum uint64[L], tot, v_high)``; coverage at n is cum[n-1]/tot.
    """
    c = _arr(counts, np.uint32, 1)
    o = _arr(order, np.int32, 1)
    cum = np.empty(o.size, np.uint64)
    tot = np.zeros(1, np.uint64)
    vh = np.zeros(1, np.int32)
    _ok(_load().or_coverage_curve(_p(c), c.size, _p(o), o.size, C.c_double(min_coverage),
                                  _p(cum), _p(tot), _p(vh)), "coverage_curve")
    return cum, int(tot[0]), int(vh[0])
