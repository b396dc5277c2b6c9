"""Seeded synthetic inputs for the frequency-ranked drafter LM head.

This module only draws inputs. It holds none of the method's arithmetic:
no counting, ranking, gathering, dot products, softmax or top-k. Both the
CPU oracle's tests and the GPU path's tests and benchmark draw their inputs
from here, so the two sides see identical bytes.

What is drawn, and why it stands in for the pages' data:

* Token ids follow a finite-support Zipf law, P(rank r) proportional to
  r**-s for r = 1..V, drawn by inverse-CDF sampling. The FR-Spec paper notes
  (Method / overall framework) justify the frequency-ranked subset with the
  Zipf long tail of token frequencies; the corpora the pages count on
  (SlimPajama, ShareGPT; FR-Spec notes, key design and ablations) and the
  drafter samples of the VocabTrim page (Implementation, Step 1) are not
  available, so seeded Zipf ids stand in for them. ``numpy.random.zipf`` is
  not used: it has unbounded support and rejects s = 1.
* Optionally the rank -> id map is a seeded random permutation, so that hot
  ids are spread over the id range as in a real tokenizer.
* The head weight W[V, d] is N(0, 0.02) in float32, rounded to bfloat16 with
  round-to-nearest-even; the draft hidden states h[M, d] are N(0, 1) float32
  rounded the same way. Trained weights are not available; the head's cost
  does not depend on weight values.

bfloat16 values are carried as their uint16 bit patterns (numpy has no
bfloat16 dtype).

Every workload uses ``numpy.random.SeedSequence(seed).spawn(4)`` to derive
four independent PCG64 streams, in this order: ids, permutation, W, h.
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "zipf_ids",
    "head_weights",
    "hidden_states",
    "streams",
    "make_ids",
    "make_weights",
    "make_hidden",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes plus the recipe of its inputs."""

    name: str
    d: int            # hidden size
    V: int            # full vocabulary
    V_high: int       # kept (frequency-ranked) vocabulary
    M: int            # draft rows per call
    k: int            # top-k per draft row
    n_ids: int        # token ids in the frequency-counting stream
    zipf_s: float     # Zipf exponent of the id stream
    permute: bool     # whether rank -> id goes through a seeded permutation
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The pages' model shapes (FR-Spec notes: LLaMA-3-8B with a 128k vocabulary
# trimmed to 32k, Qwen-2-7B with 152k, LLaMA-3.2-1B) with synthetic inputs.
WORKLOADS = {
    "tiny": Workload("tiny", d=256, V=4096, V_high=1024, M=1, k=8,
                     n_ids=100_000, zipf_s=1.1, permute=False),
    "llama3_8b": Workload("llama3_8b", d=4096, V=128256, V_high=32768, M=1,
                          k=10, n_ids=100_000_000, zipf_s=1.0, permute=True),
    "eagle2_tree": Workload("eagle2_tree", d=4096, V=128256, V_high=32768,
                            M=60, k=10, n_ids=100_000_000, zipf_s=1.0,
                            permute=True),
    "qwen2_7b": Workload("qwen2_7b", d=3584, V=152064, V_high=32768, M=1,
                         k=10, n_ids=100_000_000, zipf_s=1.05, permute=True),
    "llama32_1b": Workload("llama32_1b", d=2048, V=128256, V_high=32768, M=1,
                           k=10, n_ids=100_000_000, zipf_s=1.0, permute=True),
}

# V_high points of the vocabulary-size sweep on the LLaMA-3-8B shape; the
# last one is the untrimmed head.
SWEEP_V_HIGH = (8192, 16384, 32768, 65536, 128256)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Inputs must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def streams(seed: int):
    """Four independent generators: ids, permutation, W, h."""
    ss = np.random.SeedSequence(seed).spawn(4)
    return tuple(np.random.Generator(np.random.PCG64(s)) for s in ss)


def zipf_ids(n: int, V: int, s: float, rng: np.random.Generator,
             perm: np.ndarray | None = None, chunk: int = 1 << 22) -> np.ndarray:
    """n ids from a finite Zipf law over ranks 1..V, as int32.

    Rank r (1-based) has probability r**-s / H_{V,s}. The sampled 0-based
    rank r-1 is the id itself, or ``perm[r-1]`` when a permutation is given.
    Drawn chunk by chunk so that 1e8 ids need little memory; the chunk size
    is fixed, so the stream is a pure function of (n, V, s, rng state).
    """
    w = np.arange(1, V + 1, dtype=np.float64) ** (-float(s))
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    out = np.empty(n, dtype=np.int32)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        u = rng.random(hi - lo)
        r = np.searchsorted(cdf, u, side="right")
        np.minimum(r, V - 1, out=r)
        out[lo:hi] = r if perm is None else perm[r]
    return out


def head_weights(V: int, d: int, rng: np.random.Generator, std: float = 0.02,
                 rows_per_chunk: int = 8192) -> np.ndarray:
    """bf16 bit patterns of W[V, d] ~ N(0, std), row-major."""
    out = np.empty((V, d), dtype=np.uint16)
    for lo in range(0, V, rows_per_chunk):
        hi = min(V, lo + rows_per_chunk)
        x = rng.standard_normal((hi - lo, d), dtype=np.float32)
        x *= np.float32(std)
        out[lo:hi] = bf16_bits_from_f32(x)
    return out


def hidden_states(M: int, d: int, rng: np.random.Generator,
                  scale: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of h[M, d] ~ N(0, 1) (times ``scale``), row-major.

    ``scale`` is applied in float32 before rounding; a power of two keeps the
    bf16 values an exact multiple of the unscaled ones.
    """
    x = rng.standard_normal((M, d), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_bits_from_f32(x)


@functools.lru_cache(maxsize=4)
def _ids_cached(n: int, V: int, s: float, permute: bool, seed: int) -> np.ndarray:
    g_ids, g_perm, _, _ = streams(seed)
    perm = g_perm.permutation(V).astype(np.int32) if permute else None
    return zipf_ids(n, V, s, g_ids, perm)


def make_ids(w: Workload, n: int | None = None) -> np.ndarray:
    """The workload's id stream (cached per process; do not modify it)."""
    return _ids_cached(int(w.n_ids if n is None else n), w.V, w.zipf_s,
                       w.permute, w.seed)


def permutation(w: Workload) -> np.ndarray | None:
    """The workload's rank -> id permutation (None when not permuted)."""
    if not w.permute:
        return None
    _, g_perm, _, _ = streams(w.seed)
    return g_perm.permutation(w.V).astype(np.int32)


def make_weights(w: Workload) -> np.ndarray:
    """The workload's full head W[V, d] (bf16 bits)."""
    _, _, g_w, _ = streams(w.seed)
    return head_weights(w.V, w.d, g_w)


def make_hidden(w: Workload, M: int | None = None, scale: float = 1.0) -> np.ndarray:
    """The workload's draft hidden states h[M, d] (bf16 bits)."""
    _, _, _, g_h = streams(w.seed)
    return hidden_states(int(w.M if M is None else M), w.d, g_h, scale)
