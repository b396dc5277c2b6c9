"""Python binding of libvocabtrim, the gfx950 frequency-ranked drafter head.

Argument marshalling only: every step runs in the HIP library declared in
``include/vocabtrim.h``. torch supplies device memory and the current
stream. The functions keep the C names:

* ``vt_count_freq(ids, V)``            -> (counts uint32[V], n_invalid)
* ``vt_select_vocab(counts, V_high)``  -> (t2f, f2t, sel_sum, tot_sum)
* ``vt_gather_head(W, t2f)``           -> W_trim
* ``vt_gather_bias(b, t2f)``           -> b_trim (heads with a bias)
* ``vt_draft_head(h, W_trim, t2f, k)`` -> (full_ids int32[M, k], probs f32[M, k])
* ``vt_draft_head_bias(h, W_trim, bias, t2f, k)``, ``vt_draft_sample(...)``,
  ``vt_draft_sample_bias(...)``: the same with a bias, or one draw per row
* ``vt_head_logits(h, W_trim)``        -> logits f32[M, V_high] (checks only),
  with ``stats=True`` also (row_max f32[M], row_sum f32[M])
* ``vt_draft_head_trimmed(h, W_trim, k)`` -> (trimmed_ids, probs): the draft
  step without the remap (measures the remap's cost)
* ``vt_draft_head_noalloc(h, W_trim, t2f, k)``: vt_draft_head on the
  library's fixed per-GPU scratch (no workspace, no device allocation inside)
* ``vt_draft_head_status(ws)``         -> raises VtError if a bounded wait in a
  kernel gave up since the last query (host-blocking)
* ``vt_stream_read(buf)``              : a plain streaming read of a buffer
  (the draft head's practical bandwidth ceiling)

bfloat16 arrays may be passed as ``torch.bfloat16`` or as their 16-bit
patterns (``torch.int16`` / ``torch.uint16``). Results stay on the device;
nothing here synchronises with the host. If the library is missing the
calls raise: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

__all__ = [
    "VtError", "lib", "lib_path", "VT_K_MAX", "VT_M_MAX", "VT_D_MAX",
    "VT_VHIGH_MAX", "VT_V_MAX", "vt_count_freq", "vt_select_vocab", "vt_gather_head",
    "vt_draft_head", "vt_draft_sample", "vt_head_logits", "vt_count_freq_workspace_size",
    "vt_gather_bias", "vt_draft_head_bias", "vt_draft_sample_bias",
    "vt_select_vocab_workspace_size", "vt_draft_head_workspace_size",
    "coverage", "vt_coverage_curve", "vt_coverage_curve_workspace_size",
    "vt_draft_head_trimmed", "vt_draft_head_status", "vt_stream_read",
    "vt_draft_head_noalloc", "VT_NOALLOC_WS_BYTES", "VT_ERR_SCRATCH_LIMIT",
    "VT_WS_ERROR_OFFSET", "VT_WS_HOLD_OFFSET", "VT_WS_SPIN_LIMIT_OFFSET",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libvocabtrim.so")

VT_OK, VT_ERR_INVALID_ARG, VT_ERR_UNSUPPORTED, VT_ERR_WORKSPACE, VT_ERR_HIP = 0, -1, -2, -3, -4
VT_ERR_TIMEOUT, VT_ERR_SCRATCH_LIMIT = -5, -6
VT_NOALLOC_WS_BYTES = 16 << 20
VT_K_MAX, VT_M_MAX, VT_D_MAX, VT_VHIGH_MAX, VT_V_MAX = 64, 512, 8192, 262144, 1 << 26
VT_WS_ERROR_OFFSET, VT_WS_HOLD_OFFSET, VT_WS_SPIN_LIMIT_OFFSET = 128, 132, 136

_lock = threading.Lock()
_lib = None

_P, _I32, _U64, _SZ, _INT = C.c_void_p, C.c_int32, C.c_uint64, C.c_size_t, C.c_int
_SIGS = {
    "vt_status_string": (C.c_char_p, [_INT]),
    "vt_version": (_INT, []),
    "vt_count_freq_workspace_size": (_SZ, [_U64, _I32]),
    "vt_count_freq": (_INT, [_P, _U64, _I32, _P, _INT, _P, _P, _SZ, _P]),
    "vt_select_vocab_workspace_size": (_SZ, [_I32, _I32]),
    "vt_select_vocab": (_INT, [_P, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "vt_gather_head": (_INT, [_P, _I32, _I32, _P, _I32, _P, _P, _P]),
    "vt_draft_head_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
    "vt_draft_head": (_INT, [_P, _I32, _I32, _P, _I32, _P, _I32, _P, _P, _P, _SZ, _P]),
    "vt_draft_sample": (_INT, [_P, _I32, _I32, _P, _I32, _P, _U64, _U64, _P, _P, _P, _SZ, _P]),
    "vt_gather_bias": (_INT, [_P, _I32, _P, _I32, _P, _P, _P]),
    "vt_draft_head_bias": (_INT, [_P, _I32, _I32, _P, _P, _I32, _P, _I32, _P, _P, _P, _SZ, _P]),
    "vt_draft_sample_bias": (_INT, [_P, _I32, _I32, _P, _P, _I32, _P, _U64, _U64, _P, _P, _P, _SZ,
                                    _P]),
    "vt_head_logits": (_INT, [_P, _I32, _I32, _P, _I32, _P, _P, _P, _P]),
    "vt_draft_head_trimmed": (_INT, [_P, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "vt_draft_head_status": (_INT, [_P, _P]),
    "vt_draft_head_noalloc": (_INT, [_P, _I32, _I32, _P, _I32, _P, _I32, _P, _P, _P]),
    "vt_stream_read": (_INT, [_P, _SZ, _P, _P]),
    "vt_coverage_curve_workspace_size": (_SZ, [_I32, _I32]),
    "vt_coverage_curve": (_INT, [_P, _I32, _P, _I32, C.c_double, _P, _P, _P, _P, _SZ, _P]),
}


class VtError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().vt_status_string(status).decode()} (status {status})")


def lib():
    """The loaded library (ctypes handle). Raises if it was not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(lib_path):
                raise RuntimeError(
                    f"{lib_path} is missing: build it with python -m drafter_lm_head_amd.build "
                    "(hipcc, gfx950); there is no fallback implementation")
            h = C.CDLL(lib_path)
            for name, (res, args) in _SIGS.items():
                f = getattr(h, name)
                f.restype, f.argtypes = res, args
            _lib = h
    return _lib


def _check(status: int, what: str):
    if status != VT_OK:
        raise VtError(status, what)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int | None = None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-d, got shape {tuple(t.shape)}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)

# Cached workspaces, one per (device, stream, kind), grown on demand. Keyed by
# stream because calls that share a workspace must run in stream order; a
# buffer replaced by a larger one is released to torch's caching allocator,
# which reuses it only in the order of that same stream. The draft-head
# workspace is zero-filled when allocated, as the C ABI requires.
_ws_cache: dict = {}


def _workspace(device: torch.device, kind: str, nbytes: int, zero: bool) -> torch.Tensor:
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError(f"pass an explicit {kind} workspace (ws=...) when capturing a graph: "
                           "an implicit one may be reallocated after the capture")
    stream = torch.cuda.current_stream(device).cuda_stream
    key = (device.index, stream, kind)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        n = max(nbytes, 256)
        ws = (torch.zeros if zero else torch.empty)(n, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def vt_count_freq_workspace_size(n: int, V: int) -> int:
    return int(lib().vt_count_freq_workspace_size(n, V))


def vt_select_vocab_workspace_size(V: int, V_high: int) -> int:
    return int(lib().vt_select_vocab_workspace_size(V, V_high))


def vt_draft_head_workspace_size(M: int, V_high: int, d: int, k: int) -> int:
    return int(lib().vt_draft_head_workspace_size(M, V_high, d, k))


def vt_count_freq(ids: torch.Tensor, V: int, counts: torch.Tensor | None = None,
                  n_invalid: torch.Tensor | None = None, accumulate: bool = False,
                  ws: torch.Tensor | None = None):
    """Histogram of token ids (VocabTrim Step 1). Returns (counts, n_invalid)."""
    _dev(ids, "ids", (torch.int32,), 1)
    dev = ids.device
    if counts is None:
        if accumulate:
            raise ValueError("accumulate needs existing counts")
        counts = torch.empty(V, dtype=torch.int32, device=dev).view(torch.uint32)
    if n_invalid is None:
        if accumulate:
            raise ValueError("accumulate needs an existing n_invalid")
        n_invalid = torch.empty(1, dtype=torch.int64, device=dev).view(torch.uint64)
    _dev(counts, "counts", (torch.uint32, torch.int32), 1)
    _dev(n_invalid, "n_invalid", (torch.uint64, torch.int64), 1)
    n = ids.numel()
    need = vt_count_freq_workspace_size(n, V)
    ws = ws if ws is not None else _workspace(dev, "count", need, False)
    _check(lib().vt_count_freq(_ptr(ids) if n else None, n, V, _ptr(counts), int(bool(accumulate)),
                               _ptr(n_invalid), _ptr(ws), ws.numel(), _stream(ids)),
           "vt_count_freq")
    return counts, n_invalid


def vt_select_vocab(counts: torch.Tensor, V_high: int, want_f2t: bool = True,
                    ws: torch.Tensor | None = None):
    """Top-V_high ids by (count desc, id asc) (VocabTrim Step 2).

    Returns device tensors (t2f int32[V_high], f2t int32[V] or None,
    sel_sum uint64[1], tot_sum uint64[1]).
    """
    _dev(counts, "counts", (torch.uint32, torch.int32), 1)
    dev = counts.device
    V = counts.numel()
    t2f = torch.empty(V_high, dtype=torch.int32, device=dev)
    f2t = torch.empty(V, dtype=torch.int32, device=dev) if want_f2t else None
    sums = torch.empty(2, dtype=torch.int64, device=dev).view(torch.uint64)
    need = vt_select_vocab_workspace_size(V, V_high)
    ws = ws if ws is not None else _workspace(dev, "select", need, False)
    _check(lib().vt_select_vocab(_ptr(counts), V, V_high, _ptr(t2f), _ptr(f2t),
                                 _ptr(sums[0:1]), _ptr(sums[1:2]), _ptr(ws), ws.numel(),
                                 _stream(counts)), "vt_select_vocab")
    return t2f, f2t, sums[0:1], sums[1:2]


def coverage(sel_sum: torch.Tensor, tot_sum: torch.Tensor) -> float:
    """sel / tot on the host (synchronises); NaN when nothing was counted."""
    s = int(sel_sum.view(torch.int64).item())
    t = int(tot_sum.view(torch.int64).item())
    return float("nan") if t == 0 else s / t


def vt_gather_head(W: torch.Tensor, t2f: torch.Tensor, out: torch.Tensor | None = None,
                   n_bad: torch.Tensor | None = None) -> torch.Tensor:
    """W_trim = W[t2f] (VocabTrim Step 3)."""
    _dev(W, "W", _BF16, 2)
    _dev(t2f, "t2f", (torch.int32,), 1)
    V, d = W.shape
    V_high = t2f.numel()
    if out is None:
        out = torch.empty((V_high, d), dtype=W.dtype, device=W.device)
    _dev(out, "out", _BF16, 2)
    if tuple(out.shape) != (V_high, d):
        raise ValueError("out must be [V_high, d]")
    if n_bad is not None:
        _dev(n_bad, "n_bad", (torch.int32, torch.uint32), 1)
    _check(lib().vt_gather_head(_ptr(W), V, d, _ptr(t2f), V_high, _ptr(out), _ptr(n_bad),
                                _stream(W)), "vt_gather_head")
    return out


def vt_gather_bias(b: torch.Tensor, t2f: torch.Tensor, out: torch.Tensor | None = None,
                   n_bad: torch.Tensor | None = None) -> torch.Tensor:
    """b_trim = b[t2f], the bias of a trimmed head (VocabTrim Step 3)."""
    _dev(b, "b", _BF16, 1)
    _dev(t2f, "t2f", (torch.int32,), 1)
    V, V_high = b.numel(), t2f.numel()
    if out is None:
        out = torch.empty(V_high, dtype=b.dtype, device=b.device)
    _dev(out, "out", _BF16, 1)
    if out.numel() != V_high:
        raise ValueError("out must hold V_high entries")
    if n_bad is not None:
        _dev(n_bad, "n_bad", (torch.int32, torch.uint32), 1)
    _check(lib().vt_gather_bias(_ptr(b), V, _ptr(t2f), V_high, _ptr(out), _ptr(n_bad),
                                _stream(b)), "vt_gather_bias")
    return out


def _head_shapes(h, W_trim, t2f, bias):
    _dev(h, "h", _BF16, 2)
    _dev(W_trim, "W_trim", _BF16, 2)
    _dev(t2f, "t2f", (torch.int32,), 1)
    M, d = h.shape
    V_high = W_trim.shape[0]
    if W_trim.shape[1] != d or t2f.numel() != V_high:
        raise ValueError("shape mismatch between h, W_trim and t2f")
    if bias is not None:
        _dev(bias, "bias", _BF16, 1)
        if bias.numel() != V_high:
            raise ValueError("bias must hold V_high entries")
    return M, d, V_high


def vt_draft_head(h: torch.Tensor, W_trim: torch.Tensor, t2f: torch.Tensor, k: int,
                  full_ids: torch.Tensor | None = None, probs: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None):
    """One draft step (VocabTrim Step 4): (full_ids[M, k], probs[M, k])."""
    return _draft_head(h, W_trim, None, t2f, k, full_ids, probs, ws)


def vt_draft_head_bias(h: torch.Tensor, W_trim: torch.Tensor, bias: torch.Tensor,
                       t2f: torch.Tensor, k: int, full_ids: torch.Tensor | None = None,
                       probs: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """vt_draft_head for a trimmed head with a bias bf16[V_high]."""
    return _draft_head(h, W_trim, bias, t2f, k, full_ids, probs, ws)


def _draft_head(h, W_trim, bias, t2f, k, full_ids, probs, ws):
    M, d, V_high = _head_shapes(h, W_trim, t2f, bias)
    dev = h.device
    if full_ids is None:
        full_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    if probs is None:
        probs = torch.empty((M, k), dtype=torch.float32, device=dev)
    _dev(full_ids, "full_ids", (torch.int32,))
    _dev(probs, "probs", (torch.float32,))
    if full_ids.numel() != M * k or probs.numel() != M * k:
        raise ValueError("outputs must hold M * k entries")
    if ws is None:
        need = vt_draft_head_workspace_size(M, V_high, d, k)
        ws = _workspace(dev, "head", need, True)
    if bias is None:
        _check(lib().vt_draft_head(_ptr(h), M, d, _ptr(W_trim), V_high, _ptr(t2f), k,
                                   _ptr(full_ids), _ptr(probs), _ptr(ws), ws.numel(),
                                   _stream(h)), "vt_draft_head")
    else:
        _check(lib().vt_draft_head_bias(_ptr(h), M, d, _ptr(W_trim), _ptr(bias), V_high,
                                        _ptr(t2f), k, _ptr(full_ids), _ptr(probs), _ptr(ws),
                                        ws.numel(), _stream(h)), "vt_draft_head_bias")
    return full_ids, probs


def vt_draft_sample(h: torch.Tensor, W_trim: torch.Tensor, t2f: torch.Tensor, seed: int,
                    offset: int, full_ids: torch.Tensor | None = None,
                    probs: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """One sampled draft token per row (VocabTrim Step 4's multinomial draw,
    remapped): (full_ids[M], probs[M])."""
    return _draft_sample(h, W_trim, None, t2f, seed, offset, full_ids, probs, ws)


def vt_draft_sample_bias(h: torch.Tensor, W_trim: torch.Tensor, bias: torch.Tensor,
                         t2f: torch.Tensor, seed: int, offset: int,
                         full_ids: torch.Tensor | None = None,
                         probs: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """vt_draft_sample for a trimmed head with a bias bf16[V_high]."""
    return _draft_sample(h, W_trim, bias, t2f, seed, offset, full_ids, probs, ws)


def _draft_sample(h, W_trim, bias, t2f, seed, offset, full_ids, probs, ws):
    M, d, V_high = _head_shapes(h, W_trim, t2f, bias)
    dev = h.device
    if full_ids is None:
        full_ids = torch.empty(M, dtype=torch.int32, device=dev)
    if probs is None:
        probs = torch.empty(M, dtype=torch.float32, device=dev)
    _dev(full_ids, "full_ids", (torch.int32,))
    _dev(probs, "probs", (torch.float32,))
    if full_ids.numel() != M or probs.numel() != M:
        raise ValueError("outputs must hold M entries")
    if ws is None:
        need = vt_draft_head_workspace_size(M, V_high, d, 1)
        ws = _workspace(dev, "head", need, True)
    seed, offset = int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1)
    if bias is None:
        _check(lib().vt_draft_sample(_ptr(h), M, d, _ptr(W_trim), V_high, _ptr(t2f), seed,
                                     offset, _ptr(full_ids), _ptr(probs), _ptr(ws), ws.numel(),
                                     _stream(h)), "vt_draft_sample")
    else:
        _check(lib().vt_draft_sample_bias(_ptr(h), M, d, _ptr(W_trim), _ptr(bias), V_high,
                                          _ptr(t2f), seed, offset, _ptr(full_ids), _ptr(probs),
                                          _ptr(ws), ws.numel(), _stream(h)),
               "vt_draft_sample_bias")
    return full_ids, probs


def vt_head_logits(h: torch.Tensor, W_trim: torch.Tensor,
                   out: torch.Tensor | None = None, stats: bool = False):
    """fp32 trimmed logits [M, V_high] (parity diagnostics); with
    ``stats=True`` returns (logits, row_max[M], row_sum[M]), the subset
    softmax statistics of each row."""
    _dev(h, "h", _BF16, 2)
    _dev(W_trim, "W_trim", _BF16, 2)
    M, d = h.shape
    V_high = W_trim.shape[0]
    if W_trim.shape[1] != d:
        raise ValueError("shape mismatch between h and W_trim")
    if out is None:
        out = torch.empty((M, V_high), dtype=torch.float32, device=h.device)
    _dev(out, "out", (torch.float32,))
    if out.numel() != M * V_high:
        raise ValueError("out must hold M * V_high entries")
    rmax = torch.empty(M, dtype=torch.float32, device=h.device) if stats else None
    rsum = torch.empty(M, dtype=torch.float32, device=h.device) if stats else None
    _check(lib().vt_head_logits(_ptr(h), M, d, _ptr(W_trim), V_high, _ptr(out), _ptr(rmax),
                                _ptr(rsum), _stream(h)), "vt_head_logits")
    return (out, rmax, rsum) if stats else out


def vt_draft_head_trimmed(h: torch.Tensor, W_trim: torch.Tensor, k: int,
                          trimmed_ids: torch.Tensor | None = None,
                          probs: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """The draft step without the remap: (trimmed_ids[M, k], probs[M, k])."""
    _dev(h, "h", _BF16, 2)
    _dev(W_trim, "W_trim", _BF16, 2)
    M, d = h.shape
    V_high = W_trim.shape[0]
    if W_trim.shape[1] != d:
        raise ValueError("shape mismatch between h and W_trim")
    dev = h.device
    if trimmed_ids is None:
        trimmed_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    if probs is None:
        probs = torch.empty((M, k), dtype=torch.float32, device=dev)
    _dev(trimmed_ids, "trimmed_ids", (torch.int32,))
    _dev(probs, "probs", (torch.float32,))
    if trimmed_ids.numel() != M * k or probs.numel() != M * k:
        raise ValueError("outputs must hold M * k entries")
    if ws is None:
        ws = _workspace(dev, "head", vt_draft_head_workspace_size(M, V_high, d, k), True)
    _check(lib().vt_draft_head_trimmed(_ptr(h), M, d, _ptr(W_trim), V_high, k,
                                       _ptr(trimmed_ids), _ptr(probs), _ptr(ws), ws.numel(),
                                       _stream(h)), "vt_draft_head_trimmed")
    return trimmed_ids, probs


def vt_draft_head_noalloc(h: torch.Tensor, W_trim: torch.Tensor, t2f: torch.Tensor, k: int,
                          full_ids: torch.Tensor | None = None,
                          probs: torch.Tensor | None = None):
    """vt_draft_head on the library's fixed per-GPU scratch: the C call takes
    no workspace and allocates nothing (pass ``full_ids`` and ``probs`` to
    allocate nothing here either, e.g. under graph capture)."""
    M, d, V_high = _head_shapes(h, W_trim, t2f, None)
    dev = h.device
    if full_ids is None:
        full_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    if probs is None:
        probs = torch.empty((M, k), dtype=torch.float32, device=dev)
    _dev(full_ids, "full_ids", (torch.int32,))
    _dev(probs, "probs", (torch.float32,))
    if full_ids.numel() != M * k or probs.numel() != M * k:
        raise ValueError("outputs must hold M * k entries")
    _check(lib().vt_draft_head_noalloc(_ptr(h), M, d, _ptr(W_trim), V_high, _ptr(t2f), k,
                                       _ptr(full_ids), _ptr(probs), _stream(h)),
           "vt_draft_head_noalloc")
    return full_ids, probs


def vt_draft_head_status(ws: torch.Tensor | None, device: torch.device | None = None) -> None:
    """Raises VtError(VT_ERR_TIMEOUT) if a bounded wait inside a kernel that
    used this draft-head workspace (None: the library's own scratch of
    vt_draft_head_noalloc on ``device``) gave up since the last query,
    clearing the flag. Blocks the host until the stream's work is done."""
    if ws is None:
        dev = torch.device(device if device is not None else "cuda")
        with torch.cuda.device(dev):
            st = lib().vt_draft_head_status(None, torch.cuda.current_stream(dev).cuda_stream)
        _check(st, "vt_draft_head_status")
        return
    _dev(ws, "ws", (torch.uint8,), 1)
    _check(lib().vt_draft_head_status(_ptr(ws), _stream(ws)), "vt_draft_head_status")


def vt_stream_read(buf: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """A plain streaming read of ``buf`` (16-byte aligned, size a multiple of
    16 bytes): the practical ceiling of the draft head."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int64, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().vt_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf)), "vt_stream_read")
    return sink


def vt_coverage_curve_workspace_size(V: int, L: int) -> int:
    return int(lib().vt_coverage_curve_workspace_size(V, L))


def vt_coverage_curve(counts: torch.Tensor, order: torch.Tensor, min_coverage: float = 1.0):
    """Cumulative counts along a ranking and the smallest prefix reaching a
    coverage threshold (VocabTrim Step 2 coverage for every V_high; guidance
    table threshold): (cum uint64[L], tot_sum uint64[1], v_high int32[1])."""
    _dev(counts, "counts", (torch.uint32, torch.int32), 1)
    _dev(order, "order", (torch.int32,), 1)
    V, L = counts.numel(), order.numel()
    dev = counts.device
    cum = torch.empty(L, dtype=torch.int64, device=dev).view(torch.uint64)
    tot = torch.empty(1, dtype=torch.int64, device=dev).view(torch.uint64)
    vh = torch.empty(1, dtype=torch.int32, device=dev)
    need = vt_coverage_curve_workspace_size(V, L)
    if need == 0:
        raise ValueError("need 1 <= len(order) <= len(counts)")
    ws = _workspace(dev, "coverage", need, False)
    _check(lib().vt_coverage_curve(_ptr(counts), V, _ptr(order), L, float(min_coverage),
                                   _ptr(cum), _ptr(tot), _ptr(vh), _ptr(ws), ws.numel(),
                                   _stream(counts)), "vt_coverage_curve")
    return cum, tot, vh
