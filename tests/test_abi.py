"""The C-ABI library loads, exports every function vocabtrim.h declares, and
rejects bad arguments with the documented status before any HIP call (so
these run without a GPU: no call here reaches a kernel launch)."""
import ctypes as C
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "vocabtrim.h")
LIB = os.path.join(ROOT, "drafter_lm_head_amd", "libvocabtrim.so")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, -1, -2, -3, -4
P = C.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vt_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from drafter_lm_head_amd import build
        build.build()
    import drafter_lm_head_amd as dlh
    return dlh.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("vt_count_freq", "vt_select_vocab", "vt_gather_head", "vt_draft_head",
              "vt_head_logits", "vt_status_string", "vt_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(vt_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.vt_version() == 1
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, 12345):
        assert lib.vt_status_string(s)
    assert lib.vt_status_string(WORKSPACE) != lib.vt_status_string(INVALID)


# fake, never dereferenced device addresses: every call below fails validation
A = 0x7F0000000000          # 256-byte aligned
A16 = A + 16


def test_count_validation(lib):
    ws_n = lib.vt_count_freq_workspace_size(1000, 4096)
    assert ws_n > 0 and lib.vt_count_freq_workspace_size(1000, 0) == 0
    f = lib.vt_count_freq
    assert f(None, 10, 4096, A, 0, A, A, ws_n, None) == INVALID          # ids NULL
    assert f(A, 10, 0, A, 0, A, A, ws_n, None) == INVALID                # V = 0
    assert f(A, 2**32, 4096, A, 0, A, A, 10**12, None) == INVALID        # n too big
    assert f(A + 4, 10, 4096, A, 0, A, A, ws_n, None) == INVALID         # misaligned ids
    assert f(A, 10, 4096, None, 0, A, A, ws_n, None) == INVALID          # counts NULL
    assert f(A, 10, 4096, A, 0, None, A, ws_n, None) == INVALID          # n_invalid NULL
    assert f(A, 1000, 4096, A, 0, A, None, ws_n, None) == WORKSPACE
    assert f(A, 1000, 4096, A, 0, A, A + 16, ws_n, None) == WORKSPACE    # misaligned ws
    assert f(A, 1000, 4096, A, 0, A, A, ws_n - 1, None) == WORKSPACE


def test_select_validation(lib):
    n = lib.vt_select_vocab_workspace_size(4096, 1024)
    assert n > 0
    assert lib.vt_select_vocab_workspace_size(100, 101) == 0
    f = lib.vt_select_vocab
    assert f(A, 100, 101, A, A, A, A, A, 10**9, None) == INVALID         # V_high > V
    assert f(A, 100, 0, A, A, A, A, A, 10**9, None) == INVALID
    assert f(None, 100, 10, A, A, A, A, A, 10**9, None) == INVALID
    assert f(A + 4, 100, 10, A, A, A, A, A, 10**9, None) == INVALID     # misaligned counts
    assert f(A, 100, 10, None, A, A, A, A, 10**9, None) == INVALID
    assert f(A, 100, 10, A, A, None, A, A, 10**9, None) == INVALID
    assert f(A, 4096, 1024, A, None, A, A, A, n - 1, None) == WORKSPACE
    assert f(A, 4096, 1024, A, None, A, A, None, n, None) == WORKSPACE


def test_gather_validation(lib):
    f = lib.vt_gather_head
    far = A + (1 << 40)
    assert f(A, 100, 12, A, 10, far, None, None) == INVALID              # d % 8
    assert f(A, 100, 0, A, 10, far, None, None) == INVALID
    assert f(A, 100, 8200, A, 10, far, None, None) == INVALID            # d > VT_D_MAX
    assert f(A + 8, 100, 64, A, 10, far, None, None) == INVALID          # misaligned W
    assert f(A, 100, 64, A, 10, far + 2, None, None) == INVALID          # misaligned out
    assert f(A, 100, 64, A, 10, A + 64, None, None) == INVALID           # overlap
    assert f(None, 100, 64, A, 10, far, None, None) == INVALID
    assert f(A, 100, 64, None, 10, far, None, None) == INVALID
    assert f(A, 0, 64, A, 10, far, None, None) == INVALID


def test_draft_head_validation(lib):
    n = lib.vt_draft_head_workspace_size(1, 32768, 4096, 10)
    assert n > 0
    assert lib.vt_draft_head_workspace_size(513, 32768, 4096, 10) == 0
    assert lib.vt_draft_head_workspace_size(512, 32768, 4096, 10) > 0
    assert lib.vt_draft_head_workspace_size(1, 32768, 4096, 65) == 0
    f = lib.vt_draft_head
    args = dict(h=A, M=1, d=4096, W=A, V_high=32768, t2f=A, k=10, ids=A, probs=A,
                ws=A, ws_n=n)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["h"], a["M"], a["d"], a["W"], a["V_high"], a["t2f"], a["k"], a["ids"],
                 a["probs"], a["ws"], a["ws_n"], None)

    assert call(M=0) == INVALID
    assert call(M=513) == UNSUPPORTED
    assert call(d=4100) == INVALID
    assert call(d=8200) == INVALID
    assert call(V_high=0) == INVALID
    assert call(V_high=262145) == UNSUPPORTED
    assert call(k=0) == INVALID
    assert call(V_high=5, k=6) == INVALID
    assert call(k=65) == UNSUPPORTED
    assert call(h=A + 2) == INVALID
    assert call(W=A + 8) == INVALID
    assert call(h=None) == INVALID
    assert call(t2f=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(probs=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(ws=A16) == WORKSPACE
    assert call(ws_n=n - 1) == WORKSPACE


def test_head_logits_validation(lib):
    f = lib.vt_head_logits
    assert f(A, 1, 4096, A, 32768, None, None, None, None) == INVALID
    assert f(A, 1, 4096, A, 32768, None, A, A, None) == INVALID
    assert f(A, 0, 4096, A, 32768, A, None, None, None) == INVALID
    assert f(A, 1, 4095, A, 32768, A, None, None, None) == INVALID
    assert f(A, 513, 4096, A, 32768, A, A, A, None) == UNSUPPORTED


def test_draft_head_trimmed_validation(lib):
    n = lib.vt_draft_head_workspace_size(1, 32768, 4096, 10)
    f = lib.vt_draft_head_trimmed
    assert f(None, 1, 4096, A, 32768, 10, A, A, A, n, None) == INVALID
    assert f(A, 1, 4096, A, 32768, 10, None, A, A, n, None) == INVALID
    assert f(A, 1, 4096, A, 32768, 10, A, None, A, n, None) == INVALID
    assert f(A, 1, 4096, A, 32768, 0, A, A, A, n, None) == INVALID
    assert f(A, 1, 4096, A, 32768, 65, A, A, A, n, None) == UNSUPPORTED
    assert f(A, 1, 4096, A, 5, 6, A, A, A, n, None) == INVALID
    assert f(A, 1, 4096, A, 32768, 10, A, A, None, n, None) == WORKSPACE
    assert f(A, 1, 4096, A, 32768, 10, A, A, A, n - 1, None) == WORKSPACE


def test_noalloc_validation(lib):
    f = lib.vt_draft_head_noalloc
    assert f(None, 1, 4096, A, 32768, A, 10, A, A, None) == INVALID
    assert f(A, 1, 4096, A, 32768, None, 10, A, A, None) == INVALID
    assert f(A, 1, 4096, A, 32768, A, 10, None, A, None) == INVALID
    assert f(A, 1, 4096, A, 32768, A, 10, A, None, None) == INVALID
    assert f(A, 1, 4096, A, 32768, A, 0, A, A, None) == INVALID
    assert f(A, 1, 4096, A, 32768, A, 65, A, A, None) == UNSUPPORTED
    assert f(A, 513, 4096, A, 32768, A, 10, A, A, None) == UNSUPPORTED
    # beyond the fixed scratch: refused before any HIP call
    assert lib.vt_draft_head_workspace_size(512, 262144, 64, 10) > (16 << 20)
    assert f(A, 512, 64, A, 262144, A, 10, A, A, None) == -6
    assert lib.vt_status_string(-6) != lib.vt_status_string(-2)


def test_status_and_stream_read_validation(lib):
    f = lib.vt_stream_read
    assert f(None, 1024, A, None) == INVALID
    assert f(A, 1024, None, None) == INVALID
    assert f(A, 0, A, None) == INVALID
    assert f(A, 1000, A, None) == INVALID                              # not a multiple of 16
    assert f(A + 8, 1024, A, None) == INVALID                           # misaligned
    assert lib.vt_status_string(-5) != lib.vt_status_string(-4)


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import drafter_lm_head_amd as dlh
    with pytest.raises(TypeError):
        dlh.vt_count_freq(torch.zeros(4, dtype=torch.int32), 10)
    with pytest.raises(TypeError):
        dlh.vt_draft_head(torch.zeros((1, 8), dtype=torch.bfloat16),
                          torch.zeros((4, 8), dtype=torch.bfloat16),
                          torch.zeros(4, dtype=torch.int32), 2)


def test_draft_sample_validation(lib):
    n = lib.vt_draft_head_workspace_size(1, 32768, 4096, 1)
    f = lib.vt_draft_sample
    args = dict(h=A, M=1, d=4096, W=A, V_high=32768, t2f=A, seed=1, off=2, ids=A, probs=A,
                ws=A, ws_n=n)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["h"], a["M"], a["d"], a["W"], a["V_high"], a["t2f"], a["seed"], a["off"],
                 a["ids"], a["probs"], a["ws"], a["ws_n"], None)

    assert call(M=0) == INVALID
    assert call(M=513) == UNSUPPORTED
    assert call(d=4100) == INVALID
    assert call(V_high=0) == INVALID
    assert call(h=A + 2) == INVALID
    assert call(t2f=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(ws_n=n - 1) == WORKSPACE


def test_coverage_curve_validation(lib):
    assert lib.vt_coverage_curve_workspace_size(0, 1) == 0
    assert lib.vt_coverage_curve_workspace_size(10, 11) == 0
    n = lib.vt_coverage_curve_workspace_size(100000, 50000)
    assert n > 0
    f = lib.vt_coverage_curve
    assert f(None, 100, A, 10, 0.9, A, A, None, A, n, None) == INVALID
    assert f(A, 100, None, 10, 0.9, A, A, None, A, n, None) == INVALID
    assert f(A, 100, A, 101, 0.9, A, A, None, A, n, None) == INVALID
    assert f(A, 100, A, 10, 0.9, None, A, None, A, n, None) == INVALID
    assert f(A, 100, A, 10, 0.9, A, None, None, A, n, None) == INVALID
    assert f(A, 100000, A, 50000, 0.9, A, A, None, None, n, None) == WORKSPACE
    assert f(A, 100000, A, 50000, 0.9, A, A, None, A, n - 1, None) == WORKSPACE


def test_bias_entry_points_validation(lib):
    far = A + (1 << 40)
    g = lib.vt_gather_bias
    assert g(None, 100, A, 10, far, None, None) == INVALID
    assert g(A, 100, None, 10, far, None, None) == INVALID
    assert g(A, 100, A, 10, None, None, None) == INVALID
    assert g(A, 0, A, 10, far, None, None) == INVALID
    assert g(A, 100, A, 0, far, None, None) == INVALID
    assert g(A, 100, A, 10, A + 100, None, None) == INVALID              # overlap
    n = lib.vt_draft_head_workspace_size(3, 32768, 4096, 10)
    hb = lib.vt_draft_head_bias
    assert hb(A, 3, 4096, A, None, 32768, A, 10, A, A, A, n, None) == INVALID   # no bias
    assert hb(A, 3, 4096, A, A, 32768, A, 0, A, A, A, n, None) == INVALID
    assert hb(A, 513, 4096, A, A, 32768, A, 10, A, A, A, n, None) == UNSUPPORTED
    assert hb(A, 3, 4096, A, A, 32768, A, 10, A, A, A, n - 1, None) == WORKSPACE
    assert hb(A + 2, 3, 4096, A, A, 32768, A, 10, A, A, A, n, None) == INVALID
    n1 = lib.vt_draft_head_workspace_size(3, 32768, 4096, 1)
    sb = lib.vt_draft_sample_bias
    assert sb(A, 3, 4096, A, None, 32768, A, 1, 2, A, A, A, n1, None) == INVALID
    assert sb(A, 3, 4096, A, A, 32768, None, 1, 2, A, A, A, n1, None) == INVALID
    assert sb(A, 3, 4096, A, A, 32768, A, 1, 2, A, A, None, n1, None) == WORKSPACE
    assert sb(A, 3, 4096, A, A, 32768, A, 1, 2, A, A, A, n1 - 1, None) == WORKSPACE


def test_vocabulary_limit(lib):
    # past VT_V_MAX ids the sizing functions give 0 and the calls refuse
    import drafter_lm_head_amd as dlh
    big = dlh.VT_V_MAX + 1
    f = lib.vt_count_freq_workspace_size
    assert f(1000, dlh.VT_V_MAX) > 0 and f(1000, big) == 0
    assert lib.vt_select_vocab_workspace_size(big, 10) == 0
    assert lib.vt_coverage_curve_workspace_size(big, 10) == 0
    assert lib.vt_count_freq(A, 1000, big, A, 0, A, A, 1 << 40, None) == UNSUPPORTED
    assert lib.vt_select_vocab(A, big, 10, A, A, A, A, A, 1 << 40, None) == UNSUPPORTED
    assert lib.vt_coverage_curve(A, big, A, 10, C.c_double(0.9), A, A, A, A, 1 << 40,
                                 None) == UNSUPPORTED
    assert lib.vt_gather_head(A, big, 64, A, 10, A + (1 << 40), None, None) == UNSUPPORTED
    assert lib.vt_gather_bias(A, big, A, 10, A + (1 << 40), None, None) == UNSUPPORTED
