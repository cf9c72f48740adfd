"""The C-ABI library loads, exports what include/attn.h declares, and rejects
bad arguments on the host (no GPU needed: validation runs before any HIP call)."""
import ctypes
import os
import re

import pytest

from exact_softmax_attention_amd import _lib
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = 0x1000  # a non-NULL pointer that is never dereferenced: every call below fails validation


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert declared == sorted(_lib.SIGNATURES)
    lib = ctypes.CDLL(_lib.library_path())
    for name in declared:
        assert hasattr(lib, name), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name in ("ATTN_OK", "ATTN_E_NULL", "ATTN_E_SHAPE", "ATTN_E_HEADDIM", "ATTN_E_MASK",
                 "ATTN_E_WORKSPACE", "ATTN_E_LAUNCH"):
        val = int(re.search(rf"\b{name}\s*=\s*(-?\d+)", text).group(1))
        assert getattr(_lib, name) == val
        assert _lib.status_str(val)
    assert _lib.status_str(12345) == "unknown status"


def _fwd(fn="attn_fwd", ptr=FAKE, lse=None, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0,
         window=0):
    return getattr(_lib.lib(), fn)(ptr, ptr, ptr, ptr, lse, B, Hq, Hkv, Nq, Nk, d, causal,
                                   window, 0.125, None)


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_fwd_validation(fn):
    assert _fwd(fn, ptr=None) == _lib.ATTN_E_NULL
    assert _fwd(fn, Hq=3, Hkv=2) == _lib.ATTN_E_SHAPE          # Hq % Hkv
    assert _fwd(fn, Hkv=0) == _lib.ATTN_E_SHAPE
    assert _fwd(fn, B=-1) == _lib.ATTN_E_SHAPE
    assert _fwd(fn, Nq=-1) == _lib.ATTN_E_SHAPE
    assert _fwd(fn, d=96) == _lib.ATTN_E_HEADDIM
    assert _fwd(fn, d=256) == _lib.ATTN_E_HEADDIM
    assert _fwd(fn, window=4) == _lib.ATTN_E_MASK               # window needs causal
    assert _fwd(fn, causal=2) == _lib.ATTN_E_MASK
    assert _fwd(fn, causal=1, Nq=9, Nk=8) == _lib.ATTN_E_SHAPE  # causal with Nq > Nk
    assert _fwd(fn, B=1 << 20, Hq=1 << 10, Nq=1 << 20) == _lib.ATTN_E_SHAPE  # grid too large
    # empty problems are accepted without touching memory (no launch happens)
    assert _fwd(fn, ptr=None, B=0) == _lib.ATTN_OK
    assert _fwd(fn, ptr=None, Nq=0, Nk=0) == _lib.ATTN_OK


def test_decode_workspace_size():
    L = _lib.lib()
    n = L.attn_decode_paged_workspace_size(16, 32, 128, 16, 2000)
    # per query head: one (m, l) pair and d floats for each of up to 512 block
    # ranges plus one per sequence (a range may end inside a sequence), and a
    # (first, last) range pair per sequence
    slots = 32 * (512 + 16)
    assert n >= slots * (128 * 4 + 8) + 16 * 8
    assert n < slots * (128 * 4 + 8) + 16 * 8 + 1024
    assert L.attn_decode_paged_workspace_size(16, 32, 128, 32, 2000) == 0   # block size
    assert L.attn_decode_paged_workspace_size(16, 32, 96, 16, 2000) == 0    # head dim
    assert L.attn_decode_paged_workspace_size(16, 32, 64, 16, 0) == 0


def _dec(ptr=FAKE, B=2, Hq=8, Hkv=2, d=128, bs=16, maxb=10, nb=100, window=0, ws=FAKE,
         ws_bytes=1 << 30):
    return _lib.lib().attn_decode_paged(ptr, ptr, ptr, ptr, ptr, ptr, None, B, Hq, Hkv, d, bs,
                                        maxb, nb, window, 0.1, ws, ws_bytes, None)


def test_decode_validation():
    assert _dec(ptr=None) == _lib.ATTN_E_NULL
    assert _dec(Hq=6, Hkv=4) == _lib.ATTN_E_SHAPE
    assert _dec(d=32) == _lib.ATTN_E_HEADDIM
    assert _dec(bs=8) == _lib.ATTN_E_SHAPE
    assert _dec(maxb=0) == _lib.ATTN_E_SHAPE
    assert _dec(nb=0) == _lib.ATTN_E_SHAPE
    assert _dec(ws=None) == _lib.ATTN_E_WORKSPACE
    need = _lib.lib().attn_decode_paged_workspace_size(2, 8, 128, 16, 10)
    assert _dec(ws_bytes=need - 1) == _lib.ATTN_E_WORKSPACE
    assert _dec(B=65535, maxb=40000) == _lib.ATTN_E_SHAPE  # batch block count beyond int32
    assert _dec(B=65536) == _lib.ATTN_E_SHAPE
    assert _dec(ptr=None, B=0) == _lib.ATTN_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib.lib()


def _bwd(ptr=FAKE, lse=FAKE, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0, window=0,
         ws=FAKE, ws_bytes=1 << 20):
    return _lib.lib().attn_bwd(ptr, ptr, ptr, ptr, ptr, lse, ptr, ptr, ptr, B, Hq, Hkv, Nq, Nk,
                               d, causal, window, 0.125, ws, ws_bytes, None)


def test_bwd_workspace_size():
    L = _lib.lib()
    n = L.attn_bwd_workspace_size(2, 4, 1000)
    assert n >= 2 * 2 * 4 * 1000 * 4 and n % 256 == 0
    assert L.attn_bwd_workspace_size(-1, 4, 10) == 0
    assert L.attn_bwd_workspace_size(1, 0, 10) == 0


def test_bwd_validation():
    assert _bwd(ptr=None) == _lib.ATTN_E_NULL
    assert _bwd(lse=None) == _lib.ATTN_E_NULL
    assert _bwd(Hq=3, Hkv=2) == _lib.ATTN_E_SHAPE
    assert _bwd(d=96) == _lib.ATTN_E_HEADDIM
    assert _bwd(window=4) == _lib.ATTN_E_MASK
    assert _bwd(causal=1, Nq=9, Nk=8) == _lib.ATTN_E_SHAPE
    assert _bwd(B=70000) == _lib.ATTN_E_SHAPE
    assert _bwd(ws=None) == _lib.ATTN_E_WORKSPACE
    assert _bwd(ws_bytes=16) == _lib.ATTN_E_WORKSPACE
    assert _bwd(ptr=None, lse=None, B=0) == _lib.ATTN_OK


def _varlen(ptr=1 << 20, cu=1 << 21, n=3, tq=100, tk=120, Hq=8, Hkv=2, d=128, causal=1, window=0):
    return _lib.lib().attn_fwd_varlen(ptr, ptr, ptr, ptr, None, cu, cu, n, tq, tk, Hq, Hkv, d,
                                      causal, window, 0.1, None)


def test_varlen_validation():
    # every rejection happens on the host, before any HIP call
    assert _varlen(ptr=None) == _lib.ATTN_E_NULL
    assert _varlen(cu=None) == _lib.ATTN_E_NULL
    assert _varlen(n=-1) == _lib.ATTN_E_SHAPE
    assert _varlen(tq=-1) == _lib.ATTN_E_SHAPE
    assert _varlen(Hq=3, Hkv=2) == _lib.ATTN_E_SHAPE
    assert _varlen(d=80) == _lib.ATTN_E_HEADDIM
    assert _varlen(causal=0, window=5) == _lib.ATTN_E_MASK
    assert _varlen(causal=2) == _lib.ATTN_E_MASK
    assert _varlen(Hq=1 << 16, Hkv=1, n=1 << 15) == _lib.ATTN_E_SHAPE  # schedule size
    # empty problems are no-ops whatever the pointers
    assert _varlen(ptr=None, cu=None, n=0) == _lib.ATTN_OK
    assert _varlen(ptr=None, cu=None, tq=0) == _lib.ATTN_OK


def _prefill(ptr=1 << 20, n=3, tq=100, Hq=8, Hkv=2, d=128, bs=16, mb=8, nb=40, window=0,
             ws=None, ws_bytes=0):
    return _lib.lib().attn_prefill_paged(ptr, ptr, ptr, ptr, ptr, ptr, ptr, None, n, tq, Hq,
                                         Hkv, d, bs, mb, nb, window, 0.1, ws, ws_bytes, None)


def test_prefill_paged_validation():
    assert _prefill(ptr=None) == _lib.ATTN_E_NULL
    assert _prefill(n=-1) == _lib.ATTN_E_SHAPE
    assert _prefill(Hq=6, Hkv=4) == _lib.ATTN_E_SHAPE
    assert _prefill(d=32) == _lib.ATTN_E_HEADDIM
    assert _prefill(bs=32) == _lib.ATTN_E_SHAPE
    assert _prefill(mb=0) == _lib.ATTN_E_SHAPE
    assert _prefill(nb=0) == _lib.ATTN_E_SHAPE
    assert _prefill(n=1 << 20, mb=1 << 12) == _lib.ATTN_E_SHAPE   # table entries
    assert _prefill(ptr=None, n=0) == _lib.ATTN_OK
    assert _prefill(ptr=None, tq=0) == _lib.ATTN_OK
    # a table longer than one 8192-key chunk needs the partial-result workspace
    assert _prefill(mb=600) == _lib.ATTN_E_WORKSPACE
    need = _lib.lib().attn_prefill_paged_workspace_size(3, 100, 8, 128, 16, 600)
    assert _prefill(mb=600, ws=1 << 20, ws_bytes=need - 1) == _lib.ATTN_E_WORKSPACE


def test_prefill_paged_workspace_size():
    ws = _lib.lib().attn_prefill_paged_workspace_size
    assert ws(3, 100, 8, 128, 16, 512) == 0          # 8192 keys: one chunk, no partials
    slots, chunks = 100 // 256 + 3, 2                  # 513 blocks: two chunks
    rows = 8 * slots * chunks * 256
    align = lambda x: (x + 255) // 256 * 256
    assert ws(3, 100, 8, 128, 16, 513) == align(rows * 128 * 4) + align(rows * 4)
    assert ws(3, 100, 8, 128, 32, 513) == 0           # bad block size
    assert ws(-1, 100, 8, 128, 16, 513) == 0


def _bwdv(ptr=1 << 20, n=2, tq=300, tk=300, Hq=4, Hkv=2, d=128, causal=1, window=0, ws=1 << 22,
          ws_bytes=1 << 20):
    return _lib.lib().attn_bwd_varlen(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, n,
                                      tq, tk, Hq, Hkv, d, causal, window, 0.1, ws, ws_bytes, None)


def test_bwd_varlen_validation():
    assert _bwdv(ptr=None) == _lib.ATTN_E_NULL
    assert _bwdv(n=-1) == _lib.ATTN_E_SHAPE
    assert _bwdv(Hq=3, Hkv=2) == _lib.ATTN_E_SHAPE
    assert _bwdv(d=96) == _lib.ATTN_E_HEADDIM
    assert _bwdv(causal=0, window=3) == _lib.ATTN_E_MASK
    assert _bwdv(Hq=70000, Hkv=1) == _lib.ATTN_E_SHAPE
    assert _bwdv(ws=None) == _lib.ATTN_E_WORKSPACE
    assert _bwdv(ws_bytes=16) == _lib.ATTN_E_WORKSPACE
    assert _bwdv(ptr=None, n=0) == _lib.ATTN_OK


def test_merge_validation():
    f = _lib.lib().attn_merge
    p = 1 << 20
    assert f(None, p, p, p, p, None, 1, 8, 2, 128, None) == _lib.ATTN_E_NULL
    assert f(p, p, p, p, p, None, 1, 8, 0, 128, None) == _lib.ATTN_E_SHAPE
    assert f(p, p, p, p, p, None, -1, 8, 2, 128, None) == _lib.ATTN_E_SHAPE
    assert f(p, p, p, p, p, None, 1, 8, 2, 96, None) == _lib.ATTN_E_HEADDIM
    assert f(None, None, None, None, None, None, 0, 8, 2, 128, None) == _lib.ATTN_OK
