"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any launch (no GPU needed: every call below returns
before touching the device)."""
import ctypes
import os
import re

import pytest

import block_diffusion_draft_position_amd as ddt
from block_diffusion_draft_position_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ddt.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libddt.so not built (run __graft_entry__.build())")


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ddt_[a-z_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert declared() == sorted(_lib.EXPORTS)


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = ddt.load()
    assert lib.ddt_status_string(0) == b"ok"
    assert lib.ddt_status_string(-3) == b"workspace too small"
    assert lib.ddt_status_string(12345) == b"unknown status"


def _fake(n=1):
    return ctypes.c_void_p(0x1000 * n)  # never dereferenced: calls fail validation first


def test_topk_validation():
    lib = ddt.load()
    f = lib.ddt_topk
    assert f(None, 4, 64, 64, 4, _fake(), _fake(2), _fake(3), 1 << 20, None) == -1
    assert f(_fake(), 0, 64, 64, 4, _fake(), _fake(2), _fake(3), 1 << 20, None) == -1
    assert f(_fake(), 4, 64, 63, 4, _fake(), _fake(2), _fake(3), 1 << 20, None) == -1  # stride < V
    assert f(_fake(), 4, 64, 64, 65, _fake(), _fake(2), _fake(3), 1 << 20, None) == -1  # k > 64
    assert f(_fake(), 4, 3, 3, 4, _fake(), _fake(2), _fake(3), 1 << 20, None) == -1   # k > V
    need = lib.ddt_topk_workspace_size(4, 64, 4)
    assert need > 0
    assert f(_fake(), 4, 64, 64, 4, _fake(), _fake(2), _fake(3), need - 1, None) == -3
    assert lib.ddt_topk_workspace_size(4, 64, 0) == 0


def test_build_tree_validation():
    f = ddt.load().ddt_build_tree
    a = [_fake(i) for i in range(1, 10)]
    assert f(None, a[1], a[2], 1, 4, 4, 8, a[3], a[4], a[5], None, a[6], None) == -1
    assert f(a[0], a[1], a[2], 0, 4, 4, 8, a[3], a[4], a[5], None, a[6], None) == -1
    assert f(a[0], a[1], a[2], 1, 65, 4, 8, a[3], a[4], a[5], None, a[6], None) == -1
    assert f(a[0], a[1], a[2], 1, 4, 65, 8, a[3], a[4], a[5], None, a[6], None) == -1
    assert f(a[0], a[1], a[2], 1, 4, 4, 1024, a[3], a[4], a[5], None, a[6], None) == -1
    assert f(a[0], a[1], a[2], 1, 4, 4, -1, a[3], a[4], a[5], None, a[6], None) == -1


def test_draft_tree_validation():
    lib = ddt.load()
    f = lib.ddt_draft_tree
    a = [_fake(i) for i in range(1, 20)]

    def call(S=1, L=4, V=64, K=4, B=8, stride=64, ws_bytes=1 << 20, logits=a[0]):
        return f(logits, stride, a[1], a[2], S, L, V, K, B, a[3], a[4], a[5], a[6], a[7], a[8],
                 a[9], a[10], a[11], a[12], ws_bytes, None)
    assert call(logits=None) == -1
    assert f(a[0], 64, a[1], a[2], 1, 4, 64, 4, 8, None, a[4], a[5], a[6], a[7], a[8], a[9],
             a[10], a[11], a[12], 1 << 20, None) == -1   # top-K outputs are required
    assert call(S=0) == -1
    assert call(L=65) == -1
    assert call(K=65) == -1
    assert call(V=3, stride=3) == -1          # K > V
    assert call(stride=63) == -1              # stride < V
    assert call(B=1024) == -1
    need = lib.ddt_draft_tree_workspace_size(1, 4, 64, 4)
    assert need == lib.ddt_topk_workspace_size(4, 64, 4) > 0
    assert call(ws_bytes=need - 1) == -3


def test_mask_validation():
    f = ddt.load().ddt_tree_mask
    a = [_fake(i) for i in range(1, 10)]
    assert f(a[0], a[1], a[2], None, 1, 8, None, None, None) == -1
    assert f(a[0], a[1], a[2], None, 0, 8, a[3], None, None) == -1
    assert f(a[0], a[1], a[2], None, 1, 1024, a[3], None, None) == -1


def test_attention_validation():
    f = ddt.load().ddt_tree_attention
    a = [_fake(i) for i in range(1, 12)]

    def call(S=1, B=8, Hq=4, Hkv=2, D=128, dt=1, scale=0.1, maxp=64, ws_bytes=0, q=a[0]):
        return f(q, a[1], a[2], a[3], a[4], a[5], a[6], a[7], S, B, Hq, Hkv, D, dt, scale, maxp,
                 a[8], None, a[9], ws_bytes, None)
    assert call(q=None) == -1
    assert call(Hq=6, Hkv=4) == -1        # Hq % Hkv
    assert call(D=96) == -2               # no kernel for D=96
    assert call(dt=7) == -2
    assert call(scale=0.0) == -1
    assert call(scale=float("inf")) == -1
    assert call(scale=float("nan")) == -1
    assert call(maxp=-1) == -1
    assert call(B=1024) == -1


def test_walk_validation():
    lib = ddt.load()
    f = lib.ddt_tree_walk
    a = [_fake(i) for i in range(1, 12)]

    def call(S=1, B=8, L=4, V=64, ws_bytes=1 << 20, tt=a[0]):
        return f(tt, a[1], a[2], a[3], S, B, L, V, a[4], a[5], a[6], a[7], a[8], ws_bytes, None)
    assert call(tt=None) == -1
    assert call(L=0) == -1
    assert call(L=65) == -1
    assert call(V=0) == -1
    assert call(ws_bytes=lib.ddt_tree_walk_workspace_size(1, 8, 64) - 1) == -3


def test_product_path_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libddt.so")
    with pytest.raises(_lib.DDTError):
        _lib.load()
