"""The C ABI without a GPU: library loads, every declared symbol is exported,
and invalid or unsupported arguments are rejected before any HIP call."""
import ctypes
import os
import re

import pytest

from linear_attention_tensor_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libtc.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tc_scan_forward", "tc_decode_step", "tc_decode_layer_step", "tc_fused_layer", "delta_scan_forward",
              "tc_scan_workspace_bytes", "tc_fused_workspace_bytes", "delta_scan_workspace_bytes",
              "tc_last_error", "tc_version"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_version():
    assert _lib.lib().tc_version().decode().startswith("libtc")


L = None


def lib():
    return _lib.lib()


NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below is rejected first


def scan(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=_lib.TC_F32, lam=FAKE, eta=FAKE, B=1, H=1, T=128, dk=64, dv=64,
             W=16, chunk=64, m=FAKE, A=NULL, ws=NULL, ws_bytes=0)
    a.update(kw)
    return lib().tc_scan_forward(a["q"], a["k"], a["v"], a["dt"], a["lam"], a["eta"], a["B"], a["H"],
                                 a["T"], a["dk"], a["dv"], a["W"], a["chunk"], a["m"], a["A"], a["ws"],
                                 a["ws_bytes"], NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=32), _lib.TC_ERR_UNSUPPORTED),
    (dict(dk=48, dv=48), _lib.TC_ERR_UNSUPPORTED),
    (dict(dk=64, dv=32), _lib.TC_ERR_UNSUPPORTED),
    (dict(B=-1), _lib.TC_ERR_INVALID_ARG),
    (dict(T=-5), _lib.TC_ERR_INVALID_ARG),
    (dict(W=0), _lib.TC_ERR_INVALID_ARG),
    (dict(dt=7), _lib.TC_ERR_INVALID_ARG),
    (dict(q=NULL), _lib.TC_ERR_INVALID_ARG),
    (dict(lam=NULL), _lib.TC_ERR_INVALID_ARG),
    (dict(m=NULL), _lib.TC_ERR_INVALID_ARG),
])
def test_scan_rejects(kw, status):
    assert scan(**kw) == status
    assert _lib.last_error() != ""


def test_scan_empty_is_ok_without_device():
    assert scan(B=0) == _lib.TC_OK
    assert scan(H=0, q=NULL) == _lib.TC_OK
    assert _lib.last_error() == ""


def test_scan_workspace_check():
    need = lib().tc_scan_workspace_bytes(4, 8, 4096, 64, 64, 512, 64, _lib.TC_F32)
    assert 0 < need < _lib.SIZE_MAX
    assert scan(B=4, H=8, T=4096, W=512, ws=FAKE, ws_bytes=need - 1) == _lib.TC_ERR_WORKSPACE
    assert lib().tc_scan_workspace_bytes(1, 1, 10, 64, 64, 0, 64, _lib.TC_F32) == _lib.SIZE_MAX


def test_scan_noalloc_rejects_before_any_device_call():
    f = lib().tc_scan_forward_noalloc

    def call(**kw):
        a = dict(dt=_lib.TC_BF16, B=1, H=8, T=32768, d=128, W=1024, chunk=64, q=FAKE, m=FAKE)
        a.update(kw)
        return f(a["q"], FAKE, FAKE, a["dt"], FAKE, FAKE, a["B"], a["H"], a["T"], a["d"], a["d"], a["W"],
                 a["chunk"], a["m"], NULL, NULL)

    # more scratch than the library holds (64 MiB of bf16 tile states > 32 MiB)
    assert call() == _lib.TC_ERR_WORKSPACE
    assert "scratch" in _lib.last_error()
    assert call(chunk=32) == _lib.TC_ERR_UNSUPPORTED
    assert call(W=0) == _lib.TC_ERR_INVALID_ARG
    assert call(q=NULL, B=1, H=1, T=16, d=16, W=4) == _lib.TC_ERR_INVALID_ARG
    assert call(B=0) == _lib.TC_OK


def test_window_attention_rejects():
    f = lib().tc_window_attention

    def call(**kw):
        a = dict(dt=_lib.TC_F32, B=1, H=2, T=100, dk=64, dv=64, W=16, scale=0.125, q=FAKE, y=FAKE)
        a.update(kw)
        return f(a["q"], FAKE, FAKE, a["dt"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["W"], a["scale"], a["y"],
                 NULL)

    assert call(W=0) == _lib.TC_ERR_INVALID_ARG
    assert call(dk=48, dv=48) == _lib.TC_ERR_UNSUPPORTED
    assert call(dk=64, dv=32) == _lib.TC_ERR_UNSUPPORTED
    assert call(scale=0.0) == _lib.TC_ERR_INVALID_ARG
    assert call(scale=float("inf")) == _lib.TC_ERR_INVALID_ARG
    assert call(q=NULL) == _lib.TC_ERR_INVALID_ARG
    assert call(y=NULL) == _lib.TC_ERR_INVALID_ARG
    assert call(T=0, q=NULL, y=NULL) == _lib.TC_OK


def test_fused_workspace_query_covers_every_dtype_and_width():
    q = lib().tc_fused_workspace_bytes
    for dt in (_lib.TC_F32, _lib.TC_BF16):
        for d in (16, 32, 64, 128):
            assert q(2, 3, 1000, d, d, 100, 64, dt) < _lib.SIZE_MAX


def test_backward_entry_points_reject():
    L = lib()
    wq = L.tc_window_attention_backward_workspace_bytes
    assert 0 < wq(1, 2, 100, 64, 64, 16, _lib.TC_F32) < _lib.SIZE_MAX
    assert wq(1, 2, 100, 48, 48, 16, _lib.TC_F32) == _lib.SIZE_MAX
    need = wq(1, 2, 100, 64, 64, 16, _lib.TC_F32)
    f = L.tc_window_attention_backward
    base = [FAKE, FAKE, FAKE, _lib.TC_F32, 1, 2, 100, 64, 64, 16, 0.125, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL]
    bad = list(base); bad[9] = 0
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    bad = list(base); bad[16] = need - 1
    assert f(*bad) == _lib.TC_ERR_WORKSPACE
    bad = list(base); bad[11] = NULL
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    fq = L.tc_fused_layer_backward_workspace_bytes
    assert 0 < fq(1, 2, 100, 128, 128, 16, 64, _lib.TC_BF16) < _lib.SIZE_MAX  # d = 128: four d = 64 pieces in place
    assert fq(1, 2, 100, 48, 48, 16, 64, _lib.TC_BF16) == _lib.SIZE_MAX
    assert 0 < fq(1, 2, 100, 64, 64, 16, 64, _lib.TC_BF16) < _lib.SIZE_MAX
    g = L.tc_fused_layer_backward
    n2 = fq(1, 2, 100, 64, 64, 16, 64, _lib.TC_F32)
    args = [FAKE, FAKE, FAKE, _lib.TC_F32, FAKE, FAKE, FAKE, 1, 2, 100, 64, 64, 16, 64, 0.125, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, FAKE, n2, NULL]
    bad = list(args); bad[6] = NULL  # g
    assert g(*bad) == _lib.TC_ERR_INVALID_ARG
    bad = list(args); bad[23] = n2 - 1
    assert g(*bad) == _lib.TC_ERR_WORKSPACE
    bad = list(args); bad[14] = -1.0
    assert g(*bad) == _lib.TC_ERR_INVALID_ARG


def test_decode_rejects():
    f = lib().tc_decode_step
    args = [FAKE, FAKE, FAKE, _lib.TC_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 128, 16, FAKE, NULL]
    bad = list(args); bad[14] = 0
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    bad = list(args); bad[12] = 100; bad[13] = 100
    assert f(*bad) == _lib.TC_ERR_UNSUPPORTED
    bad = list(args); bad[9] = NULL
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    ok = list(args); ok[10] = 0
    assert f(*ok) == _lib.TC_OK


def test_decode_layer_rejects():
    f = lib().tc_decode_layer_step
    args = [FAKE, FAKE, FAKE, _lib.TC_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 128, 16,
            0.088, FAKE, NULL]
    bad = list(args); bad[15] = 0  # W
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    bad = list(args); bad[13] = 100; bad[14] = 100  # d
    assert f(*bad) == _lib.TC_ERR_UNSUPPORTED
    bad = list(args); bad[13] = 64  # dk != dv
    assert f(*bad) == _lib.TC_ERR_UNSUPPORTED
    bad = list(args); bad[9] = NULL  # g
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    bad = list(args); bad[16] = 0.0  # softmax scale
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    bad = list(args); bad[16] = float("nan")
    assert f(*bad) == _lib.TC_ERR_INVALID_ARG
    ok = list(args); ok[11] = 0  # B = 0: nothing to do, no device touched
    assert f(*ok) == _lib.TC_OK


def test_fused_rejects():
    f = lib().tc_fused_layer

    T = 32768  # long enough that the call needs a workspace
    need = lib().tc_fused_workspace_bytes(1, 2, T, 128, 128, 64, 64, _lib.TC_BF16)
    assert 0 < need < _lib.SIZE_MAX

    # every call below is rejected before any launch (a short workspace included)
    def call(dt=_lib.TC_BF16, d=128, scale=0.1, ws_bytes=0, W=64):
        return f(FAKE, FAKE, FAKE, dt, FAKE, FAKE, FAKE, 1, 2, T, d, d, W, 64, scale, FAKE, NULL, FAKE,
                 ws_bytes, NULL)

    # fp32 inputs and d = 32 are supported (the prefill scan's path), and need a workspace here
    assert call(dt=_lib.TC_F32) == _lib.TC_ERR_WORKSPACE
    assert call(d=32) == _lib.TC_ERR_WORKSPACE
    assert call(d=48) == _lib.TC_ERR_UNSUPPORTED
    assert call(scale=0.0) == _lib.TC_ERR_INVALID_ARG
    assert call(scale=float("nan")) == _lib.TC_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == _lib.TC_ERR_WORKSPACE
    assert lib().tc_fused_workspace_bytes(1, 2, 256, 48, 48, 64, 64, _lib.TC_F32) == _lib.SIZE_MAX


def test_delta_rejects():
    f = lib().delta_scan_forward

    def call(**kw):
        a = dict(dt=_lib.TC_BF16, beta=FAKE, B=1, H=1, T=64, d=64, chunk=64)
        a.update(kw)
        return f(FAKE, FAKE, FAKE, a["dt"], a["beta"], a["B"], a["H"], a["T"], a["d"], a["d"], a["chunk"],
                 NULL, FAKE, NULL, NULL, 0, NULL)

    assert call(chunk=128) == _lib.TC_ERR_UNSUPPORTED
    assert call(beta=NULL) == _lib.TC_ERR_INVALID_ARG
    assert call(d=24) == _lib.TC_ERR_UNSUPPORTED
    assert call(B=0) == _lib.TC_OK


def test_profile_hook_argument_check():
    L = _lib.lib()
    fake = ctypes.c_void_p(0x1000)  # never used: the call with one NULL is rejected first
    assert L.tc_profile_next_call(fake, None) == _lib.TC_ERR_INVALID_ARG
    assert "two events" in _lib.last_error()
    assert L.tc_profile_next_call(None, fake) == _lib.TC_ERR_INVALID_ARG
    assert L.tc_profile_next_call(None, None) == _lib.TC_OK  # disarmed
    assert _lib.last_error() == ""


def test_scan_backward_rejects():
    f = lib().tc_scan_backward
    need = lib().tc_scan_backward_workspace_bytes(4, 8, 4096, 64, 64, 512, 64, _lib.TC_F32)
    assert 0 < need < _lib.SIZE_MAX

    def call(**kw):
        a = dict(dt=_lib.TC_F32, B=4, H=8, T=4096, d=64, W=512, chunk=64, dm=FAKE, dlam=FAKE, ws=FAKE,
                 ws_bytes=need, g=NULL, dg=NULL)
        a.update(kw)
        return f(FAKE, FAKE, FAKE, a["dt"], FAKE, FAKE, a["g"], a["B"], a["H"], a["T"], a["d"], a["d"], a["W"],
                 a["chunk"], a["dm"], FAKE, FAKE, FAKE, a["dlam"], FAKE, a["dg"], a["ws"], a["ws_bytes"], NULL)

    # bf16 inputs are widened to fp32 copies in the workspace, which is larger by those
    need16 = lib().tc_scan_backward_workspace_bytes(4, 8, 4096, 64, 64, 512, 64, _lib.TC_BF16)
    assert need16 >= need + 3 * 4 * 8 * 4096 * 64 * 4
    assert call(dt=_lib.TC_BF16) == _lib.TC_ERR_WORKSPACE
    need128 = lib().tc_scan_backward_workspace_bytes(4, 8, 4096, 128, 128, 512, 64, _lib.TC_F32)
    assert call(d=128, ws_bytes=need128 - 1) == _lib.TC_ERR_WORKSPACE
    assert call(d=48) == _lib.TC_ERR_UNSUPPORTED
    assert call(W=0) == _lib.TC_ERR_INVALID_ARG
    assert call(chunk=128) == _lib.TC_ERR_UNSUPPORTED
    assert call(dm=NULL) == _lib.TC_ERR_INVALID_ARG
    assert call(dlam=NULL) == _lib.TC_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == _lib.TC_ERR_WORKSPACE
    assert call(ws=NULL) == _lib.TC_ERR_INVALID_ARG
    assert call(g=FAKE) == _lib.TC_ERR_INVALID_ARG  # a gate without dg
    assert call(dg=FAKE) == _lib.TC_ERR_INVALID_ARG
    assert call(B=0) == _lib.TC_OK
    # d = 128 runs four d = 64 pieces in place: the d = 64 workspace (rounded to 256 bytes); bf16 adds the
    # three widened copies, and (d in {64, 128}) the four time-reversed bf16 copies and the bf16 read's own
    # workspace
    w128 = lib().tc_scan_backward_workspace_bytes(1, 1, 10, 128, 128, 4, 64, _lib.TC_F32)
    w64 = lib().tc_scan_backward_workspace_bytes(1, 1, 10, 64, 64, 4, 64, _lib.TC_F32)
    assert w64 <= w128 == (w64 + 255) // 256 * 256
    w128b = lib().tc_scan_backward_workspace_bytes(1, 1, 10, 128, 128, 4, 64, _lib.TC_BF16)
    r256 = lambda n: (n + 255) // 256 * 256
    assert w128b > w128 + 3 * r256(10 * 128 * 4) + 4 * r256(10 * 128 * 2)
    w32b = lib().tc_scan_backward_workspace_bytes(1, 1, 10, 32, 32, 4, 64, _lib.TC_BF16)
    w32 = lib().tc_scan_backward_workspace_bytes(1, 1, 10, 32, 32, 4, 64, _lib.TC_F32)
    assert w32b == r256(w32) + 3 * r256(10 * 32 * 4)
    # the query is exactly what the call checks
    assert call(dt=_lib.TC_BF16, B=1, H=1, T=10, d=128, W=4, ws_bytes=w128b - 1) == _lib.TC_ERR_WORKSPACE


def test_memory_entry_points_reject():
    L = lib()
    assert L.hebbian_workspace_bytes(100, 100, 64) == _lib.SIZE_MAX  # m not a multiple of 64
    assert L.hebbian_workspace_bytes(100, 128, 48) == _lib.SIZE_MAX
    assert 0 < L.hebbian_workspace_bytes(100, 128, 64) < _lib.SIZE_MAX
    need = L.hebbian_workspace_bytes(100, 128, 64)
    w = L.hebbian_write
    assert w(FAKE, FAKE, FAKE, 100, 100, FAKE, FAKE, 128, 64, FAKE, FAKE, need - 1, NULL) == _lib.TC_ERR_WORKSPACE
    assert w(FAKE, FAKE, NULL, 100, 100, FAKE, FAKE, 128, 64, FAKE, FAKE, need, NULL) == _lib.TC_ERR_INVALID_ARG
    assert w(FAKE, FAKE, FAKE, 0, 100, FAKE, FAKE, 128, 64, FAKE, FAKE, need, NULL) == _lib.TC_ERR_INVALID_ARG
    assert L.hebbian_read(FAKE, 0, FAKE, FAKE, FAKE, 128, 64, FAKE, NULL) == _lib.TC_OK
    assert L.hebbian_read(FAKE, 10, FAKE, FAKE, FAKE, 96, 64, FAKE, NULL) == _lib.TC_ERR_UNSUPPORTED
    assert L.tc_memory_read(FAKE, FAKE, 2, 10, 16, FAKE, NULL) == _lib.TC_ERR_UNSUPPORTED
    assert L.tc_memory_read(FAKE, FAKE, 0, 10, 64, FAKE, NULL) == _lib.TC_OK
    assert L.tc_memory_read(NULL, FAKE, 2, 10, 64, FAKE, NULL) == _lib.TC_ERR_INVALID_ARG
    assert L.recall_argmax(FAKE, FAKE, 1, 10, 0, 64, FAKE, NULL, NULL) == _lib.TC_ERR_INVALID_ARG
    assert L.recall_argmax(FAKE, FAKE, 70000, 10, 5, 64, FAKE, NULL, NULL) == _lib.TC_ERR_UNSUPPORTED
    assert L.recall_argmax(FAKE, FAKE, 1, 0, 5, 64, FAKE, NULL, NULL) == _lib.TC_OK


def test_delta_backward_workspace_query_widths():
    q = lib().delta_scan_backward_workspace_bytes
    for dt in (_lib.TC_F32, _lib.TC_BF16):
        for d in (16, 32, 64, 128):
            assert 0 < q(2, 3, 300, d, d, 64, dt) < _lib.SIZE_MAX
        assert q(2, 3, 300, 48, 48, 64, dt) == _lib.SIZE_MAX
        assert q(2, 3, 300, 128, 64, 64, dt) == _lib.SIZE_MAX
