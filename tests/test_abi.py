"""CPU checks of the C ABI: the shared library loads, exports every function
that include/qat.h declares, and rejects invalid arguments with the
documented status before any device work (no GPU is touched here)."""
import ctypes
import os
import re

import pytest
import torch

import query_aware_top_amd as qat
from query_aware_top_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qat.h")

QAT_OK, QAT_EINVAL, QAT_EUNSUPPORTED, QAT_EWORKSPACE = 0, -1, -2, -3


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return [n for n in names if n not in ("if", "return")]


@pytest.fixture(scope="module")
def lib():
    path = B.lib_path
    if not os.path.exists(path):
        pytest.skip("libqat.so not built")
    return ctypes.CDLL(path)


def test_header_declares_the_entry_points():
    names = set(header_functions())
    for n in ("esa_compress", "esa_select", "esa_sparse_attn", "moba_block_select", "moba_sparse_attn",
              "esa_workspace_size", "moba_workspace_size", "qat_last_error", "qat_abi_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    names = header_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(B.EXPORTED_SYMBOLS)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+QAT_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert m and lib.qat_abi_version() == int(m.group(1))


def _moba(**kw):
    base = dict(batch=1, seq_len=4096, n_q_heads=4, n_kv_heads=2, head_dim=64, block=256, topk=3)
    base.update(kw)
    return qat.moba_params(**base)


def _esa(**kw):
    base = dict(batch=1, n_heads=4, head_dim=64, d_c=64, ctx_len=2048, chunk_start=1792, chunk_len=256,
                n_init=16, window=128, topk=64, radius=2, clip=48.0)
    base.update(kw)
    return qat.esa_params(**base)


def _size(lib, fn, p):
    n = ctypes.c_size_t(0)
    rc = getattr(lib, fn)(ctypes.byref(p), ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,rc", [
    ({}, QAT_OK),
    (dict(topk=0), QAT_EINVAL),
    (dict(topk=17), QAT_EINVAL),
    (dict(n_kv_heads=3), QAT_EINVAL),
    (dict(head_dim=96), QAT_EUNSUPPORTED),
    (dict(block=0), QAT_EINVAL),
    (dict(q_start=4000, q_len=200), QAT_EINVAL),
    (dict(window=-1), QAT_EINVAL),
    (dict(scale=float("inf")), QAT_EINVAL),
    (dict(scale=-1.0), QAT_EINVAL),
])
def test_moba_params_validation(lib, kw, rc):
    p = _moba(**kw)
    got, n = _size(lib, "moba_workspace_size", p)
    assert got == rc
    if rc == QAT_OK:
        assert n > 0 and n % 256 == 0
    else:
        lib.qat_last_error.restype = ctypes.c_char_p
        assert lib.qat_last_error()   # a message names the bad argument


@pytest.mark.parametrize("kw,rc", [
    ({}, QAT_OK),
    (dict(chunk_len=1, chunk_start=2047), QAT_OK),
    (dict(head_dim=80), QAT_EUNSUPPORTED),
    (dict(d_c=48), QAT_EUNSUPPORTED),
    (dict(chunk_start=2000, chunk_len=100), QAT_EINVAL),
    (dict(topk=0), QAT_EINVAL),
    (dict(clip=0.0), QAT_EINVAL),
    (dict(radius=-1), QAT_EINVAL),
    (dict(scale=0.0), QAT_EINVAL),
    (dict(per_head=True), QAT_OK),
    (dict(per_head=True, d_c=48), QAT_OK),                        # d_c is unused per head
    (dict(per_head=True, dtype=torch.float32), QAT_EUNSUPPORTED),
])
def test_esa_params_validation(lib, kw, rc):
    got, n = _size(lib, "esa_workspace_size", _esa(**kw))
    assert got == rc
    if rc == QAT_OK:
        assert n > 0


def test_workspace_too_small_is_rejected_before_device_work(lib):
    # dummy non-NULL device pointers: nothing may be dereferenced or launched
    dummy = ctypes.c_void_p(0x1000)
    p = _moba()
    rc, need = _size(lib, "moba_workspace_size", p)
    assert rc == QAT_OK
    rc = lib.moba_block_select(ctypes.byref(p), dummy, dummy, dummy, dummy, ctypes.c_size_t(need - 1),
                               ctypes.c_void_p(0))
    assert rc == QAT_EWORKSPACE
    rc = lib.moba_sparse_attn(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, None, dummy,
                              ctypes.c_size_t(need - 256), ctypes.c_void_p(0))
    assert rc == QAT_EWORKSPACE
    pe = _esa()
    rc, need = _size(lib, "esa_workspace_size", pe)
    rc = lib.esa_select(ctypes.byref(pe), dummy, dummy, None, dummy, dummy, dummy, None, dummy,
                        ctypes.c_size_t(need - 1), ctypes.c_void_p(0))
    assert rc == QAT_EWORKSPACE
    rc = lib.esa_sparse_attn(ctypes.byref(pe), dummy, dummy, dummy, dummy, dummy, dummy, None, None,
                             ctypes.c_size_t(0), ctypes.c_void_p(0))
    assert rc == QAT_EWORKSPACE


def test_null_pointers_are_rejected(lib):
    dummy = ctypes.c_void_p(0x1000)
    p = _moba()
    rc = lib.moba_block_select(ctypes.byref(p), None, dummy, dummy, dummy, ctypes.c_size_t(1 << 30),
                               ctypes.c_void_p(0))
    assert rc == QAT_EINVAL
    rc = lib.moba_sparse_attn(ctypes.byref(p), dummy, dummy, dummy, dummy, None, None, dummy,
                              ctypes.c_size_t(1 << 30), ctypes.c_void_p(0))
    assert rc == QAT_EINVAL
    pe = _esa()
    rc = lib.esa_select(ctypes.byref(pe), dummy, None, None, dummy, dummy, dummy, None, dummy,
                        ctypes.c_size_t(1 << 30), ctypes.c_void_p(0))
    assert rc == QAT_EINVAL
    assert lib.moba_block_select(None, dummy, dummy, dummy, dummy, ctypes.c_size_t(0), None) == QAT_EINVAL


def test_per_head_flag_picks_the_selection_entry(lib):
    """esa_select merges the heads (per_head 0), esa_select_heads selects
    per head (per_head 1); the other combination and per_head values other
    than 0 / 1 are rejected before any device work. The per-head gradient
    workspace holds one key list per (sequence, head)."""
    dummy = ctypes.c_void_p(0x1000)
    big = ctypes.c_size_t(1 << 40)
    pm, ph = _esa(), _esa(per_head=True)
    assert lib.esa_select(ctypes.byref(ph), dummy, dummy, None, dummy, dummy, dummy, None, dummy, big,
                          ctypes.c_void_p(0)) == QAT_EINVAL
    assert lib.esa_select_heads(ctypes.byref(pm), dummy, dummy, dummy, dummy, None, dummy, big,
                                ctypes.c_void_p(0)) == QAT_EINVAL
    bad = _esa()
    bad.per_head = 2
    assert _size(lib, "esa_workspace_size", bad)[0] == QAT_EINVAL
    assert _size(lib, "esa_workspace_size", ph)[0] == QAT_OK
    assert _size(lib, "esa_bwd_workspace_size", ph)[1] > _size(lib, "esa_bwd_workspace_size", pm)[1]


def test_plan_defers_the_call_and_raises_on_replay(lib):
    """qat.plan records the entry-point call instead of making it (size
    queries run at once); the replay makes it and turns a failing status
    into QatError. Invalid parameters fail before any device work."""
    p = _esa(topk=0)
    dummy = ctypes.c_void_p(0x1000)

    def call():
        n = ctypes.c_size_t(0)
        assert B.lib().esa_workspace_size(ctypes.byref(_esa()), ctypes.byref(n)) == QAT_OK and n.value > 0
        return B.lib().esa_select(ctypes.byref(p), dummy, dummy, None, dummy, dummy, dummy, None, dummy,
                                  ctypes.c_size_t(1 << 40), ctypes.c_void_p(0))

    replay = qat.plan(call)
    assert replay.calls == ["esa_select"]
    with pytest.raises(qat.QatError):
        replay()


def test_plan_keeps_allocated_buffers_alive_and_records_per_thread(lib):
    """A buffer the planned function allocates itself (an output or a
    workspace it was not given) stays referenced by the plan, so the
    replays never write into memory the allocator has handed on; the
    function's return value is the plan's `result`; and a binding call made
    from another thread while the plan records is not recorded."""
    import gc
    import threading
    import weakref

    import torch
    seen = {}

    def call():
        ws = torch.empty(64, dtype=torch.uint8)   # allocated inside, like an omitted workspace
        seen["ws"] = weakref.ref(ws)
        other = {}
        th = threading.Thread(target=lambda: other.setdefault("lib", B.lib()))
        th.start()
        th.join()
        seen["other_is_recorder"] = isinstance(other["lib"], B._Recorder)
        B.lib().esa_select(None, B._ptr(ws), None, None, None, None, None, None, None, ctypes.c_size_t(0),
                           ctypes.c_void_p(0))
        return "outputs"

    replay = qat.plan(call)
    gc.collect()
    assert replay.calls == ["esa_select"]
    assert replay.result == "outputs"
    assert seen["ws"]() is not None, "a buffer the recorded call points at was freed"
    assert not seen["other_is_recorder"], "another thread's binding call was recorded"
    assert not isinstance(B.lib(), B._Recorder)
    del replay
    gc.collect()
    assert seen["ws"]() is None


def test_compress_validation(lib):
    dummy = ctypes.c_void_p(0x1000)
    n = ctypes.c_size_t(0)
    assert lib.esa_compress_workspace_size(ctypes.c_int64(16), ctypes.c_int64(4096), ctypes.c_int64(128),
                                           ctypes.byref(n)) == QAT_OK
    assert n.value > 0
    # d_c not supported
    rc = lib.esa_compress(dummy, ctypes.c_int64(16), ctypes.c_int64(4096), ctypes.c_int64(4096), ctypes.c_int32(1),
                          dummy, None, ctypes.c_int64(100), dummy, ctypes.c_int64(100), ctypes.c_int32(1), dummy,
                          ctypes.c_size_t(n.value), None)
    assert rc == QAT_EUNSUPPORTED
    # row stride shorter than the row
    rc = lib.esa_compress(dummy, ctypes.c_int64(16), ctypes.c_int64(1024), ctypes.c_int64(4096), ctypes.c_int32(1),
                          dummy, None, ctypes.c_int64(128), dummy, ctypes.c_int64(128), ctypes.c_int32(1), dummy,
                          ctypes.c_size_t(n.value), None)
    assert rc == QAT_EINVAL


def test_decode_entry_points_validation(lib):
    dummy = ctypes.c_void_p(0x1000)
    p = _moba(q_start=4095, q_len=1)
    rc, need = _size(lib, "moba_workspace_size", p)
    assert rc == QAT_OK
    # block range past the complete blocks (4096 / 256 = 16)
    for first, n in ((15, 2), (-1, 1), (0, -1)):
        rc = lib.moba_block_means(ctypes.byref(p), dummy, ctypes.c_int64(first), ctypes.c_int64(n), dummy, dummy,
                                  ctypes.c_size_t(need), ctypes.c_void_p(0))
        assert rc == QAT_EINVAL, (first, n)
    rc = lib.moba_block_means(ctypes.byref(p), dummy, ctypes.c_int64(0), ctypes.c_int64(16), dummy, dummy,
                              ctypes.c_size_t(need - 1), ctypes.c_void_p(0))
    assert rc == QAT_EWORKSPACE
    # the cache is needed once a row has an earlier block
    assert lib.moba_decode_select(ctypes.byref(p), dummy, None, dummy, ctypes.c_void_p(0)) == QAT_EINVAL
    rc = lib.moba_decode_attn(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, None, dummy,
                              ctypes.c_size_t(need - 256), ctypes.c_void_p(0))
    assert rc == QAT_EWORKSPACE
    rc = lib.moba_decode_attn(ctypes.byref(p), dummy, None, dummy, dummy, dummy, None, dummy,
                              ctypes.c_size_t(need), ctypes.c_void_p(0))
    assert rc == QAT_EINVAL


def test_decode_workspace_holds_the_piece_buffers(lib):
    # few rows: the split-key buffers are part of the workspace
    few = _size(lib, "moba_workspace_size", _moba(q_start=4095, q_len=1, n_q_heads=2, n_kv_heads=2))[1]
    many = _size(lib, "moba_workspace_size", _moba(q_start=4000, q_len=9, n_q_heads=2, n_kv_heads=2))[1]
    assert few > 0 and many > 0
