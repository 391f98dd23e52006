"""ctypes marshalling for libqat.so (see include/qat.h for the contract)."""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.environ.get("QAT_LIB_PATH") or os.path.join(_HERE, "libqat.so")

QAT_F32, QAT_BF16 = 0, 1
_STATUS = {0: "QAT_OK", -1: "QAT_EINVAL", -2: "QAT_EUNSUPPORTED", -3: "QAT_EWORKSPACE", -4: "QAT_EHIP"}

EXPORTED_SYMBOLS = (
    "qat_last_error", "qat_abi_version", "qat_timing_enable", "qat_timing_select", "qat_timing_reset",
    "qat_timing_query",
    "esa_workspace_size", "esa_compress_workspace_size", "esa_compress", "esa_select", "esa_select_heads",
    "esa_sparse_attn",
    "esa_bwd_workspace_size", "esa_sparse_attn_bwd",
    "moba_workspace_size", "moba_block_select", "moba_sparse_attn", "moba_block_means", "moba_decode_select",
    "moba_decode_attn", "moba_decode_attn_noalloc", "moba_bwd_workspace_size", "moba_sparse_attn_bwd", "cca_pool", "cca_attn",
)


class QatError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class EsaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("n_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("d_c", ctypes.c_int64), ("ctx_len", ctypes.c_int64), ("chunk_start", ctypes.c_int64),
        ("chunk_len", ctypes.c_int64), ("n_init", ctypes.c_int32), ("window", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("radius", ctypes.c_int32), ("clip", ctypes.c_float),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("correction", ctypes.c_int32),
        ("vote_tau", ctypes.c_float), ("per_head", ctypes.c_int32),
    ]


QAT_CORR_CLAMP, QAT_CORR_VOTES = 0, 1


class CcaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("n_q_heads", ctypes.c_int64),
        ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("q_start", ctypes.c_int64),
        ("q_len", ctypes.c_int64), ("group", ctypes.c_int32), ("window", ctypes.c_int32),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


class MobaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("n_q_heads", ctypes.c_int64),
        ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("q_start", ctypes.c_int64),
        ("q_len", ctypes.c_int64), ("block", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("window", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


_lib = None
_tls = threading.local()   # .recorder: the _Recorder of a plan() running on this thread


def lib():
    """Loads libqat.so once; raises if it has not been built. Inside plan(),
    on the planning thread only, returns that plan's recorder instead."""
    global _lib
    rec = getattr(_tls, "recorder", None)
    if rec is not None:
        return rec
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with `python -m query_aware_top_amd.build`")
        L = ctypes.CDLL(lib_path)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.qat_last_error.restype = ctypes.c_char_p
        L.qat_abi_version.restype = ctypes.c_int
        L.esa_workspace_size.argtypes = [ctypes.POINTER(EsaParams), ctypes.POINTER(sz)]
        L.esa_compress_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
        L.esa_compress.argtypes = [vp, i64, i64, i64, ctypes.c_int32, vp, vp, i64, vp, i64, ctypes.c_int32,
                                   vp, sz, vp]
        L.esa_select.argtypes = [ctypes.POINTER(EsaParams), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.esa_sparse_attn.argtypes = [ctypes.POINTER(EsaParams), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.esa_bwd_workspace_size.argtypes = [ctypes.POINTER(EsaParams), ctypes.POINTER(sz)]
        L.esa_sparse_attn_bwd.argtypes = [ctypes.POINTER(EsaParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                          vp]
        L.moba_workspace_size.argtypes = [ctypes.POINTER(MobaParams), ctypes.POINTER(sz)]
        L.cca_pool.argtypes = [ctypes.POINTER(CcaParams), vp, vp, vp, vp, vp, vp]
        L.cca_attn.argtypes = [ctypes.POINTER(CcaParams), vp, vp, vp, vp, vp, vp, vp, vp]
        L.moba_block_select.argtypes = [ctypes.POINTER(MobaParams), vp, vp, vp, vp, sz, vp]
        L.qat_timing_enable.argtypes = [ctypes.c_int]
        L.qat_timing_select.argtypes = [ctypes.c_char_p]
        L.qat_timing_reset.argtypes = []
        L.qat_timing_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
        L.moba_sparse_attn.argtypes = [ctypes.POINTER(MobaParams), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moba_block_means.argtypes = [ctypes.POINTER(MobaParams), vp, i64, i64, vp, vp, sz, vp]
        L.moba_decode_select.argtypes = [ctypes.POINTER(MobaParams), vp, vp, vp, vp]
        L.moba_decode_attn.argtypes = [ctypes.POINTER(MobaParams), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moba_decode_attn_noalloc.argtypes = [ctypes.POINTER(MobaParams), vp, vp, vp, vp, vp, vp, vp]
        L.moba_bwd_workspace_size.argtypes = [ctypes.POINTER(MobaParams), ctypes.POINTER(sz)]
        L.moba_sparse_attn_bwd.argtypes = [ctypes.POINTER(MobaParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                           vp]
        for name in EXPORTED_SYMBOLS:
            getattr(L, name).restype = ctypes.c_int if name != "qat_last_error" else ctypes.c_char_p
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().qat_abi_version()


def timing_enable(on: bool = True):
    """Per-kernel HIP-event timing inside the library (see qat_timing_enable)."""
    _check(lib().qat_timing_enable(1 if on else 0))


def timing_select(name=None):
    """Restrict the library's timing records to one stage (None: every stage)."""
    _check(lib().qat_timing_select(name.encode() if name else None))


def timing_reset():
    _check(lib().qat_timing_reset())


def timing_query(name: str):
    """Returns (total_ms, launches) recorded for one kernel name."""
    tot, n = ctypes.c_double(0), ctypes.c_int(0)
    _check(lib().qat_timing_query(name.encode(), ctypes.byref(tot), ctypes.byref(n)))
    return tot.value, n.value


def _check(rc: int):
    if rc != 0:
        raise QatError(rc, lib().qat_last_error().decode())


class _Recorder:
    """Stands in for the loaded library while a binding function runs under
    plan(): workspace-size queries go to the library at once (their results
    shape the call), every other entry point is recorded with its marshalled
    arguments and reported as successful."""

    def __init__(self, real):
        self._real = real
        self.calls = []
        self.keep = []   # every tensor whose pointer a recorded call holds

    def __getattr__(self, name):
        f = getattr(self._real, name)
        if name.endswith("workspace_size") or name.startswith("qat_"):
            return f

        def record(*args):
            self.calls.append((name, f, args))
            return 0

        return record


def plan(fn, *args, **kwargs):
    """Marshals one binding call once and returns a callable that re-issues
    the same C ABI call(s) with the same arguments: the same tensors (by
    pointer), parameters and the stream current now. For loops that repeat
    one call on fixed buffers (decode steps), where the per-call Python
    checks cost as much host time as the kernels take. The library still
    validates each call and a failing status raises.

    Every tensor whose pointer the recorded calls hold (inputs, and outputs
    or workspaces the binding function allocated when they were not passed
    in) is kept alive by the returned callable, so its memory cannot be
    handed to another tensor while the plan exists; fn's own return value
    (its outputs) is the callable's `result`. Recording is per thread: other
    threads calling the binding meanwhile run their calls normally."""
    real = lib()
    if getattr(_tls, "recorder", None) is not None:
        raise RuntimeError("plan() cannot be nested")
    rec = _Recorder(real)
    _tls.recorder = rec
    try:
        result = fn(*args, **kwargs)
    finally:
        _tls.recorder = None
    calls = rec.calls
    keep = rec.keep

    def replay():
        for name, f, a in calls:
            rc = f(*a)
            if rc != 0:
                raise QatError(rc, f"{name}: " + real.qat_last_error().decode())

    replay.calls = [c[0] for c in calls]
    replay.result = result
    replay.tensors = keep
    return replay


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return QAT_BF16
    if t == torch.float32:
        return QAT_F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    if t is None:
        return None
    rec = getattr(_tls, "recorder", None)
    if rec is not None:
        rec.keep.append(t)
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, device=True):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes: int, device, ws=None):
    if ws is not None:
        _need(ws, "ws", torch.uint8)
        if ws.numel() < nbytes:
            raise ValueError(f"workspace of {ws.numel()} bytes is smaller than the {nbytes} needed")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ ESA
def esa_params(*, batch, n_heads, head_dim, d_c, ctx_len, chunk_start, chunk_len, n_init, window, topk,
               radius, clip, scale=None, dtype=torch.bfloat16, correction="clamp", vote_tau=0.0,
               per_head=False) -> EsaParams:
    """correction: "clamp" (default reading) or "votes" (per-query softmax
    votes at temperature vote_tau; 0 means 1/sqrt(d_c), per head 1/sqrt(d)).
    per_head: one selection per (sequence, head) by esa_select_heads."""
    corr = {"clamp": QAT_CORR_CLAMP, "votes": QAT_CORR_VOTES}[correction]
    return EsaParams(batch, n_heads, head_dim, d_c, ctx_len, chunk_start, chunk_len, n_init, window, topk,
                     radius, float(clip), float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                     _dt(dtype), corr, float(vote_tau), 1 if per_head else 0)


def esa_workspace_size(p: EsaParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().esa_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def esa_compress(x, W, bias=None, out=None, out_dtype=torch.bfloat16, n=None, x_stride=None, out_stride=None,
                 ws=None):
    """out[i] = round(W x[i] + bias) (float64 accumulation). x: [n, d_model]
    rows (or a strided view described by n/x_stride over a contiguous base);
    W: [d_c, d_model]."""
    d_c, d_model = W.shape
    _need(W, "W", x.dtype)
    _need(bias, "bias", torch.float32)
    if n is None:
        _need(x, "x")
        n = x.shape[0]
        x_stride = d_model
    if out is None:
        out = torch.empty(n, d_c, dtype=out_dtype, device=x.device)
        out_stride = d_c
    elif out_stride is None:
        _need(out, "out")
        out_stride = d_c
    nb = ctypes.c_size_t(0)
    _check(lib().esa_compress_workspace_size(n, d_model, d_c, ctypes.byref(nb)))
    ws = _workspace(nb.value, x.device, ws)
    _check(lib().esa_compress(_ptr(x), n, x_stride, d_model, _dt(x.dtype), _ptr(W), _ptr(bias), d_c,
                              _ptr(out), out_stride, _dt(out.dtype), _ptr(ws), ws.numel(), _stream()))
    return out


def esa_select(p: EsaParams, q, Wq, bq, kc_cache, sel=None, n_sel=None, scores=None, want_scores=False, ws=None):
    """Returns (sel [batch, topk] int32, n_sel [batch] int32, scores or None)."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    _need(q, "q", dt)
    _need(Wq, "Wq", dt)
    _need(bq, "bq", torch.float32)
    _need(kc_cache, "kc_cache", torch.bfloat16)
    dev = q.device
    if sel is None:
        sel = torch.empty(p.batch, p.topk, dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty(p.batch, dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        n_mid = max(0, max(p.n_init, p.chunk_start - p.window) - p.n_init) if p.chunk_start > p.n_init else 0
        scores = torch.empty(p.batch, max(n_mid, 1), dtype=torch.float32, device=dev)
    ws = _workspace(esa_workspace_size(p), dev, ws)
    _check(lib().esa_select(ctypes.byref(p), _ptr(q), _ptr(Wq), _ptr(bq), _ptr(kc_cache), _ptr(sel),
                            _ptr(n_sel), _ptr(scores), _ptr(ws), ws.numel(), _stream()))
    return sel, n_sel, scores


def esa_select_heads(p: EsaParams, q, k_cache, sel=None, n_sel=None, scores=None, want_scores=False, ws=None):
    """Per-head selection. Returns (sel [batch, H, topk] int32, n_sel
    [batch, H] int32, scores [batch, H, |M|] or None)."""
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16)
    dev = q.device
    if sel is None:
        sel = torch.empty(p.batch, p.n_heads, p.topk, dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty(p.batch, p.n_heads, dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        n_mid = max(0, max(p.n_init, p.chunk_start - p.window) - p.n_init) if p.chunk_start > p.n_init else 0
        scores = torch.empty(p.batch, p.n_heads, max(n_mid, 1), dtype=torch.float32, device=dev)
    ws = _workspace(esa_workspace_size(p), dev, ws)
    _check(lib().esa_select_heads(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(sel), _ptr(n_sel), _ptr(scores),
                                  _ptr(ws), ws.numel(), _stream()))
    return sel, n_sel, scores


def esa_sparse_attn(p: EsaParams, q, k_cache, v_cache, sel, n_sel, out=None, lse=None, want_lse=True, ws=None):
    """Returns (out [batch, chunk_len, H, d], lse [batch, chunk_len, H] or None)."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, dt)
    _need(sel, "sel", torch.int32)
    _need(n_sel, "n_sel", torch.int32)
    dev = q.device
    if out is None:
        out = torch.empty(p.batch, p.chunk_len, p.n_heads, p.head_dim, dtype=dt, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(p.batch, p.chunk_len, p.n_heads, dtype=torch.float32, device=dev)
    ws = _workspace(esa_workspace_size(p), dev, ws)
    _check(lib().esa_sparse_attn(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sel), _ptr(n_sel),
                                 _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return out, lse


def esa_bwd_workspace_size(p: EsaParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().esa_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def esa_sparse_attn_bwd(p: EsaParams, q, k_cache, v_cache, sel, n_sel, dout, lse, dq=None, dk=None, dv=None,
                        ws=None):
    """Gradients of esa_sparse_attn with the selection held fixed (lse: that
    call's output). dk, dv [batch, ctx_len, H, d] float32 are ADDED to
    (allocated zeroed when None). Returns (dq [batch, chunk_len, H, d], dk, dv)."""
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (dout, "dout")):
        _need(t, name, torch.bfloat16)
    _need(sel, "sel", torch.int32)
    _need(n_sel, "n_sel", torch.int32)
    _need(lse, "lse", torch.float32)
    dev = q.device
    if dq is None:
        dq = torch.empty(p.batch, p.chunk_len, p.n_heads, p.head_dim, dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros(p.batch, p.ctx_len, p.n_heads, p.head_dim, dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.zeros(p.batch, p.ctx_len, p.n_heads, p.head_dim, dtype=torch.float32, device=dev)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, torch.float32)
    ws = _workspace(esa_bwd_workspace_size(p), dev, ws)
    _check(lib().esa_sparse_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sel), _ptr(n_sel),
                                     _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                                     _stream()))
    return dq, dk, dv


# ------------------------------------------------------------------ MoBA
def moba_params(*, batch, seq_len, n_q_heads, n_kv_heads, head_dim, q_start=0, q_len=None, block, topk,
                window=0, scale=None, dtype=torch.bfloat16) -> MobaParams:
    return MobaParams(batch, seq_len, n_q_heads, n_kv_heads, head_dim, q_start,
                      seq_len - q_start if q_len is None else q_len, block, topk, window,
                      float(scale if scale is not None else 1.0 / math.sqrt(head_dim)), _dt(dtype))


def moba_workspace_size(p: MobaParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moba_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moba_block_select(p: MobaParams, q, k, blk=None, ws=None):
    """Returns blk [batch, q_len, Hq, topk] int32 (ascending, -1 padded)."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    _need(q, "q", dt)
    _need(k, "k", dt)
    if blk is None:
        blk = torch.empty(p.batch, p.q_len, p.n_q_heads, p.topk, dtype=torch.int32, device=q.device)
    ws = _workspace(moba_workspace_size(p), q.device, ws)
    _check(lib().moba_block_select(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(blk), _ptr(ws), ws.numel(), _stream()))
    return blk


def moba_sparse_attn(p: MobaParams, q, k, v, blk, out=None, lse=None, want_lse=True, ws=None):
    """Returns (out [batch, q_len, Hq, d], lse [batch, q_len, Hq] or None)."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, dt)
    _need(blk, "blk", torch.int32)
    dev = q.device
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.n_q_heads, p.head_dim, dtype=dt, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(p.batch, p.q_len, p.n_q_heads, dtype=torch.float32, device=dev)
    ws = _workspace(moba_workspace_size(p), dev, ws)
    _check(lib().moba_sparse_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(blk), _ptr(out), _ptr(lse),
                                  _ptr(ws), ws.numel(), _stream()))
    return out, lse


def moba_block_means(p: MobaParams, k, first_block, n_blocks, kbar=None, ws=None):
    """Fills blocks [first_block, first_block + n_blocks) of the mean cache
    kbar [batch, seq_len // block, Hkv, d] float32 (allocated, zeroed, when
    None) and returns it."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    _need(k, "k", dt)
    if kbar is None:
        kbar = torch.zeros(p.batch, p.seq_len // p.block, p.n_kv_heads, p.head_dim, dtype=torch.float32,
                           device=k.device)
    _need(kbar, "kbar", torch.float32)
    ws = _workspace(moba_workspace_size(p), k.device, ws)
    _check(lib().moba_block_means(ctypes.byref(p), _ptr(k), int(first_block), int(n_blocks), _ptr(kbar), _ptr(ws),
                                  ws.numel(), _stream()))
    return kbar


def moba_decode_select(p: MobaParams, q, kbar, blk=None):
    """q: [batch, q_len, Hq, d] (the processed rows only). Returns blk
    [batch, q_len, Hq, topk] int32, as moba_block_select."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    _need(q, "q", dt)
    _need(kbar, "kbar", torch.float32)
    if blk is None:
        blk = torch.empty(p.batch, p.q_len, p.n_q_heads, p.topk, dtype=torch.int32, device=q.device)
    _check(lib().moba_decode_select(ctypes.byref(p), _ptr(q), _ptr(kbar), _ptr(blk), _stream()))
    return blk


def moba_decode_attn(p: MobaParams, q, k, v, blk, out=None, lse=None, want_lse=True, ws=None):
    """q: [batch, q_len, Hq, d] (the processed rows only); k, v the whole
    sequence. Returns (out [batch, q_len, Hq, d], lse [batch, q_len, Hq] or None)."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, dt)
    _need(blk, "blk", torch.int32)
    dev = q.device
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.n_q_heads, p.head_dim, dtype=dt, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(p.batch, p.q_len, p.n_q_heads, dtype=torch.float32, device=dev)
    ws = _workspace(moba_workspace_size(p), dev, ws)
    _check(lib().moba_decode_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(blk), _ptr(out), _ptr(lse),
                                  _ptr(ws), ws.numel(), _stream()))
    return out, lse


def moba_bwd_workspace_size(p: MobaParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moba_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moba_sparse_attn_bwd(p: MobaParams, q, k, v, blk, dout, lse, dq=None, dk=None, dv=None, ws=None):
    """Gradients of moba_sparse_attn for the same rows with the gating held
    fixed (lse: that call's output). Returns (dq [batch, q_len, Hq, d],
    dk, dv [batch, seq_len, Hkv, d]), all float32."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, name, dt)
    _need(blk, "blk", torch.int32)
    _need(lse, "lse", torch.float32)
    dev = q.device
    if dq is None:
        dq = torch.empty(p.batch, p.q_len, p.n_q_heads, p.head_dim, dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty(p.batch, p.seq_len, p.n_kv_heads, p.head_dim, dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty(p.batch, p.seq_len, p.n_kv_heads, p.head_dim, dtype=torch.float32, device=dev)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, torch.float32)
    ws = _workspace(moba_bwd_workspace_size(p), dev, ws)
    _check(lib().moba_sparse_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(blk), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv


# ------------------------------------------------------------------ CCA
def cca_params(*, batch, seq_len, n_q_heads, n_kv_heads, head_dim, group, window, q_start=0, q_len=None,
               scale=None) -> CcaParams:
    return CcaParams(batch, seq_len, n_q_heads, n_kv_heads, head_dim, q_start,
                     seq_len - q_start if q_len is None else q_len, group, window,
                     float(scale if scale is not None else 1.0 / math.sqrt(head_dim)), QAT_BF16)


def cca_pool(p: CcaParams, q, k, v, kc=None, vc=None):
    """Returns the core keys / values kc, vc [batch, seq_len // group, Hq, d]
    (bfloat16; allocated when None)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16)
    ng = p.seq_len // p.group
    if kc is None:
        kc = torch.empty(p.batch, max(ng, 1), p.n_q_heads, p.head_dim, dtype=torch.bfloat16, device=q.device)
    if vc is None:
        vc = torch.empty_like(kc)
    _check(lib().cca_pool(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _stream()))
    return kc, vc


def cca_attn(p: CcaParams, q, k, v, kc, vc, out=None, lse=None, want_lse=True):
    """Returns (out [batch, q_len, Hq, d] bfloat16, lse [batch, q_len, Hq] or None)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (kc, "kc"), (vc, "vc")):
        _need(t, name, torch.bfloat16)
    dev = q.device
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.n_q_heads, p.head_dim, dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(p.batch, p.q_len, p.n_q_heads, dtype=torch.float32, device=dev)
    _check(lib().cca_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), _ptr(lse),
                          _stream()))
    return out, lse


def moba_decode_attn_noalloc(p: MobaParams, q, k, v, blk, out, lse=None):
    """moba_decode_attn through the entry point that allocates nothing (its
    partials live in the library's fixed per-GPU scratch array): out (and
    lse, if wanted) must be given. Returns (out, lse)."""
    dt = torch.bfloat16 if p.dtype == QAT_BF16 else torch.float32
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, name, dt)
    _need(blk, "blk", torch.int32)
    _need(lse, "lse", torch.float32)
    _check(lib().moba_decode_attn_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(blk), _ptr(out),
                                          _ptr(lse), _stream()))
    return out, lse
