"""Python binding of libsepattn: SepLLM separator-sparse attention and the
SepCache streaming decode on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libsepattn.so`` (built from ``csrc/`` by ``build.py``); torch
supplies device memory and the current stream.  There is no fallback: if the
library is missing or cannot be loaded, every call raises.

Names follow the C ABI in ``include/sepattn.h``:

* ``build_index(tok, sep_ids, a, n)``          -> :class:`Index`
* ``fwd(q, k, v, index, scale)``                -> (o, lse)
* ``bwd(q, k, v, o, lse, dout, index, scale)``  -> (dq, dk, dv)
* :class:`SepCache` with ``init``, ``update`` and ``decode``
* ``rope_table(theta, c, d)``                   -> (cos, sin) fp32 host arrays
"""

import ctypes
import os

import numpy as np
import torch

__all__ = ["Index", "SepCache", "build_index", "fwd", "bwd", "attention", "rope_table", "load_library",
           "SepattnError", "QTILE", "KTILE", "QTILE_FIELDS"]

QTILE = 128
KTILE = 64
QTILE_FIELDS = 8
F32, BF16 = 0, 1

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsepattn.so")
_lib = None


class SepattnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = load_library().sepattn_strerror(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")


class _Index(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("S", ctypes.c_int), ("a", ctypes.c_int), ("n", ctypes.c_int),
                ("is_sep", ctypes.c_void_p), ("sep_prefix", ctypes.c_void_p),
                ("anchor_pos", ctypes.c_void_p), ("anchor_count", ctypes.c_void_p),
                ("qtile", ctypes.c_void_p), ("tile_class", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int), ("c", ctypes.c_int),
                ("a", ctypes.c_int), ("s", ctypes.c_int), ("w", ctypes.c_int),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("tok", ctypes.c_void_p), ("state", ctypes.c_void_p)]


EXPORTS = ["sepattn_strerror", "sepattn_index_bytes", "sepattn_index_bind", "sepattn_build_index",
           "sepattn_build_index_interval",
           "sepattn_fwd", "sepattn_bwd_workspace", "sepattn_bwd", "sepattn_bwd_profiled",
           "sepcache_init", "sepcache_update", "sepcache_prefill",
           "sepcache_decode_workspace", "sepcache_decode", "sepcache_decode_noalloc", "sepcache_decode_profiled",
           "sepattn_rope_table_host"]


def load_library(path=None):
    """Load libsepattn.so (torch must be imported first so the process uses
    torch's HIP runtime for both).  Raises if the library is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libsepattn.so not built at {p}; run python -m sparse_attention_sepattn_amd.build")
    L = ctypes.CDLL(p)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.sepattn_strerror.restype = ctypes.c_char_p
    L.sepattn_strerror.argtypes = [i32]
    L.sepattn_index_bytes.restype = sz
    L.sepattn_index_bytes.argtypes = [i32, i32]
    L.sepattn_index_bind.restype = i32
    L.sepattn_index_bind.argtypes = [vp, sz, i32, i32, ctypes.POINTER(_Index)]
    L.sepattn_build_index.restype = i32
    L.sepattn_build_index.argtypes = [vp, i32, i32, vp, i32, i32, i32, ctypes.POINTER(_Index), vp]
    L.sepattn_build_index_interval.restype = i32
    L.sepattn_build_index_interval.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(_Index), vp]
    L.sepattn_fwd.restype = i32
    L.sepattn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, ctypes.POINTER(_Index),
                              vp, vp, vp]
    L.sepattn_bwd_workspace.restype = sz
    L.sepattn_bwd_workspace.argtypes = [i32] * 6
    L.sepattn_bwd.restype = i32
    L.sepattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                              ctypes.POINTER(_Index), vp, vp, vp, vp, sz, vp]
    L.sepattn_bwd_profiled.restype = i32
    L.sepattn_bwd_profiled.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                       ctypes.POINTER(_Index), vp, vp, vp, vp, sz, vp, vp, i32]
    L.sepcache_init.restype = i32
    L.sepcache_init.argtypes = [ctypes.POINTER(_Cache), vp]
    L.sepcache_prefill.restype = i32
    L.sepcache_prefill.argtypes = [ctypes.POINTER(_Cache), vp, vp, vp, i32, ctypes.POINTER(_Index), vp]
    L.sepcache_update.restype = i32
    L.sepcache_update.argtypes = [ctypes.POINTER(_Cache), vp, vp, vp, vp, i32, vp]
    L.sepcache_decode_workspace.restype = sz
    L.sepcache_decode_workspace.argtypes = [ctypes.POINTER(_Cache), i32]
    L.sepcache_decode.restype = i32
    L.sepcache_decode.argtypes = [ctypes.POINTER(_Cache), vp, i32, vp, vp, f32, vp, vp, sz, vp]
    L.sepcache_decode_noalloc.restype = i32
    L.sepcache_decode_noalloc.argtypes = [ctypes.POINTER(_Cache), vp, i32, vp, vp, f32, vp, vp]
    L.sepcache_decode_profiled.restype = i32
    L.sepcache_decode_profiled.argtypes = [ctypes.POINTER(_Cache), vp, i32, vp, vp, f32, vp, vp, sz, vp, vp, i32]
    L.sepattn_rope_table_host.restype = i32
    L.sepattn_rope_table_host.argtypes = [ctypes.c_double, i32, i32, vp, vp]
    if path is None:
        _lib = L
    return L


def _check(status, what):
    if status != 0:
        raise SepattnError(status, what)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _host_ids(sep_ids):
    arr = np.ascontiguousarray(np.asarray(sep_ids, dtype=np.int32).reshape(-1))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class Index:
    """Device index of a batch of token sequences (see sepattn_index in
    include/sepattn.h).  Holds one device buffer and torch views into it."""

    def __init__(self, B, S, device="cuda"):
        L = load_library()
        nbytes = L.sepattn_index_bytes(B, S)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.st = _Index()
        _check(L.sepattn_index_bind(_ptr(self.buf), nbytes, B, S, ctypes.byref(self.st)), "index_bind")
        self.B, self.S = B, S
        QT = (S + QTILE - 1) // QTILE
        KT = (S + KTILE - 1) // KTILE
        base = self.buf.data_ptr()

        def view(addr, n, dt):
            off = addr - base
            esz = torch.tensor([], dtype=dt).element_size()
            return self.buf[off:off + n * esz].view(dt)

        self.is_sep = view(self.st.is_sep, B * S, torch.uint8).view(B, S)
        self.sep_prefix = view(self.st.sep_prefix, B * (S + 1), torch.int32).view(B, S + 1)
        self.anchor_pos = view(self.st.anchor_pos, B * S, torch.int32).view(B, S)
        self.anchor_count = view(self.st.anchor_count, B, torch.int32)
        self.qtile = view(self.st.qtile, B * QT * QTILE_FIELDS, torch.int32).view(B, QT, QTILE_FIELDS)
        self.tile_class = view(self.st.tile_class, B * QT * KT, torch.uint8).view(B, QT, KT)

    @property
    def a(self):
        return self.st.a

    @property
    def n(self):
        return self.st.n


def build_index(tok, sep_ids, a, n, index=None):
    """Separator flags, anchors and tile schedule of ``tok`` [B,S] int32."""
    _need(tok, "tok", torch.int32)
    B, S = tok.shape
    if index is None:
        index = Index(B, S, device=tok.device)
    ids, ids_p = _host_ids(sep_ids)
    _check(load_library().sepattn_build_index(_ptr(tok), B, S, ids_p, len(ids), a, n,
                                              ctypes.byref(index.st), _stream()), "build_index")
    return index


def build_index_interval(B, S, interval, a, n, index=None, device=None):
    """Index with anchors at fixed intervals (position j is an anchor iff
    j % interval == interval - 1) besides the ``a`` initial tokens."""
    if index is None:
        index = Index(B, S, device=device if device is not None else torch.device("cuda", torch.cuda.current_device()))
    _check(load_library().sepattn_build_index_interval(B, S, int(interval), a, n, ctypes.byref(index.st), _stream()),
           "build_index_interval")
    return index


def fwd(q, k, v, index, scale=None, o=None, lse=None):
    """Forward: q [B,Hq,S,d], k/v [B,Hkv,S,d] (bf16 or fp32) -> (o, lse)."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, Hkv, S, d), q.device)
    _need(v, "v", q.dtype, (B, Hkv, S, d), q.device)
    if scale is None:
        scale = d ** -0.5
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(o, "o", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, Hq, S), q.device)
    _check(load_library().sepattn_fwd(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, S, d, _dtype_code(q),
                                      float(scale), ctypes.byref(index.st), _ptr(o), _ptr(lse),
                                      _stream()), "fwd")
    return o, lse


def bwd_workspace_bytes(B, Hq, Hkv, S, d, dtype=torch.bfloat16):
    code = BF16 if dtype == torch.bfloat16 else F32
    return load_library().sepattn_bwd_workspace(B, Hq, Hkv, S, d, code)


def bwd(q, k, v, o, lse, dout, index, scale=None, dq=None, dk=None, dv=None, ws=None, events=None):
    """Backward: gradients of sum(o * dout) -> (dq, dk, dv).  ``events``: an
    optional sequence of 4 hipEvent_t handles (ints) recorded around the three
    kernels (see sepattn_bwd_profiled)."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for t, name in ((q, "q"), (o, "o"), (dout, "dout")):
        _need(t, name, q.dtype, q.shape, dev)
    _need(k, "k", q.dtype, (B, Hkv, S, d), dev)
    _need(v, "v", q.dtype, (B, Hkv, S, d), dev)
    _need(lse, "lse", torch.float32, (B, Hq, S), dev)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, q.shape, dev)
    _need(dk, "dk", q.dtype, k.shape, dev)
    _need(dv, "dv", q.dtype, v.shape, dev)
    L = load_library()
    nbytes = L.sepattn_bwd_workspace(B, Hq, Hkv, S, d, _dtype_code(q))
    if ws is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _need(ws, "ws", torch.uint8, None, dev)  # its size is checked by the library (EWORKSPACE)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), B, Hq, Hkv, S, d, _dtype_code(q),
            float(scale), ctypes.byref(index.st), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream())
    if events is None:
        _check(L.sepattn_bwd(*args), "bwd")
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(L.sepattn_bwd_profiled(*args, arr, len(events)), "bwd_profiled")
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """fwd in forward, bwd in backward (the saved O and LSE are the
    forward's, as in training)."""

    @staticmethod
    def forward(ctx, q, k, v, index, scale):
        o, lse = fwd(q, k, v, index, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.index, ctx.scale = index, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.index, ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, index, scale=None):
    """SepLLM attention of q [B,Hq,S,d] over k/v [B,Hkv,S,d] under ``index``
    (from build_index), differentiable through torch.autograd: the forward
    and the backward are the library's kernels."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _Attention.apply(q, k, v, index, float(scale))


def rope_table(theta, c, d):
    """(cos, sin) float32 numpy arrays [c, d/2] from the library's host helper."""
    cos = np.empty((c, d // 2), dtype=np.float32)
    sin = np.empty((c, d // 2), dtype=np.float32)
    _check(load_library().sepattn_rope_table_host(float(theta), c, d, cos.ctypes.data_as(ctypes.c_void_p),
                                                  sin.ctypes.data_as(ctypes.c_void_p)), "rope_table")
    return cos, sin


class SepCache:
    """Batched SepCache in device tensors (see sepcache in include/sepattn.h).

    k/v [B,Hkv,c,d] bf16 (rows stored without rotary embedding), pos/tok
    [B,c] int32, state [B,4] int32 (n_init, n_sep, n_win, tokens seen)."""

    def __init__(self, B, Hkv, d, c, a, s, w, device="cuda"):
        self.B, self.Hkv, self.d, self.c, self.a, self.s, self.w = B, Hkv, d, c, a, s, w
        self.k = torch.zeros((B, Hkv, c, d), dtype=torch.bfloat16, device=device)
        self.v = torch.zeros((B, Hkv, c, d), dtype=torch.bfloat16, device=device)
        self.pos = torch.empty((B, c), dtype=torch.int32, device=device)
        self.tok = torch.empty((B, c), dtype=torch.int32, device=device)
        self.state = torch.empty((B, 4), dtype=torch.int32, device=device)
        self.st = _Cache(B, Hkv, d, c, a, s, w, self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(),
                         self.tok.data_ptr(), self.state.data_ptr())
        self._ws = None
        self.init()

    def init(self):
        _check(load_library().sepcache_init(ctypes.byref(self.st), _stream()), "sepcache_init")

    def update(self, k_new, v_new, tok_new, sep_ids):
        dev = self.k.device
        _need(k_new, "k_new", torch.bfloat16, (self.B, self.Hkv, self.d), dev)
        _need(v_new, "v_new", torch.bfloat16, (self.B, self.Hkv, self.d), dev)
        _need(tok_new, "tok_new", torch.int32, (self.B,), dev)
        ids, ids_p = _host_ids(sep_ids)
        _check(load_library().sepcache_update(ctypes.byref(self.st), _ptr(k_new), _ptr(v_new), _ptr(tok_new),
                                              ids_p, len(ids), _stream()), "sepcache_update")

    def prefill(self, k, v, tok, index):
        """Set the caches to what streaming the prompt ``tok`` [B,P] (rows
        k/v [B,Hkv,P,d] bf16) through ``update`` would leave; ``index`` is
        build_index(tok, sep_ids, a, n) with this cache's ``a``."""
        dev = self.k.device
        _need(tok, "tok", torch.int32, None, dev)
        B, P = tok.shape
        _need(k, "k", torch.bfloat16, (self.B, self.Hkv, P, self.d), dev)
        _need(v, "v", torch.bfloat16, (self.B, self.Hkv, P, self.d), dev)
        _check(load_library().sepcache_prefill(ctypes.byref(self.st), _ptr(k), _ptr(v), _ptr(tok), P,
                                               ctypes.byref(index.st), _stream()), "sepcache_prefill")

    def workspace_bytes(self, Hq):
        return load_library().sepcache_decode_workspace(ctypes.byref(self.st), Hq)

    def decode(self, q, rope_cos, rope_sin, scale=None, o=None, ws=None, events=None):
        """Decode attention of the newest token; ``events``: optional 3
        hipEvent_t handles recorded around the two kernels."""
        B, Hq, d = q.shape
        dev = self.k.device
        _need(q, "q", torch.bfloat16, (self.B, Hq, self.d), dev)
        _need(rope_cos, "rope_cos", torch.float32, (self.c, self.d // 2), dev)
        _need(rope_sin, "rope_sin", torch.float32, (self.c, self.d // 2), dev)
        if scale is None:
            scale = d ** -0.5
        if o is None:
            o = torch.empty_like(q)
        _need(o, "o", torch.bfloat16, (self.B, Hq, self.d), dev)
        L = load_library()
        nbytes = L.sepcache_decode_workspace(ctypes.byref(self.st), Hq)
        if ws is None:
            if self._ws is None or self._ws.numel() < nbytes:
                self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
            ws = self._ws
        _need(ws, "ws", torch.uint8, None, dev)  # its size is checked by the library (EWORKSPACE)
        args = (ctypes.byref(self.st), _ptr(q), Hq, _ptr(rope_cos), _ptr(rope_sin), float(scale), _ptr(o),
                _ptr(ws), ws.numel(), _stream())
        if events is None:
            _check(L.sepcache_decode(*args), "sepcache_decode")
        else:
            arr = (ctypes.c_void_p * len(events))(*events)
            _check(L.sepcache_decode_profiled(*args, arr, len(events)), "sepcache_decode_profiled")
        return o

    def decode_noalloc(self, q, rope_cos, rope_sin, scale=None, o=None):
        """``decode`` through sepcache_decode_noalloc: no workspace, the
        library's fixed per-device scratch holds the partials (calls that
        overlap on one GPU race)."""
        B, Hq, d = q.shape
        dev = self.k.device
        _need(q, "q", torch.bfloat16, (self.B, Hq, self.d), dev)
        _need(rope_cos, "rope_cos", torch.float32, (self.c, self.d // 2), dev)
        _need(rope_sin, "rope_sin", torch.float32, (self.c, self.d // 2), dev)
        if scale is None:
            scale = d ** -0.5
        if o is None:
            o = torch.empty_like(q)
        _need(o, "o", torch.bfloat16, (self.B, Hq, self.d), dev)
        _check(load_library().sepcache_decode_noalloc(ctypes.byref(self.st), _ptr(q), Hq, _ptr(rope_cos),
                                                      _ptr(rope_sin), float(scale), _ptr(o), _stream()),
               "sepcache_decode_noalloc")
        return o
