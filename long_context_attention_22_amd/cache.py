"""Binding of the paged heterogeneous KV cache (include/lca_cache.h).

"DeepSeek-V4 中文翻译" section 3.5.1: compressed CSA / HCA entries live in a classical cache
of blocks (any multiple of lcm(m, m') raw tokens per block); sliding-window rows and the
uncompressed tail live in a fixed, preallocated state-cache pool handed out per sequence.
Section 3.5.2: a shared prefix's stored entries are reused rather than prefilled again.

The library keeps every plane of the cache in one reserved virtual range laid out as the
[B][cap][...] planes the attention, indexer and compressor calls take, backed page by page from a
pool (classical streams) or whole (state streams).  PagedCache.kv(name) returns a KV whose
tensors view those ranges, for the calls of this package as they are.  Only rows a slot has
reserved (PagedCache.reserve) may be touched; the views must not outlive the cache.
"""
from __future__ import annotations

import ctypes as C
import math
from dataclasses import dataclass

import torch

from . import BF16, F32, FP8, KV, MXFP4, LcaError, lib

_DLROCM = 10  # DLPack device type of ROCm devices
_DL_CODES = {torch.uint8: (1, 8), torch.bfloat16: (4, 16), torch.float32: (2, 32)}


class _Plane(C.Structure):
    _fields_ = [("row_bytes", C.c_int64), ("rows", C.c_int64), ("m", C.c_int32), ("reserved", C.c_int32)]


class _Stats(C.Structure):
    _fields_ = [("pool_pages", C.c_int64), ("free_pages", C.c_int64), ("mapped_pages", C.c_int64),
                ("shared_pages", C.c_int64), ("device_bytes", C.c_int64), ("page_bytes", C.c_int64),
                ("open_slots", C.c_int32), ("max_seqs", C.c_int32)]


class _DLDevice(C.Structure):
    _fields_ = [("device_type", C.c_int32), ("device_id", C.c_int32)]


class _DLDataType(C.Structure):
    _fields_ = [("code", C.c_uint8), ("bits", C.c_uint8), ("lanes", C.c_uint16)]


class _DLTensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("device", _DLDevice), ("ndim", C.c_int32), ("dtype", _DLDataType),
                ("shape", C.POINTER(C.c_int64)), ("strides", C.POINTER(C.c_int64)), ("byte_offset", C.c_uint64)]


class _DLManaged(C.Structure):
    _fields_ = [("dl_tensor", _DLTensor), ("manager_ctx", C.c_void_p), ("deleter", C.c_void_p)]


_bound = False


def _lib():
    global _bound
    L = lib()
    if not _bound:
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.lca_cache_create.argtypes = [C.POINTER(_Plane), i32, i32, i64, i64, C.POINTER(vp)]
        L.lca_cache_destroy.argtypes = [vp]
        L.lca_cache_plane_base.argtypes = [vp, i32, C.POINTER(vp)]
        L.lca_cache_open.argtypes = [vp, C.POINTER(i32)]
        L.lca_cache_reserve.argtypes = [vp, i32, i64]
        L.lca_cache_fork.argtypes = [vp, i32, i64, vp, C.POINTER(i32)]
        L.lca_cache_close.argtypes = [vp, i32]
        L.lca_cache_tokens.argtypes = [vp, i32, C.POINTER(i64)]
        L.lca_cache_get_stats.argtypes = [vp, C.POINTER(_Stats)]
        for n in ("create", "destroy", "plane_base", "open", "reserve", "fork", "close", "tokens", "get_stats"):
            getattr(L, "lca_cache_" + n).restype = C.c_int
        _bound = True
    return L


def _check(rc: int):
    if rc != 0:
        raise LcaError(rc, lib().lca_last_error().decode())


@dataclass
class CacheStream:
    """One KV stream kept in the cache.  m >= 1: classical stream of compressed entries (one row per m
    raw tokens), `rows` entries per sequence at most (rounded up to whole pages); m = 0: state-cache
    ring of exactly `rows` rows per sequence (sliding-window rows)."""
    name: str
    fmt: int
    d_nope: int
    d_rope: int
    m: int
    rows: int


def _planes_of(s: CacheStream):
    """(plane name, torch dtype, elements per row) of a stream's storage planes (the KV layout)."""
    if s.fmt == F32:
        out = [("nope", torch.float32, s.d_nope), ("rope", torch.float32, s.d_rope)]
    elif s.fmt == BF16:
        out = [("nope", torch.bfloat16, s.d_nope), ("rope", torch.bfloat16, s.d_rope)]
    elif s.fmt == FP8:
        out = [("nope", torch.uint8, s.d_nope), ("rope", torch.bfloat16, s.d_rope),
               ("scale", torch.float32, s.d_nope // 128)]
    elif s.fmt == MXFP4:
        out = [("nope", torch.uint8, s.d_nope // 2), ("scale", torch.uint8, s.d_nope // 32)]
    else:
        raise ValueError(s.fmt)
    return [p for p in out if p[2] > 0]


def _row_bytes(dt, n):
    return n * torch.empty(0, dtype=dt).element_size()


class PagedCache:
    """Paged KV cache of max_seqs sequence slots (slot b = sequence b of a batch)."""

    def __init__(self, streams: list[CacheStream], max_seqs: int, page_bytes: int = 2 << 20, pool_pages: int = 0):
        """page_bytes: 2 MiB by default.  Smaller pages share prefixes at a finer grain, but on MI355X
        decode over 64 KiB pages ran about 9% slower than over contiguous memory (address-translation
        misses), while 2 MiB pages matched it."""
        self.streams = {s.name: s for s in streams}
        self.max_seqs, self.page_bytes = max_seqs, page_bytes
        self._keep = []
        descs, layout = [], []
        for s in streams:
            planes = _planes_of(s)
            if s.m > 0:  # cap: whole pages in every plane
                unit = 1
                for _, dt, n in planes:
                    rb = _row_bytes(dt, n)
                    unit = math.lcm(unit, page_bytes // math.gcd(page_bytes, rb))
                cap = -(-s.rows // unit) * unit
            else:
                cap = s.rows
            for pname, dt, n in planes:
                descs.append(_Plane(_row_bytes(dt, n), cap, s.m, 0))
                layout.append((s.name, pname, dt, n, cap))
        arr = (_Plane * len(descs))(*descs)
        h = C.c_void_p()
        _check(_lib().lca_cache_create(arr, len(descs), max_seqs, page_bytes, pool_pages, C.byref(h)))
        self._h = h
        dev = torch.cuda.current_device()
        self._kv = {}
        views, caps = {}, {}
        for i, (sname, pname, dt, n, cap) in enumerate(layout):
            base = C.c_void_p()
            _check(_lib().lca_cache_plane_base(self._h, i, C.byref(base)))
            views[(sname, pname)] = self._view(base.value, (max_seqs, cap, n), dt, dev)
            caps[sname] = cap
        for s in streams:
            v = lambda p: views.get((s.name, p))
            self._kv[s.name] = KV(v("nope"), v("rope"), v("scale"), s.fmt, s.d_nope, s.d_rope, caps[s.name])

    def _view(self, ptr: int, shape, dt, dev: int) -> torch.Tensor:
        """A torch tensor over device memory the cache owns (DLPack, no copy, no deleter)."""
        nd = len(shape)
        shp = (C.c_int64 * nd)(*shape)
        st = [1] * nd
        for i in range(nd - 2, -1, -1):
            st[i] = st[i + 1] * shape[i + 1]
        strides = (C.c_int64 * nd)(*st)
        code, bits = _DL_CODES[dt]
        mt = _DLManaged(_DLTensor(C.c_void_p(ptr), _DLDevice(_DLROCM, dev), nd, _DLDataType(code, bits, 1),
                                  C.cast(shp, C.POINTER(C.c_int64)), C.cast(strides, C.POINTER(C.c_int64)), 0),
                        None, None)
        self._keep += [shp, strides, mt]
        new = C.pythonapi.PyCapsule_New
        new.restype, new.argtypes = C.py_object, [C.c_void_p, C.c_char_p, C.c_void_p]
        cap = new(C.addressof(mt), b"dltensor", None)
        return torch.utils.dlpack.from_dlpack(cap)

    def kv(self, name: str) -> KV:
        return self._kv[name]

    def open(self) -> int:
        s = C.c_int32()
        _check(_lib().lca_cache_open(self._h, C.byref(s)))
        return s.value

    def reserve(self, slot: int, n_tokens: int):
        _check(_lib().lca_cache_reserve(self._h, int(slot), int(n_tokens)))

    def fork(self, parent: int, n_tokens: int, stream=None) -> int:
        if stream is None:
            stream = torch.cuda.current_stream()
        s = C.c_int32()
        _check(_lib().lca_cache_fork(self._h, int(parent), int(n_tokens), C.c_void_p(stream.cuda_stream),
                                     C.byref(s)))
        return s.value

    def close(self, slot: int):
        _check(_lib().lca_cache_close(self._h, int(slot)))

    def tokens(self, slot: int) -> int:
        n = C.c_int64()
        _check(_lib().lca_cache_tokens(self._h, int(slot), C.byref(n)))
        return n.value

    def stats(self) -> dict:
        st = _Stats()
        _check(_lib().lca_cache_get_stats(self._h, C.byref(st)))
        return {f: getattr(st, f) for f, _ in _Stats._fields_}

    def destroy(self):
        if getattr(self, "_h", None):
            _check(_lib().lca_cache_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
