"""Python access to the plain C fp64 oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never calls it and
it never serves as a fallback for it.

Arrays are numpy: float32 for f32, uint16 bit patterns for bf16, uint8 codes
for fp8, and for MXFP4 uint8 bytes holding two E2M1 codes (even element in the
low nibble) with uint8 E8M0 scale bytes, one per 32 elements.  Shapes follow the library's layouts ([B][rows][dims], row-major).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3
_lib = None


def lib():
    """The built oracle library; LCA_ORACLE_LIB names another build of oracle.c (the sanitizer test)."""
    global _lib
    if _lib is None:
        path = os.environ.get("LCA_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


class _KV(C.Structure):
    _fields_ = [("nope", C.c_void_p), ("rope", C.c_void_p), ("scale", C.c_void_p),
                ("fmt", C.c_int32), ("d_nope", C.c_int32), ("d_rope", C.c_int32),
                ("cap", C.c_int64)]


def _declare(L):
    vp, i32, i64, f64 = C.c_void_p, C.c_int32, C.c_int64, C.c_double
    L.orc_bf16_to_f64.argtypes = [C.c_uint16]
    L.orc_bf16_to_f64.restype = f64
    L.orc_f32_to_bf16.argtypes = [C.c_float]
    L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_fp8_to_f64.argtypes = [C.c_uint8]
    L.orc_fp8_to_f64.restype = f64
    L.orc_f64_to_fp8.argtypes = [f64]
    L.orc_f64_to_fp8.restype = C.c_uint8
    L.orc_e2m1_to_f64.argtypes = [C.c_uint8]
    L.orc_e2m1_to_f64.restype = f64
    L.orc_f64_to_e2m1.argtypes = [f64]
    L.orc_f64_to_e2m1.restype = C.c_uint8
    L.orc_mxfp4_block.argtypes = [vp, vp]
    L.orc_mxfp4_block.restype = C.c_uint8
    L.orc_indexer_score_mxfp4.argtypes = [vp, i32, vp, _KV, i32, i32, i32, i32, vp, i32, vp, i32, i64]
    L.orc_indexer_score_mxfp4.restype = C.c_int
    L.orc_linear.argtypes = [vp, i32, i64, i64, vp, i32, i64, i64, vp, i32, i64, i64, i32, i32, i32, i32]
    L.orc_linear.restype = C.c_int
    L.orc_grouped_out_proj.argtypes = [vp, i32, i32, i32, i32, i32, vp, i32, vp, i32, i32, vp, i32]
    L.orc_grouped_out_proj.restype = C.c_int
    L.orc_kv_decode.argtypes = [_KV, i64, i64, i64, vp]
    L.orc_kv_decode.restype = None
    L.orc_kv_compress.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, f64, f64, i32, i32, i32, i64,
                                  vp, _KV, i32]
    L.orc_kv_compress.restype = i64
    L.orc_indexer_score.argtypes = [vp, i32, vp, vp, i32, i64, i32, i32, i32, i32, vp, i32, vp, i32,
                                    i64]
    L.orc_indexer_score.restype = C.c_int
    L.orc_topk_select.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, vp]
    L.orc_topk_select.restype = C.c_int
    L.orc_attention.argtypes = [vp, i32, i32, i32, i32, vp, _KV, i32, vp, i32, _KV, i32, vp, f64,
                                f64, vp, i32, vp]
    L.orc_attention.restype = C.c_int


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _fmt_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported array dtype {a.dtype}")


@dataclass
class KV:
    """Stored KV rows: planes nope [B][cap][d_nope], rope [B][cap][d_rope], scale [B][cap][d_nope/128]."""
    nope: np.ndarray
    rope: np.ndarray
    scale: np.ndarray | None
    fmt: int
    d_nope: int
    d_rope: int
    cap: int

    @staticmethod
    def empty(fmt: int, B: int, cap: int, d_nope: int, d_rope: int) -> "KV":
        if fmt == F32:
            nope = np.zeros((B, cap, d_nope), np.float32)
            rope = np.zeros((B, cap, d_rope), np.float32)
            scale = None
        elif fmt == BF16:
            nope = np.zeros((B, cap, d_nope), np.uint16)
            rope = np.zeros((B, cap, d_rope), np.uint16)
            scale = None
        elif fmt == FP8:
            assert d_nope % 128 == 0
            nope = np.zeros((B, cap, d_nope), np.uint8)
            rope = np.zeros((B, cap, d_rope), np.uint16)
            scale = np.ones((B, cap, d_nope // 128), np.float32)
        elif fmt == MXFP4:
            assert d_nope % 32 == 0 and d_rope == 0
            nope = np.zeros((B, cap, d_nope // 2), np.uint8)
            rope = np.zeros((B, cap, 0), np.uint16)
            scale = np.full((B, cap, d_nope // 32), 127, np.uint8)
        else:
            raise ValueError(fmt)
        return KV(nope, rope, scale, fmt, d_nope, d_rope, cap)

    def c(self) -> _KV:
        for a in (self.nope, self.rope, self.scale):
            assert a is None or a.flags.c_contiguous
        return _KV(self.nope.ctypes.data, self.rope.ctypes.data,
                   None if self.scale is None else self.scale.ctypes.data,
                   self.fmt, self.d_nope, self.d_rope, self.cap)

    def decode(self, b: int, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        if nrows is None:
            nrows = self.cap - row0
        out = np.zeros((nrows, self.d_nope + self.d_rope), np.float64)
        lib().orc_kv_decode(self.c(), b, row0, nrows, _p(out))
        return out


def bf16_to_f64(h: int) -> float:
    return lib().orc_bf16_to_f64(int(h))


def f32_to_bf16(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(x)))


def fp8_to_f64(code: int) -> float:
    return lib().orc_fp8_to_f64(int(code))


def f64_to_fp8(x: float) -> int:
    return int(lib().orc_f64_to_fp8(float(x)))


def e2m1_to_f64(code: int) -> float:
    return lib().orc_e2m1_to_f64(int(code))


def f64_to_e2m1(x: float) -> int:
    return int(lib().orc_f64_to_e2m1(float(x)))


def mxfp4_block(v) -> tuple[int, np.ndarray]:
    """32 values -> (E8M0 scale byte, 32 E2M1 codes)."""
    v = np.ascontiguousarray(np.asarray(v, np.float64).reshape(32))
    codes = np.zeros(32, np.uint8)
    sc = lib().orc_mxfp4_block(_p(v), _p(codes))
    return int(sc), codes


def mxfp4_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """[..., d] values (d % 32 == 0) -> (codes [..., d] uint8, scale bytes [..., d/32] uint8)."""
    x = np.asarray(x, np.float64)
    blocks = x.reshape(-1, 32)
    codes = np.zeros(blocks.shape, np.uint8)
    scales = np.zeros(blocks.shape[0], np.uint8)
    for i, blk in enumerate(blocks):
        scales[i], codes[i] = mxfp4_block(blk)
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1] + (x.shape[-1] // 32,))


def kv_compress(c_a, z_a, c_b, z_b, out: KV, *, m: int, overlap: int, first_pos,
                bias_a=None, bias_b=None, gamma=None, eps: float = 1e-6,
                rope_theta: float = 0.0, ring: int = 0) -> int:
    """Compress [B][n_rows][c] inputs into `out` (in place).  Returns entries written."""
    B, n_rows, c = c_a.shape
    assert c == out.d_nope + out.d_rope
    fmt = _fmt_of(c_a)
    arrs = [np.ascontiguousarray(a) if a is not None else None for a in (c_a, z_a, c_b, z_b)]
    for a in arrs:
        assert a is None or (a.shape == c_a.shape and a.dtype == c_a.dtype)
    fp = np.ascontiguousarray(np.asarray(first_pos, np.int64).reshape(B))
    ba = None if bias_a is None else np.ascontiguousarray(bias_a, np.float32)
    bb = None if bias_b is None else np.ascontiguousarray(bias_b, np.float32)
    g = None if gamma is None else np.ascontiguousarray(gamma, np.float32)
    n = lib().orc_kv_compress(_p(arrs[0]), _p(arrs[1]), _p(arrs[2]), _p(arrs[3]), fmt, _p(ba), _p(bb),
                              _p(g), float(eps), float(rope_theta), int(m), int(overlap), int(B),
                              int(n_rows), _p(fp), out.c(), int(ring))
    if n < 0:
        raise ValueError("orc_kv_compress rejected its arguments")
    return int(n)


def indexer_score(q, w, k, *, q_pos, m: int, score_fmt: int, s_stride: int | None = None,
                  out=None):
    """q [B][T][H_I][d_I], w [B][T][H_I] or None, k [B][cap][d_I] -> scores [B][T][s_stride]."""
    B, T, H_I, d_I = q.shape
    k_cap = k.shape[1]
    if s_stride is None:
        s_stride = k_cap
    if out is None:
        out = np.zeros((B, T, s_stride), np.float32 if score_fmt == F32 else np.uint16)
    qp = np.ascontiguousarray(np.asarray(q_pos, np.int64).reshape(B))
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    wc = None if w is None else np.ascontiguousarray(w, np.float32)
    rc = lib().orc_indexer_score(_p(q), _fmt_of(q), _p(wc), _p(k), _fmt_of(k), k_cap, H_I, d_I, B, T,
                                 _p(qp), m, _p(out), score_fmt, s_stride)
    assert rc == 0
    return out


def indexer_score_mxfp4(q, w, k: KV, *, q_pos, m: int, score_fmt: int, s_stride: int | None = None,
                        out=None):
    """q [B][T][H_I][d_I] (f32 or bf16 bits), keys stored MXFP4 in `k` -> scores [B][T][s_stride]."""
    B, T, H_I, d_I = q.shape
    assert k.fmt == MXFP4 and k.d_nope == d_I
    if s_stride is None:
        s_stride = k.cap
    if out is None:
        out = np.zeros((B, T, s_stride), np.float32 if score_fmt == F32 else np.uint16)
    qp = np.ascontiguousarray(np.asarray(q_pos, np.int64).reshape(B))
    q = np.ascontiguousarray(q)
    wc = None if w is None else np.ascontiguousarray(w, np.float32)
    rc = lib().orc_indexer_score_mxfp4(_p(q), _fmt_of(q), _p(wc), k.c(), H_I, d_I, B, T, _p(qp), m,
                                       _p(out), score_fmt, s_stride)
    assert rc == 0
    return out


def topk_select(scores, *, q_pos, m: int, k: int):
    B, T, s_stride = scores.shape
    scores = np.ascontiguousarray(scores)
    idx = np.zeros((B, T, k), np.int32)
    qp = np.ascontiguousarray(np.asarray(q_pos, np.int64).reshape(B))
    rc = lib().orc_topk_select(_p(scores), _fmt_of(scores), s_stride, B, T, _p(qp), m, k, _p(idx))
    assert rc == 0
    return idx


def attention(q, *, q_pos, comp: KV, m: int, idx=None, win: KV | None = None, n_win: int = 0,
              sink=None, sm_scale: float, rope_theta: float = 0.0, out_fmt: int = F32,
              want_lse: bool = True):
    """q [B][T][H][c].  idx [B][T][k] (CSA) or None (HCA).  Returns (out, lse)."""
    B, T, H, c = q.shape
    q = np.ascontiguousarray(q)
    qp = np.ascontiguousarray(np.asarray(q_pos, np.int64).reshape(B))
    out = np.zeros((B, T, H, c), np.float32 if out_fmt == F32 else np.uint16)
    lse = np.zeros((B, T, H), np.float32) if want_lse else None
    if win is None:
        win = KV.empty(comp.fmt if comp.fmt != FP8 else BF16, 1, 1, comp.d_nope, comp.d_rope)
        n_win = 0
    k = 0
    if idx is not None:
        idx = np.ascontiguousarray(idx, np.int32)
        k = idx.shape[2]
    sk = None if sink is None else np.ascontiguousarray(sink, np.float32)
    rc = lib().orc_attention(_p(q), _fmt_of(q), H, B, T, _p(qp), comp.c(), m, _p(idx), k, win.c(),
                             n_win, _p(sk), float(sm_scale), float(rope_theta), _p(out), out_fmt,
                             _p(lse))
    assert rc == 0
    return out, lse


def linear(x, w, *, y_fmt: int = F32):
    """x [batch][M][K] (or [M][K]), w [batch][N][K] (or [N][K]) -> y [batch][M][N] (f32 or bf16 bits)."""
    x2, w2 = np.ascontiguousarray(x), np.ascontiguousarray(w)
    squeeze = x2.ndim == 2
    if squeeze:
        x2, w2 = x2[None], w2[None]
    bt, M, K = x2.shape
    N = w2.shape[1]
    y = np.zeros((bt, M, N), np.float32 if y_fmt == F32 else np.uint16)
    rc = lib().orc_linear(_p(x2), _fmt_of(x2), K, M * K, _p(w2), _fmt_of(w2), K, N * K, _p(y), y_fmt, N, M * N,
                          M, N, K, bt)
    assert rc == 0
    return y[0] if squeeze else y


def grouped_out_proj(o, wg, wo, *, g: int, mid_fmt: int = BF16, out_fmt: int = F32):
    """o [T][H][c], wg [g][d_g][H/g*c] bf16 bits, wo [d][g*d_g] bf16 bits -> out [T][d]."""
    o = np.ascontiguousarray(o)
    T, H, c = o.shape
    d_g, d = wg.shape[1], wo.shape[0]
    out = np.zeros((T, d), np.float32 if out_fmt == F32 else np.uint16)
    rc = lib().orc_grouped_out_proj(_p(o), _fmt_of(o), T, H, c, g, _p(np.ascontiguousarray(wg)), d_g,
                                    _p(np.ascontiguousarray(wo)), d, mid_fmt, _p(out), out_fmt)
    assert rc == 0
    return out
