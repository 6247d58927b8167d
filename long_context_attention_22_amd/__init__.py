"""Python binding of the MI355X compressed-attention library (liblca.so, C ABI in include/lca.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no
fallback: when the built library is missing every call raises.

Calls (same names as the C ABI):
    kv_compress, indexer_score, indexer_score_mxfp4, topk_select, indexer_topk, indexer_topk_mxfp4,
    csa_attn, hca_attn,
    csa_attn_append, hca_attn_append, linear, grouped_out_proj
and helpers KV (the lca_kv storage planes), attn_workspace_size.  The paged cache
(include/lca_cache.h) is bound in the cache module (PagedCache).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3
# status codes (LcaError.code)
OK, EINVAL, ESHAPE, EDTYPE, EALIGN, EWORKSPACE, EHIP, ENOMEM = range(8)
MAX_BATCH = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
# (LCA_LIB names another build of the same sources, e.g. the host-sanitizer build the tests make)
LIB_PATH = os.environ.get("LCA_LIB", os.path.join(_HERE, "liblca.so"))
_lib = None


class LcaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lca error {code}: {msg}")
        self.code = code


class _KV(C.Structure):
    _fields_ = [("nope", C.c_void_p), ("rope", C.c_void_p), ("scale", C.c_void_p),
                ("fmt", C.c_int32), ("d_nope", C.c_int32), ("d_rope", C.c_int32),
                ("cap", C.c_int64)]


def lib():
    """Load liblca.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_attention_22_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32, f64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_size_t
        L.lca_version.restype = C.c_int
        L.lca_last_error.restype = C.c_char_p
        L.lca_kv_compress.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, f32, f64, i32, i32, i32, i64, i64,
                                      vp, _KV, i32, vp]
        L.lca_kv_compress_ws.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, f32, f64, i32, i32, i32, i64, i64,
                                         vp, _KV, i32, vp, sz, vp]
        L.lca_compress_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.lca_compress_workspace_size.restype = sz
        L.lca_indexer_score.argtypes = [vp, vp, vp, i32, i64, i32, i32, i32, i32, vp, i32, vp, i32, i64,
                                        vp]
        L.lca_indexer_score_mxfp4.argtypes = [vp, vp, _KV, i32, i32, i32, i32, vp, i32, vp, i32, i64, vp]
        L.lca_topk_select.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, vp, vp, sz, vp]
        L.lca_topk_workspace_size.argtypes = [i32, i32, i64, i32]
        L.lca_topk_workspace_size.restype = sz
        L.lca_csa_attn.argtypes = [vp, i32, i32, i32, i32, vp, _KV, i32, vp, i32, _KV, i32, vp, f32, f64,
                                   vp, i32, vp, vp, sz, vp]
        L.lca_hca_attn.argtypes = [vp, i32, i32, i32, i32, vp, _KV, i32, _KV, i32, vp, f32, f64, vp, i32,
                                   vp, vp, sz, vp]
        L.lca_hca_attn_noalloc.argtypes = [vp, i32, i32, i32, i32, vp, _KV, i32, _KV, i32, vp, f32, f64, vp, i32,
                                           vp, vp]
        L.lca_csa_attn_append.argtypes = [vp, i32, i32, i32, i32, vp, _KV, i32, vp, i32, _KV, i32, vp, i32, i64,
                                          vp, f32, vp, f32, f64, vp, i32, vp, vp, sz, vp]
        L.lca_hca_attn_append.argtypes = [vp, i32, i32, i32, i32, vp, _KV, i32, _KV, i32, vp, i32, i64, vp, f32,
                                          vp, f32, f64, vp, i32, vp, vp, sz, vp]
        L.lca_linear.argtypes = [vp, i64, i64, vp, i64, i64, vp, i32, i64, i64, i32, i32, i32, i32, vp]
        L.lca_grouped_out_proj.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, i32, vp, vp, i32, vp]
        L.lca_indexer_topk.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, vp, i32, vp, i64, i32, vp, vp, sz, vp]
        L.lca_indexer_topk_mxfp4.argtypes = [vp, vp, _KV, i32, i32, i32, i32, vp, i32, vp, i64, i32, vp, vp, sz, vp]
        L.lca_indexer_topk_workspace_size.argtypes = [i32, i32, i64, i32]
        L.lca_indexer_topk_workspace_size.restype = sz
        L.lca_attn_workspace_size.argtypes = [i32, i32, i32, i32, i64]
        L.lca_attn_workspace_size.restype = sz
        for name in ("lca_kv_compress", "lca_kv_compress_ws", "lca_indexer_score", "lca_indexer_score_mxfp4", "lca_topk_select",
                     "lca_csa_attn", "lca_hca_attn", "lca_hca_attn_noalloc", "lca_csa_attn_append",
                     "lca_hca_attn_append", "lca_linear", "lca_grouped_out_proj", "lca_indexer_topk",
                     "lca_indexer_topk_mxfp4"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _pos(p, B: int):
    arr = (C.c_int64 * B)(*[int(x) for x in (p if hasattr(p, "__len__") else [p] * B)])
    return arr


def _check(rc: int):
    if rc != 0:
        raise LcaError(rc, lib().lca_last_error().decode())


@dataclass
class KV:
    """Storage planes of one KV stream: nope [B][cap][d_nope], rope [B][cap][d_rope], scale [B][cap][d_nope/128]
    (fp8); MXFP4: nope uint8 [B][cap][d_nope/2] (two E2M1 codes per byte), scale uint8 [B][cap][d_nope/32]."""
    nope: torch.Tensor
    rope: torch.Tensor | None
    scale: torch.Tensor | None
    fmt: int
    d_nope: int
    d_rope: int
    cap: int

    @staticmethod
    def empty(fmt: int, B: int, cap: int, d_nope: int, d_rope: int, device="cuda") -> "KV":
        if fmt == F32:
            nope = torch.zeros(B, cap, d_nope, dtype=torch.float32, device=device)
            rope = torch.zeros(B, cap, d_rope, dtype=torch.float32, device=device)
            scale = None
        elif fmt == BF16:
            nope = torch.zeros(B, cap, d_nope, dtype=torch.bfloat16, device=device)
            rope = torch.zeros(B, cap, d_rope, dtype=torch.bfloat16, device=device)
            scale = None
        elif fmt == FP8:
            nope = torch.zeros(B, cap, d_nope, dtype=torch.uint8, device=device)
            rope = torch.zeros(B, cap, d_rope, dtype=torch.bfloat16, device=device)
            scale = torch.ones(B, cap, d_nope // 128, dtype=torch.float32, device=device)
        elif fmt == MXFP4:
            nope = torch.zeros(B, cap, d_nope // 2, dtype=torch.uint8, device=device)
            rope = None
            scale = torch.full((B, cap, d_nope // 32), 127, dtype=torch.uint8, device=device)
        else:
            raise ValueError(fmt)
        return KV(nope, rope if rope is not None and d_rope > 0 else None, scale, fmt, d_nope, d_rope, cap)

    @property
    def B(self) -> int:
        return self.nope.shape[0]

    def c(self) -> _KV:
        return _KV(self.nope.data_ptr(), 0 if self.rope is None else self.rope.data_ptr(),
                   0 if self.scale is None else self.scale.data_ptr(), self.fmt, self.d_nope,
                   self.d_rope, self.cap)


def kv_compress(c_a, z_a, c_b, z_b, out: KV, *, m: int, overlap: int, first_pos, bias_a=None,
                bias_b=None, gamma=None, eps: float = 1e-6, rope_theta: float = 0.0, ring: int = 0,
                ws=None, stream=None):
    """Inputs [B][n_rows][c]; each may be a row window of a longer per-sequence stream (rows contiguous,
    the same sequence stride for all four).  ws: a workspace of compress_workspace_size() bytes, with
    which calls of few long entries split each entry's rows over several workgroups (lca_kv_compress_ws)."""
    B, n_rows, c = c_a.shape
    for t in (c_a, z_a, c_b, z_b):
        if t is not None and (t.shape != c_a.shape or t.stride() != c_a.stride() or t.stride(2) != 1
                              or t.stride(1) != c):
            raise ValueError("kv_compress inputs must share shape and row-contiguous strides")
    in_stride = c_a.stride(0) // c if B > 1 else n_rows
    args = (_ptr(c_a), _ptr(z_a), _ptr(c_b), _ptr(z_b), _dtype(c_a), _ptr(bias_a), _ptr(bias_b), _ptr(gamma),
            float(eps), float(rope_theta), int(m), int(overlap), int(B), int(n_rows), int(in_stride),
            _pos(first_pos, B), out.c(), int(ring))
    if ws is None:
        _check(lib().lca_kv_compress(*args, _stream(stream)))
    else:
        _check(lib().lca_kv_compress_ws(*args, _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)))


def compress_workspace_size(in_dtype: int, m: int, overlap: int, d_nope: int, d_rope: int) -> int:
    """Bytes of the workspace with which kv_compress splits long entries (0: such calls never split)."""
    return int(lib().lca_compress_workspace_size(int(in_dtype), int(m), int(overlap), int(d_nope), int(d_rope)))


def indexer_score(q, w, k, scores, *, q_pos, m: int, stream=None):
    """q [B][T][H_I][d_I], w [B][T][H_I] f32 or None, k [B][k_cap][d_I], scores [B][T][s_stride]."""
    _dense(("q", q), ("w", w), ("scores", scores))
    B, T, H_I, d_I = q.shape
    _check(lib().lca_indexer_score(_ptr(q), _ptr(w), _ptr(k), _dtype(q), int(k.shape[1]), int(H_I),
                                   int(d_I), int(B), int(T), _pos(q_pos, B), int(m), _ptr(scores),
                                   _dtype(scores), int(scores.shape[2]), _stream(stream)))


def indexer_score_mxfp4(q, w, k: KV, scores, *, q_pos, m: int, stream=None):
    """q [B][T][H_I][d_I] bf16 (quantised to MXFP4 in the call), w [B][T][H_I] f32 or None, k MXFP4 key
    rows (KV with fmt MXFP4), scores [B][T][s_stride]."""
    _dense(("q", q), ("w", w), ("scores", scores))
    B, T, H_I, d_I = q.shape
    _check(lib().lca_indexer_score_mxfp4(_ptr(q), _ptr(w), k.c(), int(H_I), int(d_I), int(B), int(T),
                                         _pos(q_pos, B), int(m), _ptr(scores), _dtype(scores),
                                         int(scores.shape[2]), _stream(stream)))


def topk_select(scores, idx, *, q_pos, m: int, ws=None, stream=None):
    """scores [B][T][s_stride] -> idx [B][T][k] int32."""
    _dense(("scores", scores), ("idx", idx))
    B, T, s_stride = scores.shape
    k = idx.shape[2]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_topk_select(_ptr(scores), _dtype(scores), int(s_stride), int(B), int(T),
                                 _pos(q_pos, B), int(m), int(k), _ptr(idx), _ptr(ws), nbytes,
                                 _stream(stream)))


def indexer_topk(q, w, k, scores, idx, *, q_pos, m: int, ws=None, stream=None):
    """indexer_score then topk_select, the top-k's first pass fused into the indexer.  q [B][T][16][128]
    bf16, w [B][T][16] f32 or None, k [B][k_cap][128] bf16, scores [B][T][s_stride] bf16, idx [B][T][k]
    int32; ws: indexer_topk_workspace_size(B, T, s_stride, k) bytes, zeroed before its first use and kept
    for this call only (every call leaves it ready for the next: what must start at zero is zeroed again)."""
    _dense(("q", q), ("w", w), ("scores", scores), ("idx", idx))
    B, T = q.shape[0], q.shape[1]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_indexer_topk(_ptr(q), _ptr(w), _ptr(k), int(k.shape[1]), int(q.shape[2]), int(q.shape[3]),
                                  int(B), int(T), _pos(q_pos, B), int(m), _ptr(scores), int(scores.shape[2]),
                                  int(idx.shape[2]), _ptr(idx), _ptr(ws), nbytes, _stream(stream)))


def indexer_topk_mxfp4(q, w, k: KV, scores, idx, *, q_pos, m: int, ws=None, stream=None):
    """indexer_topk with MXFP4 keys (k: KV with fmt MXFP4; q bf16, quantised in the call)."""
    _dense(("q", q), ("w", w), ("scores", scores), ("idx", idx))
    B, T = q.shape[0], q.shape[1]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_indexer_topk_mxfp4(_ptr(q), _ptr(w), k.c(), int(q.shape[2]), int(q.shape[3]), int(B), int(T),
                                        _pos(q_pos, B), int(m), _ptr(scores), int(scores.shape[2]), int(idx.shape[2]),
                                        _ptr(idx), _ptr(ws), nbytes, _stream(stream)))


def indexer_topk_workspace_size(B: int, T: int, s_stride: int, k: int) -> int:
    return int(lib().lca_indexer_topk_workspace_size(int(B), int(T), int(s_stride), int(k)))


def topk_workspace_size(B: int, T: int, s_stride: int, k: int) -> int:
    return int(lib().lca_topk_workspace_size(int(B), int(T), int(s_stride), int(k)))


def attn_workspace_size(B: int, T: int, H: int, c: int, max_keys: int) -> int:
    return int(lib().lca_attn_workspace_size(int(B), int(T), int(H), int(c), int(max_keys)))


def _empty_kv():
    return _KV(0, 0, 0, 0, 0, 0, 0)


def _dense(*named):
    """The calls take q, w, scores, idx, out and lse as dense row-major arrays ([B][T][...], the last
    dims contiguous): a strided view (e.g. a row slice of a larger buffer with B > 1) would be
    addressed as if it were dense, so it is refused."""
    for name, t in named:
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (got strides {tuple(t.stride())})")


def csa_attn(q, out, *, q_pos, comp: KV, m: int, idx, win: KV | None, n_win: int, sink=None,
             sm_scale: float, rope_theta: float = 0.0, lse=None, ws=None, stream=None):
    _dense(("q", q), ("out", out), ("lse", lse), ("idx", idx))
    B, T, H, _ = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_csa_attn(_ptr(q), _dtype(q), int(H), int(B), int(T), _pos(q_pos, B), comp.c(),
                              int(m), _ptr(idx), int(idx.shape[2]),
                              win.c() if win is not None else _empty_kv(), int(n_win), _ptr(sink),
                              float(sm_scale), float(rope_theta), _ptr(out), _dtype(out), _ptr(lse),
                              _ptr(ws), nbytes, _stream(stream)))


def hca_attn(q, out, *, q_pos, comp: KV, m: int, win: KV | None, n_win: int, sink=None,
             sm_scale: float, rope_theta: float = 0.0, lse=None, ws=None, stream=None):
    _dense(("q", q), ("out", out), ("lse", lse))
    B, T, H, _ = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_hca_attn(_ptr(q), _dtype(q), int(H), int(B), int(T), _pos(q_pos, B), comp.c(),
                              int(m), win.c() if win is not None else _empty_kv(), int(n_win),
                              _ptr(sink), float(sm_scale), float(rope_theta), _ptr(out), _dtype(out),
                              _ptr(lse), _ptr(ws), nbytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # LCA_NOALLOC_SCRATCH_BYTES


def hca_attn_noalloc(q, out, *, q_pos, comp: KV, m: int, win: KV | None, n_win: int, sink=None,
                     sm_scale: float, rope_theta: float = 0.0, lse=None, stream=None):
    """hca_attn without a workspace: the library's static per-GPU scratch (calls on one GPU must not overlap)."""
    _dense(("q", q), ("out", out), ("lse", lse))
    B, T, H, _ = q.shape
    _check(lib().lca_hca_attn_noalloc(_ptr(q), _dtype(q), int(H), int(B), int(T), _pos(q_pos, B), comp.c(),
                                      int(m), win.c() if win is not None else _empty_kv(), int(n_win),
                                      _ptr(sink), float(sm_scale), float(rope_theta), _ptr(out), _dtype(out),
                                      _ptr(lse), _stream(stream)))


def _rows_stride(x, T: int) -> int:
    """Rows between sequences of a [B][T][c] row window (rows contiguous)."""
    B, _, c = x.shape
    if x.stride(2) != 1 or x.stride(1) != c:
        raise ValueError("x_win rows must be contiguous")
    return x.stride(0) // c if B > 1 else T


def csa_attn_append(q, out, x_win, *, q_pos, comp: KV, m: int, idx, win: KV, n_win: int, gamma=None,
                    eps: float = 1e-6, sink=None, sm_scale: float, rope_theta: float = 0.0, lse=None, ws=None,
                    stream=None):
    """Window store of rows q_pos .. q_pos+T-1 from x_win [B][T][c] (may be a row window of a longer
    per-sequence stream), then csa_attn."""
    _dense(("q", q), ("out", out), ("lse", lse), ("idx", idx))
    B, T, H, _ = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_csa_attn_append(_ptr(q), _dtype(q), int(H), int(B), int(T), _pos(q_pos, B), comp.c(),
                                     int(m), _ptr(idx), int(idx.shape[2]), win.c(), int(n_win), _ptr(x_win),
                                     _dtype(x_win), _rows_stride(x_win, T), _ptr(gamma), float(eps), _ptr(sink),
                                     float(sm_scale), float(rope_theta), _ptr(out), _dtype(out), _ptr(lse),
                                     _ptr(ws), nbytes, _stream(stream)))


def hca_attn_append(q, out, x_win, *, q_pos, comp: KV, m: int, win: KV, n_win: int, gamma=None,
                    eps: float = 1e-6, sink=None, sm_scale: float, rope_theta: float = 0.0, lse=None, ws=None,
                    stream=None):
    """Window store of rows q_pos .. q_pos+T-1 from x_win [B][T][c] (may be a row window of a longer
    per-sequence stream), then hca_attn."""
    _dense(("q", q), ("out", out), ("lse", lse))
    B, T, H, _ = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lca_hca_attn_append(_ptr(q), _dtype(q), int(H), int(B), int(T), _pos(q_pos, B), comp.c(),
                                     int(m), win.c(), int(n_win), _ptr(x_win), _dtype(x_win),
                                     _rows_stride(x_win, T), _ptr(gamma), float(eps), _ptr(sink),
                                     float(sm_scale), float(rope_theta), _ptr(out), _dtype(out), _ptr(lse),
                                     _ptr(ws), nbytes, _stream(stream)))


def linear(x, w, y, stream=None):
    """y[b][m][n] = sum_k x[b][m][k] w[b][n][k]: x [batch][M][K] or [M][K] bf16, w [batch][N][K] or [N][K] bf16
    (rows contiguous, any row / batch strides), y [batch][M][N] or [M][N] f32 / bf16."""
    x3, w3, y3 = (t if t.dim() == 3 else t.unsqueeze(0) for t in (x, w, y))
    bt, M, K = x3.shape
    N = w3.shape[1]
    for t in (x3, w3, y3):
        if t.stride(2) != 1:
            raise ValueError("linear operands need contiguous rows")
    if x3.dtype != torch.bfloat16 or w3.dtype != torch.bfloat16:
        raise TypeError("x and w must be bf16")
    _check(lib().lca_linear(_ptr(x3), x3.stride(1), x3.stride(0) if bt > 1 else 0, _ptr(w3), w3.stride(1),
                            w3.stride(0) if w3.shape[0] > 1 else 0, _ptr(y3), _dtype(y3), y3.stride(1),
                            y3.stride(0) if bt > 1 else 0, int(M), int(N), int(K), int(bt), _stream(stream)))


def grouped_out_proj(o, wg, wo, mid, out, *, g: int, stream=None):
    """o [T][H][c] bf16, wg [g][d_g][H/g*c] bf16, wo [d][g*d_g] bf16, mid [T][g*d_g] bf16 scratch,
    out [T][d] f32 / bf16."""
    T, H, c = o.shape
    d_g, d = wg.shape[1], wo.shape[0]
    _check(lib().lca_grouped_out_proj(_ptr(o), int(T), int(H), int(c), int(g), _ptr(wg), int(d_g), _ptr(wo),
                                      int(d), _ptr(mid), _ptr(out), _dtype(out), _stream(stream)))
