"""Layer driver: the order in which one CSA or HCA layer calls the library.

The DeepSeek-V4 pages ("DeepSeek-V4 中文翻译" section 2.3 and 3.5.1) describe per
layer: a sliding window of raw KV rows (kept in a fixed-size state cache), a
compressed stream that grows by one entry every m raw tokens (CSA m = 4 with
overlapping blocks, HCA m' = 128 without), and for CSA a lightning indexer
over the compressed stream followed by top-k selection.  For T new query rows
at positions t0 .. t0+T-1 of every sequence, Layer.step() issues:

    window store      kv_compress(m = 1, ring)          raw rows t0 .. t0+T-1
    compress          kv_compress(m, overlap)           entries whose block ends in the chunk
    indexer keys      kv_compress(m, overlap, d_I)      (CSA; bf16 or MXFP4 keys)
    scores            indexer_score / _mxfp4            (CSA)
    selection         topk_select                       (CSA)
                      (bf16 scores: one indexer_topk / indexer_topk_mxfp4 call, the top-k's
                      first histogram pass fused into the indexer)
    attention         csa_attn / hca_attn

Decode is T = 1; chunked prefill is T > 1.  Nothing here computes: every step
is one library call on the current stream, so a sequence of steps can be
captured in a HIP graph.  The window store rides on the attention call
(csa_attn_append / hca_attn_append), which for decode-sized launches does it
inside the attention launch; it only has to precede the attention, since
compression reads the raw rows, not the window.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (BF16, FP8, MXFP4, KV, attn_workspace_size, compress_workspace_size, csa_attn, csa_attn_append,
               hca_attn, hca_attn_append, indexer_score, indexer_score_mxfp4, indexer_topk, indexer_topk_mxfp4,
               indexer_topk_workspace_size, kv_compress, topk_select, topk_workspace_size)


@dataclass
class LayerSpec:
    kind: str                  # "csa" or "hca"
    m: int                     # compression ratio (4 / 128)
    H: int = 64                # query heads
    d_nope: int = 512
    d_rope: int = 64
    fmt: int = FP8             # storage of compressed entries and window rows
    n_win: int = 128
    k: int = 0                 # top-k (CSA)
    H_I: int = 16
    d_I: int = 128
    score_fmt: int = BF16
    key_fmt: int = BF16        # indexer keys: BF16, or MXFP4 (the QK path in FP4)
    rope_theta: float = 10000.0
    eps: float = 1e-6

    @property
    def c(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def overlap(self) -> int:
        return 1 if self.kind == "csa" else 0

    @property
    def sm_scale(self) -> float:
        return self.c ** -0.5


@dataclass
class RawStream:
    """Projected raw rows of B sequences for positions [base, base + rows): the compressor inputs
    c_a, z_a, c_b, z_b [B][rows][c] (and the indexer's [B][rows][d_I] for CSA), bf16."""
    base: int
    c_a: torch.Tensor
    z_a: torch.Tensor
    c_b: torch.Tensor
    z_b: torch.Tensor
    i_ca: torch.Tensor | None = None
    i_za: torch.Tensor | None = None
    i_cb: torch.Tensor | None = None
    i_zb: torch.Tensor | None = None

    def rows(self, name: str, p0: int, n: int) -> torch.Tensor:
        t = getattr(self, name)
        lo = p0 - self.base
        assert lo >= 0 and lo + n <= t.shape[1], (name, p0, n, self.base, t.shape)
        return t[:, lo:lo + n]


@dataclass
class Params:
    """Learned per-layer parameters (synthetic here): compressor biases [m][c] and RMSNorm weight [c],
    indexer-key compressor biases [m][d_I], sink logits [H] (f32)."""
    bias_a: torch.Tensor
    bias_b: torch.Tensor
    gamma: torch.Tensor
    sink: torch.Tensor
    i_bias_a: torch.Tensor | None = None
    i_bias_b: torch.Tensor | None = None


def _rows(buf: torch.Tensor, T: int) -> torch.Tensor:
    """The first B x T rows of a [B][t_max][n] buffer as a dense [B][T][n] array (its leading
    elements: the calls take dense arrays, and a [:, :T] slice is strided when B > 1)."""
    B, _, n = buf.shape
    return buf.view(-1)[:B * T * n].view(B, T, n)


class Layer:
    def __init__(self, spec: LayerSpec, B: int, comp_cap: int, win_cap: int, t_max: int, params: Params,
                 device="cuda", kvs: dict | None = None):
        """kvs: the layer's storage from elsewhere (e.g. a PagedCache): {"comp", "win", "keys" (CSA)} KVs of
        B sequences; default: fresh contiguous planes of comp_cap / win_cap rows."""
        self.spec, self.B, self.params = spec, B, params
        if kvs is not None:
            self.comp, self.win, self.keys = kvs["comp"], kvs["win"], kvs.get("keys")
        else:
            self.comp = KV.empty(spec.fmt, B, comp_cap, spec.d_nope, spec.d_rope, device)
            self.win = KV.empty(spec.fmt, B, win_cap, spec.d_nope, spec.d_rope, device)
            self.keys = KV.empty(spec.key_fmt, B, comp_cap, spec.d_I, 0, device) if spec.kind == "csa" else None
        self.t_max = t_max
        if spec.kind == "csa":
            sdt = torch.bfloat16 if spec.score_fmt == BF16 else torch.float32
            self.scores = torch.zeros(B, t_max, comp_cap, dtype=sdt, device=device)
            self.idx = torch.zeros(B, t_max, spec.k, dtype=torch.int32, device=device)
            tws = max(topk_workspace_size(B, T, comp_cap, spec.k) for T in range(1, min(t_max, 128) + 1))
            self.topk_ws = torch.zeros(max(16, tws), dtype=torch.uint8, device=device)
            # bf16 scores: indexer_topk (its own workspace, zeroed once; sized for the largest row count)
            itk = max(indexer_topk_workspace_size(B, T, comp_cap, spec.k) for T in sorted({1, min(t_max, 127), t_max}))
            self.itk_ws = torch.zeros(max(16, itk), dtype=torch.uint8, device=device)
            self.fuse_topk = True
            max_keys = spec.k + spec.n_win
        else:
            self.scores = self.idx = self.topk_ws = self.itk_ws = None
            self.fuse_topk = False
            max_keys = comp_cap + spec.n_win
        # the compressor's workspace: long blocks (m' = 128) of few entries split over workgroups
        cws = compress_workspace_size(BF16, spec.m, spec.overlap, spec.d_nope, spec.d_rope)
        self.comp_ws = torch.empty(cws, dtype=torch.uint8, device=device) if cws > 0 else None
        # split partials are needed only for short launches (few query rows); size for the largest
        ws = max(attn_workspace_size(B, T, spec.H, spec.c, max_keys) for T in range(1, min(t_max, 128) + 1))
        self.ws = torch.zeros(max(16, ws), dtype=torch.uint8, device=device)

    def reserve_rows(self, T: int):
        """Buffers and workspaces for calls of T query rows per sequence (a prefill chunk on a layer built
        for decode): scores, idx, the fused indexer + top-k workspace (zeroed) and the attention's."""
        s, B = self.spec, self.B
        if s.kind == "csa":
            cap = self.keys.cap
            if self.scores.shape[1] < T:
                self.scores = torch.zeros(B, T, cap, dtype=self.scores.dtype, device=self.scores.device)
                self.idx = torch.zeros(B, T, s.k, dtype=torch.int32, device=self.idx.device)
            need = indexer_topk_workspace_size(B, T, cap, s.k)
            if need > self.itk_ws.numel():
                self.itk_ws = torch.zeros(need, dtype=torch.uint8, device=self.itk_ws.device)
            need = topk_workspace_size(B, T, cap, s.k)
            if need > self.topk_ws.numel():
                self.topk_ws = torch.zeros(need, dtype=torch.uint8, device=self.topk_ws.device)
            keys = s.k + s.n_win
        else:
            keys = self.comp.cap + s.n_win
        need = attn_workspace_size(B, T, s.H, s.c, keys)
        if need > self.ws.numel():
            self.ws = torch.zeros(need, dtype=torch.uint8, device=self.ws.device)
        self.t_max = max(self.t_max, T)

    # ------------------------------------------------------------------
    def compress(self, raw: RawStream, t0: int, T: int):
        """Entries whose block ends inside [t0, t0 + T)."""
        s, p = self.spec, self.params
        m = s.m
        first_new = t0 // m                     # first entry that can complete in this chunk
        end = (t0 + T) // m                     # entries < end are complete after the chunk
        if end <= first_new:
            return
        lo = max(0, (first_new - s.overlap) * m)
        n = t0 + T - lo
        kw = dict(m=m, overlap=s.overlap, first_pos=lo)
        b_rows = (lambda nm: raw.rows(nm, lo, n)) if s.overlap else (lambda nm: None)
        kv_compress(raw.rows("c_a", lo, n), raw.rows("z_a", lo, n), b_rows("c_b"), b_rows("z_b"), self.comp,
                    bias_a=p.bias_a, bias_b=p.bias_b if s.overlap else None, gamma=p.gamma, eps=s.eps,
                    rope_theta=s.rope_theta, ws=self.comp_ws, **kw)
        if s.kind == "csa":
            kv_compress(raw.rows("i_ca", lo, n), raw.rows("i_za", lo, n), b_rows("i_cb"), b_rows("i_zb"),
                        self.keys, bias_a=p.i_bias_a, bias_b=p.i_bias_b, **kw)

    def attend(self, t0: int, q, out, q_idx=None, w=None, lse=None, record=None, x_win=None):
        """q [B][T][H][c] bf16 -> out [B][T][H][c].  record(name, fn) wraps a launch (for timing).
        x_win: raw rows [B][T][c] of positions t0 .. t0+T-1, stored into the window by the call."""
        s, p = self.spec, self.params
        T = q.shape[1]
        run = record or (lambda name, fn: fn())
        app = {} if x_win is None else dict(gamma=p.gamma, eps=s.eps)
        if s.kind == "csa":
            sc = _rows(self.scores, T)
            ix = _rows(self.idx, T)
            if self.fuse_topk and s.score_fmt == BF16 and self.keys.fmt in (BF16, MXFP4):
                if self.keys.fmt == MXFP4:
                    run("indexer_topk", lambda: indexer_topk_mxfp4(q_idx, w, self.keys, sc, ix, q_pos=t0, m=s.m,
                                                                   ws=self.itk_ws))
                else:
                    run("indexer_topk", lambda: indexer_topk(q_idx, w, self.keys.nope, sc, ix, q_pos=t0, m=s.m,
                                                             ws=self.itk_ws))
            else:
                if self.keys.fmt == MXFP4:
                    run("indexer_score", lambda: indexer_score_mxfp4(q_idx, w, self.keys, sc, q_pos=t0, m=s.m))
                else:
                    run("indexer_score", lambda: indexer_score(q_idx, w, self.keys.nope, sc, q_pos=t0, m=s.m))
                run("topk_select", lambda: topk_select(sc, ix, q_pos=t0, m=s.m, ws=self.topk_ws))
            kw = dict(q_pos=t0, comp=self.comp, m=s.m, idx=ix, win=self.win, n_win=s.n_win, sink=p.sink,
                      sm_scale=s.sm_scale, rope_theta=s.rope_theta, lse=lse, ws=self.ws, **app)
            if x_win is None:
                run("csa_attn", lambda: csa_attn(q, out, **kw))
            else:
                run("csa_attn", lambda: csa_attn_append(q, out, x_win, **kw))
        else:
            kw = dict(q_pos=t0, comp=self.comp, m=s.m, win=self.win, n_win=s.n_win, sink=p.sink,
                      sm_scale=s.sm_scale, rope_theta=s.rope_theta, lse=lse, ws=self.ws, **app)
            if x_win is None:
                run("hca_attn", lambda: hca_attn(q, out, **kw))
            else:
                run("hca_attn", lambda: hca_attn_append(q, out, x_win, **kw))

    def step(self, raw: RawStream, t0: int, q, out, q_idx=None, w=None, lse=None, record=None):
        """T = q.shape[1] new rows at positions t0 .. t0+T-1 (the same for every sequence)."""
        T = q.shape[1]
        run = record or (lambda name, fn: fn())
        run("kv_compress", lambda: self.compress(raw, t0, T))
        self.attend(t0, q, out, q_idx, w, lse, record, x_win=raw.rows("c_a", t0, T))


def cache_streams(specs: list[LayerSpec], comp_rows: list[int], win_cap: int):
    """The CacheStreams of a stack of layers for a PagedCache: per layer i the compressed entries
    ("i/comp", paged, ratio m), the window ring ("i/win", state cache) and for CSA the indexer keys
    ("i/keys", paged)."""
    from .cache import CacheStream
    out = []
    for i, (s, rows) in enumerate(zip(specs, comp_rows)):
        out.append(CacheStream(f"{i}/comp", s.fmt, s.d_nope, s.d_rope, s.m, rows))
        out.append(CacheStream(f"{i}/win", s.fmt, s.d_nope, s.d_rope, 0, win_cap))
        if s.kind == "csa":
            out.append(CacheStream(f"{i}/keys", s.key_fmt, s.d_I, 0, s.m, rows))
    return out


def slot_kvs(cache, i: int, b0: int, B: int) -> dict:
    """Layer i's KVs for the B sequences in slots b0 .. b0+B-1 of a PagedCache."""
    def sl(kv):
        cut = lambda t: None if t is None else t[b0:b0 + B]
        return KV(cut(kv.nope), cut(kv.rope), cut(kv.scale), kv.fmt, kv.d_nope, kv.d_rope, kv.cap)
    out = {"comp": sl(cache.kv(f"{i}/comp")), "win": sl(cache.kv(f"{i}/win"))}
    if f"{i}/keys" in cache.streams:
        out["keys"] = sl(cache.kv(f"{i}/keys"))
    return out
