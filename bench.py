#!/usr/bin/env python3
"""Benchmark of the CSA / HCA compressed-attention path on one MI355X.

Headline (one JSON line on stdout): decode tokens/s of the interleaved
4-layer stack (HCA, HCA, CSA, HCA) for one sequence at 1,048,576 tokens of
context -- CSA holds 262,144 fp8 entries with top-k 2048, each HCA layer 8,192
entries at m' = 128, window 128, 64 query heads of 512 + 64 -- one step being
one decode token through all four layers (window store, compression when a
block completes, indexer, top-k, attention).  Inputs are synthetic and
already resident in HBM; the K timed steps are one HIP-graph replay.  To keep
the per-step working set (about 85 MB) out of the 256 MB Infinity Cache, the
stack state is replicated R times and consecutive steps rotate through the
replicas (as a deeper model would), so every step reads its caches from HBM.

Also reported (key "extra"): the same 1M decode with the CSA indexer's QK
path in MXFP4 and the top-2048 recall of bf16 and MXFP4-QK scores against
f32 scores; the same stack's 4096-token chunked prefill at 1M context (with
the chunk's MXFP4 indexer call timed beside the bf16 one); and CSA decode for
32 sequences at 131,072 tokens; and the linear maps around one attention
layer (projections and the grouped output projection) for a 4096-token chunk
and for one decode token; a whole single-layer prefill from position 0 (CSA at 8,192 tokens,
HCA at 65,536, bf16 storage); the 1M decode again with every cache in the paged
cache (one slot per replica, 64 KiB and 2 MiB pages) and the cost of forking
the 1M-token sequence (prefix reuse).  "roofline"
covers the dominant decode call, the CSA layer's fused indexer + top-k
(HBM-bound: 67 MB of keys per token), timed with HIP events around a graph of
the step's own calls; "step_hbm" is the whole step's algorithmic bytes over
its time.  "cpu_baseline" is the fp64 oracle on the host cores, a bounded
sample (one copy of the stack per core, four decode steps each).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import lca_synth as S  # noqa: E402
import long_context_attention_22_amd as lca  # noqa: E402
from long_context_attention_22_amd.stack import (Layer, LayerSpec, Params, RawStream, cache_streams,  # noqa: E402
                                                 slot_kvs)

METRIC = "CSA/HCA decode tokens/s at 128K–1M ctx (HBM GB/s %) + prefill tokens/s"
# HBM traffic of the decode indexer + top-k call (its three kernels) from rocprofv3 FETCH_SIZE /
# WRITE_SIZE passes, scaled by the same counters on a plain copy; used only while the sources of those
# kernels are unchanged since then.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_topk_decode_1m_traffic.json")
MXFP4_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_mxfp4_decode_1m_traffic.json")
INDEXER_SOURCES = ["long_context_attention_22_amd/csrc/indexer.hip", "long_context_attention_22_amd/csrc/topk.hip",
                   "long_context_attention_22_amd/csrc/device.h", "long_context_attention_22_amd/csrc/kernels.h"]
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0   # dense MXFP4 MFMA
T0_1M = 1 << 20
C = 576


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# synthetic workload construction (library calls only; inputs from lca_synth)
# ----------------------------------------------------------------------------

def to_dev(x: np.ndarray, dtype=None):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def make_params(seed: int, spec: LayerSpec, tag: str) -> Params:
    m, c = spec.m, spec.c
    p = Params(bias_a=to_dev(S.normal(seed, f"{tag}/bias_a", (m, c), 0.5)),
               bias_b=to_dev(S.normal(seed, f"{tag}/bias_b", (m, c), 0.5)),
               gamma=to_dev((1.0 + 0.1 * S.normal(seed, f"{tag}/gamma", (c,))).astype(np.float32)),
               sink=to_dev(S.normal(seed, f"{tag}/sink", (spec.H,))))
    if spec.kind == "csa":
        p.i_bias_a = to_dev(S.normal(seed, f"{tag}/ibias_a", (m, spec.d_I), 0.5))
        p.i_bias_b = to_dev(S.normal(seed, f"{tag}/ibias_b", (m, spec.d_I), 0.5))
    return p


def make_raw(seed: int, spec: LayerSpec, tag: str, B: int, base: int, rows: int) -> RawStream:
    def act(name, c):
        return to_dev(S.to_bf16(S.activations(seed, f"{tag}/{name}", (B, rows, c))))
    r = RawStream(base, act("ca", C), act("za", C), act("cb", C), act("zb", C))
    if spec.kind == "csa":
        r.i_ca, r.i_za, r.i_cb, r.i_zb = (act(n, spec.d_I) for n in ("ica", "iza", "icb", "izb"))
    return r


def fill_entries(layer: Layer, seed: int, tag: str, n: int, chunk: int = 65536):
    """Entries [0, n) of every sequence: N(0,1)^576 times a per-entry scale log-uniform in [0.1, 10],
    stored by the library's compressor at m = 1 (no norm, no RoPE); indexer keys N(0,1) bf16."""
    for b in range(layer.B):
        x = S.block_scaled(seed, f"{tag}/entries", b, n, C)
        for lo in range(0, n, chunk):
            xs = torch.from_numpy(x[None, lo:lo + chunk]).cuda()
            lca.kv_compress(xs, torch.zeros_like(xs), None, None, _seq_view(layer.comp, b), m=1, overlap=0,
                            first_pos=lo)
        if layer.keys is not None:
            k = S.to_bf16(S.normal(seed, f"{tag}/keys/{b}", (n, layer.spec.d_I)))
            layer.keys.nope[b, :n].copy_(to_dev(k))
    torch.cuda.synchronize()


def fill_window(layer: Layer, seed: int, tag: str, t0: int):
    """Ring rows for positions [t0 - cap, t0) (same law as the entries)."""
    cap = layer.win.cap
    p0 = max(0, t0 - cap)
    for b in range(layer.B):
        x = S.block_scaled(seed, f"{tag}/window", b, t0 - p0, C)
        xs = torch.from_numpy(x[None]).cuda()
        lca.kv_compress(xs, torch.zeros_like(xs), None, None, _seq_view(layer.win, b), m=1, overlap=0,
                        first_pos=p0, ring=1)
    torch.cuda.synchronize()


def _seq_view(kv: lca.KV, b: int) -> lca.KV:
    return lca.KV(kv.nope[b:b + 1], None if kv.rope is None else kv.rope[b:b + 1],
                  None if kv.scale is None else kv.scale[b:b + 1], kv.fmt, kv.d_nope, kv.d_rope, kv.cap)


def clone_layer(src: Layer) -> Layer:
    dst = Layer.__new__(Layer)
    dst.__dict__.update(src.__dict__)
    dst.comp = lca.KV(src.comp.nope.clone(), src.comp.rope.clone(), src.comp.scale.clone(), src.comp.fmt,
                      src.comp.d_nope, src.comp.d_rope, src.comp.cap)
    dst.win = lca.KV(src.win.nope.clone(), src.win.rope.clone(), src.win.scale.clone(), src.win.fmt,
                     src.win.d_nope, src.win.d_rope, src.win.cap)
    if src.keys is not None:
        dst.keys = lca.KV(src.keys.nope.clone(), None, None, src.keys.fmt, src.keys.d_nope, 0, src.keys.cap)
        dst.scores = torch.empty_like(src.scores)
        dst.idx = torch.empty_like(src.idx)
        dst.topk_ws = torch.empty_like(src.topk_ws)
        dst.itk_ws = torch.zeros_like(src.itk_ws)
    dst.ws = torch.empty_like(src.ws)
    return dst


class Stack:
    """Layers of one sequence group with their raw streams and per-position queries."""

    def __init__(self, specs, tags, B, t0, n_pos, t_chunk, seed, win_cap, raw_span=0):
        self.specs, self.B, self.t0 = specs, B, t0
        self.layers, self.raws, self.q, self.qi, self.w = [], [], [], [], []
        span = max(n_pos, t_chunk, raw_span) + 8
        for spec, tag in zip(specs, tags):
            vis0 = (t0 + 1) // spec.m
            cap = (t0 + span) // spec.m + 2
            layer = Layer(spec, B, cap, win_cap, t_chunk, make_params(seed, spec, tag))
            fill_entries(layer, seed, tag, vis0)
            fill_window(layer, seed, tag, t0)
            self.layers.append(layer)
            self.raws.append(make_raw(seed, spec, tag, B, t0 - 2 * spec.m, span + 2 * spec.m))
            self.q.append(to_dev(S.to_bf16(S.normal(seed, f"{tag}/q", (n_pos, B, 1, spec.H, C)))))
            if spec.kind == "csa":
                self.qi.append(to_dev(S.to_bf16(S.normal(seed, f"{tag}/qi", (n_pos, B, 1, spec.H_I, spec.d_I)))))
                self.w.append(to_dev(S.normal(seed, f"{tag}/w", (n_pos, B, 1, spec.H_I), 0.25)))
            else:
                self.qi.append(None)
                self.w.append(None)
        self.out = [torch.empty(B, 1, s.H, C, dtype=torch.bfloat16, device="cuda") for s in specs]

    def replicate(self):
        other = Stack.__new__(Stack)
        other.__dict__.update(self.__dict__)
        other.layers = [clone_layer(l) for l in self.layers]
        other.out = [torch.empty_like(o) for o in self.out]
        return other

    def decode(self, j: int, record=None):
        """Decode token j (position t0 + j) through every layer."""
        t = self.t0 + j
        for li, layer in enumerate(self.layers):
            layer.step(self.raws[li], t, self.q[li][j], self.out[li],
                       q_idx=None if self.qi[li] is None else self.qi[li][j],
                       w=None if self.w[li] is None else self.w[li][j], record=record)


class KernelTimer:
    """HIP events around every launch of one kernel, recorded on its stream (inside a graph capture
    they become event-record nodes: external=True)."""

    def __init__(self, name: str, external: bool = False):
        self.name, self.pairs, self.external = name, [], external

    def __call__(self, name, fn):
        if name != self.name:
            return fn()
        a = torch.cuda.Event(enable_timing=True, external=self.external)
        b = torch.cuda.Event(enable_timing=True, external=self.external)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def mean_ms(self) -> float:
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs]))


def graph_kernel_ms(stacks, W: int, K: int, name: str, unfuse: bool = False) -> float:
    """Mean duration of one library call's launches of the timed steps (the same calls with the same
    arguments and caches), replayed back to back in a graph; HIP events on the launch stream around the
    replay, divided by the call count.  unfuse: collect the CSA layers' selection as a plain
    indexer_score call instead of the fused indexer_topk (for the separate-call figures)."""
    R = len(stacks)
    launches = []

    def grab(n, fn):
        if n == name:
            launches.append(fn)

    fused = [(ly, ly.fuse_topk) for st in stacks for ly in st.layers]
    if unfuse:
        for ly, _ in fused:
            ly.fuse_topk = False
    for i in range(W, W + K):  # collect the launches (nothing runs: only the named one is kept)
        stacks[i % R].decode(i // R, record=lambda n, fn: grab(n, fn) if n == name else None)
    for ly, f in fused:
        ly.fuse_topk = f
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in launches:
            fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / len(launches)


def timed_graph_decode(stacks, W: int, K: int, timer: KernelTimer | None):
    """W eager warm-up steps, then K steps captured as one graph; replayed once untimed, once timed."""
    R = len(stacks)
    for i in range(W):
        stacks[i % R].decode(i // R)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(W, W + K):
            stacks[i % R].decode(i // R, record=timer)
    g.replay()
    torch.cuda.synchronize()
    if timer is not None:
        warm = [(a.elapsed_time(b)) for a, b in timer.pairs]
        del warm
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e), g


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

STACK_SPECS = [LayerSpec("hca", 128), LayerSpec("hca", 128), LayerSpec("csa", 4, k=2048), LayerSpec("hca", 128)]
STACK_TAGS = ["L0_hca", "L1_hca", "L2_csa", "L3_hca"]


def indexer_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in INDEXER_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path: str = TRAFFIC_FILE):
    """Counter-derived HBM bytes per decode indexer launch, or None when absent or stale."""
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != indexer_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def calibrate_copy(nbytes: int = 256 << 20, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {reps} x {nbytes} bytes read and written")


def copy_ceiling_gbs(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Measured device-copy rate (bytes read + written per second, best of reps), the practical HBM
    ceiling beside the 8 TB/s nominal peak."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        best = min(best, s.elapsed_time(e))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (best * 1e-3) / 1e9


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def indexer_bytes(vis: int, B: int, d_I: int = 128, H_I: int = 16) -> int:
    """Algorithmic bytes of one decode indexer launch: keys read once, scores written, q and w read."""
    return B * (vis * d_I * 2 + vis * 2 + H_I * d_I * 2 + H_I * 4)


def indexer_topk_bytes(vis: int, B: int, k: int, key_bytes: int = 256, d_I: int = 128, H_I: int = 16) -> int:
    """Algorithmic bytes of one decode indexer + top-k call: keys read once, q and w read, the k selected
    indices written.  The score row between the two (written once, read by the top-k's passes) is staged,
    not algorithmic: staged_score_bytes."""
    return B * (vis * key_bytes + H_I * d_I * 2 + H_I * 4 + k * 4)


def staged_score_bytes(vis: int, B: int, reads: int = 2) -> int:
    """The bf16 score row of a fused decode call: written by the indexer, read by the top-k's two launches."""
    return B * vis * 2 * (1 + reads)


def decode_step_bytes(specs, t: int, B: int = 1) -> int:
    """Algorithmic HBM bytes of one decode token through the stack at position t: per layer the attended
    stored rows (fp8 entries of 656 bytes: CSA the top-k selected, HCA every visible one, plus the window),
    q and o (bf16), the raw row of the window store and its stored row; CSA adds the indexer keys, its
    queries and head weights.  The amortised compression of a completed block (< 0.1 %) is left out."""
    row = 512 + 128 + 16
    tot = 0
    for sp in specs:
        vis = (t + 1) // sp.m
        rows = (min(sp.k, vis) if sp.kind == "csa" else vis) + min(sp.n_win, t + 1)
        tot += rows * row + 2 * sp.H * C * 2 + C * 2 + row
        if sp.kind == "csa":
            tot += vis * sp.d_I * 2 + sp.H_I * sp.d_I * 2 + sp.H_I * 4
    return B * tot


ROOFLINE_KERNELS = ("indexer_mfma<1, unsigned short> (1025 workgroups, with the top-k's chunk histograms), "
                    "topk_split_h2, topk_split_emit")


def bench_decode_1m(W: int, K: int, R: int, seed: int = 1005):
    n_pos = (W + K + R - 1) // R + 2
    log(f"building the 1M-context stack ({R} replicas, {n_pos} positions each)")
    t_build = time.time()
    base = Stack(STACK_SPECS, STACK_TAGS, 1, T0_1M, n_pos, 1, seed, win_cap=8192, raw_span=4096)
    stacks = [base] + [base.replicate() for _ in range(R - 1)]
    torch.cuda.synchronize()
    log(f"built in {time.time() - t_build:.1f} s")
    ms, g = timed_graph_decode(stacks, W, K, None)
    del g
    # the dominant decode call, as the step runs it: the CSA layer's fused indexer + top-k
    call_ms = graph_kernel_ms(stacks, W, K, "indexer_topk")
    timing = ("HIP events on the launch stream around one graph replay of the timed steps' indexer_topk calls "
              "(the step's own arguments and caches, replicas rotating, back to back), divided by the call count")
    vis = (T0_1M + 1) // 4
    nbytes = indexer_topk_bytes(vis, 1, 2048)
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    step_bytes = decode_step_bytes(STACK_SPECS, T0_1M)
    step_gbs = step_bytes / (ms / K * 1e-3) / 1e9
    return dict(ms=ms, ms_per_step=ms / K, tokens_per_s=K / (ms * 1e-3), indexer_ms=call_ms,
                step_hbm=dict(bytes_per_step=step_bytes, gbs=step_gbs, frac=step_gbs / HBM_PEAK_GBS),
                roofline=dict(kernel="indexer_topk", kernels=ROOFLINE_KERNELS, bound="hbm", achieved=achieved,
                              peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                              traffic=measured_traffic(), bytes_per_launch=nbytes,
                              staged_bytes_per_launch=staged_score_bytes(vis, 1), launch_ms=call_ms,
                              timing=timing)), stacks


def _per_slot_pages(streams, n_tokens: int, page: int) -> int:
    from long_context_attention_22_amd.cache import _planes_of, _row_bytes
    total = 0
    for st in streams:
        if st.m > 0:
            for _, dt, n in _planes_of(st):
                total += -(-((n_tokens // st.m + 1) * _row_bytes(dt, n)) // page)
    return total


def paged_stack(base: Stack, cache, slot: int, n_tokens: int, copy: bool = True) -> Stack:
    """The stack state of `base` (one sequence) copied into slot `slot` of a PagedCache (copy=False: only
    the stack's layers over that slot, e.g. for a slot filled by a fork)."""
    cache.reserve(slot, n_tokens)
    st = Stack.__new__(Stack)
    st.__dict__.update(base.__dict__)
    st.layers = []
    for i, src in enumerate(base.layers):
        kv = slot_kvs(cache, i, slot, 1)
        vis = min((n_tokens // src.spec.m) + 1, src.comp.cap)
        for name in ("comp", "keys") if copy else ():
            a, b = getattr(src, name), kv.get(name)
            if a is None:
                continue
            for pl in ("nope", "rope", "scale"):
                if getattr(a, pl) is not None:
                    getattr(b, pl)[:, :vis].copy_(getattr(a, pl)[:, :vis])
        for pl in ("nope", "rope", "scale") if copy else ():
            if getattr(src.win, pl) is not None:
                getattr(kv["win"], pl).copy_(getattr(src.win, pl))
        dst = Layer.__new__(Layer)
        dst.__dict__.update(src.__dict__)
        dst.comp, dst.win, dst.keys = kv["comp"], kv["win"], kv.get("keys")
        if src.keys is not None:
            dst.scores, dst.idx = torch.empty_like(src.scores), torch.empty_like(src.idx)
            dst.topk_ws = torch.empty_like(src.topk_ws)
            dst.itk_ws = torch.zeros_like(src.itk_ws)
        dst.ws = torch.empty_like(src.ws)
        st.layers.append(dst)
    st.out = [torch.empty_like(o) for o in base.out]
    return st


def bench_paged(stacks, W: int, K: int, contiguous_ms: float, prefill_chunk_ms: float | None,
                pages=(64 << 10, 2 << 20)):
    """The 1M decode with every cache (compressed entries, indexer keys, window rings) in a PagedCache:
    one slot per replica, filled with the contiguous stacks' state; then a fork of the 1M-token sequence."""
    from long_context_attention_22_amd.cache import PagedCache
    R = len(stacks)
    base = stacks[0]
    n_pos = (W + K + R - 1) // R + 2
    n_tokens = T0_1M + n_pos + 1
    rows = [ly.comp.cap for ly in base.layers]
    streams = cache_streams(STACK_SPECS, rows, base.layers[0].win.cap)
    out = {}
    for page in pages:
        per = _per_slot_pages(streams, n_tokens, page)
        t = time.perf_counter()
        cache = PagedCache(streams, max_seqs=R + 1, page_bytes=page, pool_pages=R * per + 64)
        t_create = time.perf_counter() - t
        t = time.perf_counter()
        for r in range(R):
            cache.open()
            cache.reserve(r, n_tokens)
        t_map = time.perf_counter() - t
        mapped = cache.stats()["mapped_pages"]
        pst = [paged_stack(base, cache, r, n_tokens) for r in range(R)]
        torch.cuda.synchronize()
        ms, g = timed_graph_decode(pst, W, K, None)
        del g
        torch.cuda.synchronize()
        # prefix reuse: the 1M-token sequence forked at its current length
        t = time.perf_counter()
        child = cache.fork(0, n_tokens)
        torch.cuda.synchronize()
        t_fork = time.perf_counter() - t
        stf = cache.stats()
        t = time.perf_counter()
        cache.close(child)
        t_close = time.perf_counter() - t
        st = cache.stats()
        res = dict(ms_per_step=ms / K, tokens_per_s=K / (ms * 1e-3), vs_contiguous=(ms / K) / contiguous_ms,
                   create_s=t_create, map_s=t_map, pages_mapped=mapped, map_us_per_page=t_map / mapped * 1e6,
                   pool_pages=st["pool_pages"], device_bytes=st["device_bytes"],
                   fork=dict(tokens=n_tokens, ms=t_fork * 1e3, shared_pages=stf["shared_pages"],
                             fresh_pages=st["free_pages"] - stf["free_pages"], close_ms=t_close * 1e3))
        if prefill_chunk_ms:
            res["fork"]["prefill_estimate_ms"] = prefill_chunk_ms * n_tokens / 4096
        out[f"page_{page // 1024}k"] = res
        log(f"paged cache, {page // 1024} KiB pages: {res['ms_per_step'] * 1e3:.1f} us/step "
            f"({res['vs_contiguous']:.3f} x contiguous); create {t_create:.2f} s, {mapped} pages mapped in "
            f"{t_map:.2f} s; fork of {n_tokens} tokens {t_fork * 1e3:.1f} ms ({stf['shared_pages']} pages shared)")
        del pst
        cache.destroy()
        torch.cuda.empty_cache()
    return out


def mxfp4_copy(src: lca.KV) -> lca.KV:
    """bf16 indexer keys re-stored as MXFP4 through the library's compressor (m = 1, no norm, no RoPE:
    each row is quantised as it is)."""
    k4 = lca.KV.empty(lca.MXFP4, src.nope.shape[0], src.cap, src.d_nope, 0)
    lca.kv_compress(src.nope, torch.zeros_like(src.nope), None, None, k4, m=1, overlap=0, first_pos=0)
    return k4


def keys_to_mxfp4(layer: Layer):
    """Switch a CSA layer to the MXFP4 indexer, its keys re-stored as MXFP4."""
    layer.keys = mxfp4_copy(layer.keys)
    layer.spec = dataclasses.replace(layer.spec, key_fmt=lca.MXFP4)


def score_recall(stack: Stack, keys_bf16: lca.KV, keys_fp4: lca.KV, rows: int, k: int = 2048):
    """Top-k recall of bf16 scores and of MXFP4-QK scores against f32 scores of the same bf16 inputs,
    over `rows` decode rows of the CSA layer (the selections from the library's top-k)."""
    li = [i for i, s in enumerate(stack.specs) if s.kind == "csa"][0]
    layer = stack.layers[li]
    cap = keys_bf16.cap
    s32 = torch.empty(1, 1, cap, dtype=torch.float32, device="cuda")
    s16 = torch.empty(1, 1, cap, dtype=torch.bfloat16, device="cuda")
    s4 = torch.empty(1, 1, cap, dtype=torch.bfloat16, device="cuda")
    ix = [torch.empty(1, 1, k, dtype=torch.int32, device="cuda") for _ in range(3)]
    r16, r4 = [], []
    for j in range(rows):
        t = stack.t0 + j
        qi, w = stack.qi[li][j], stack.w[li][j]
        lca.indexer_score(qi, w, keys_bf16.nope, s32, q_pos=t, m=4)
        lca.indexer_score(qi, w, keys_bf16.nope, s16, q_pos=t, m=4)
        lca.indexer_score_mxfp4(qi, w, keys_fp4, s4, q_pos=t, m=4)
        for sc, o in zip((s32, s16, s4), ix):
            lca.topk_select(sc, o, q_pos=t, m=4, ws=layer.topk_ws)
        ref = set(ix[0].flatten().tolist())
        r16.append(len(ref & set(ix[1].flatten().tolist())) / k)
        r4.append(len(ref & set(ix[2].flatten().tolist())) / k)
    return float(np.mean(r16)), float(np.mean(r4))


def bench_topk_precision(stack: Stack, rows: int = 8, k: int = 2048, reps: int = 5):
    """The selector on f32 against bf16 index scores of the same 1M decode rows ("DeepSeek-V4 中文翻译"
    section 5.2.1 reports BF16 scores making the top-k selector 2x faster at 99.7 % recall): the
    library's topk_select on each, timed over a graph of the rows' calls; recall of the bf16 selections
    against the f32 ones."""
    li = [i for i, sp in enumerate(stack.specs) if sp.kind == "csa"][0]
    layer = stack.layers[li]
    cap = layer.keys.cap
    ts = [stack.t0 + j for j in range(rows)]
    s32 = [torch.empty(1, 1, cap, dtype=torch.float32, device="cuda") for _ in ts]
    s16 = [torch.empty(1, 1, cap, dtype=torch.bfloat16, device="cuda") for _ in ts]
    i32 = [torch.empty(1, 1, k, dtype=torch.int32, device="cuda") for _ in ts]
    i16 = [torch.empty(1, 1, k, dtype=torch.int32, device="cuda") for _ in ts]
    ws = torch.zeros(max(16, lca.topk_workspace_size(1, 1, cap, k)), dtype=torch.uint8, device="cuda")
    for j, t in enumerate(ts):
        qi, w = stack.qi[li][j], stack.w[li][j]
        lca.indexer_score(qi, w, layer.keys.nope, s32[j], q_pos=t, m=4)
        lca.indexer_score(qi, w, layer.keys.nope, s16[j], q_pos=t, m=4)
    out = {}
    for name, sc, ix in (("f32", s32, i32), ("bf16", s16, i16)):
        calls = [lambda j=j, t=t: lca.topk_select(sc[j], ix[j], q_pos=t, m=4, ws=ws) for j, t in enumerate(ts)]
        for fn in calls:
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                for fn in calls:
                    fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[f"{name}_ms"] = e0.elapsed_time(e1) / (reps * len(calls))
        del g
    rec = np.mean([len(set(host_list(a)) & set(host_list(b))) / k for a, b in zip(i32, i16)])
    out.update(speedup=out["f32_ms"] / out["bf16_ms"], recall_bf16_vs_f32=float(rec), rows=rows, keys=cap,
               schedules="bf16: three launches over 16,384-key chunks; f32: one 1,024-thread workgroup per row")
    return out


def host_list(t: torch.Tensor) -> list:
    return [int(x) for x in t.flatten().tolist() if x >= 0]


def bench_decode_1m_mxfp4(stacks, W: int, K: int, recall: bool = True):
    """The same 1M decode with the CSA layer's indexer QK path in MXFP4 (keys stored MXFP4, each query
    head quantised in the indexer call); top-k recall against f32 scores on the benchmark's inputs."""
    li = [i for i, s in enumerate(stacks[0].specs) if s.kind == "csa"][0]
    saved = [(st.layers[li].keys, st.layers[li].spec) for st in stacks]
    for st in stacks:
        keys_to_mxfp4(st.layers[li])
    torch.cuda.synchronize()
    ms, g = timed_graph_decode(stacks, W, K, None)
    del g
    call_ms = graph_kernel_ms(stacks, W, K, "indexer_topk")            # as the step runs it
    ind_ms = graph_kernel_ms(stacks, W, K, "indexer_score", unfuse=True)  # the plain indexer kernel
    vis = (T0_1M + 1) // 4
    nbytes = vis * (64 + 4 + 2) + 16 * 128 * 2 + 16 * 4
    call_bytes = indexer_topk_bytes(vis, 1, 2048, key_bytes=64 + 4)
    rows = min(16, len(stacks[0].qi[li]))
    rec = None
    if recall:
        r16, r4 = score_recall(stacks[0], saved[0][0], stacks[0].layers[li].keys, rows)
        rec = dict(bf16_scores_vs_f32=r16, mxfp4_qk_vs_f32=r4, rows=rows,
                   inputs="N(0,1) bf16 queries and keys, N(0,0.25) head weights")
    for st, (keys, spec) in zip(stacks, saved):
        st.layers[li].keys, st.layers[li].spec = keys, spec
    gbs = nbytes / (ind_ms * 1e-3) / 1e9
    return dict(ms_per_step=ms / K, tokens_per_s=K / (ms * 1e-3),
                indexer_topk=dict(launch_ms=call_ms, bytes=call_bytes, gbs=call_bytes / (call_ms * 1e-3) / 1e9,
                                  frac=call_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS),
                indexer=dict(launch_ms=ind_ms, bytes=nbytes, gbs=gbs, frac=gbs / HBM_PEAK_GBS,
                             traffic=measured_traffic(MXFP4_TRAFFIC_FILE),
                             note="the plain indexer kernel (indexer_score_mxfp4) on the step's arguments"),
                recall_top2048=rec)


def attn_flops(T: int, t0: int, m: int, H: int, n_win: int, k: int | None) -> float:
    """Multiply-add flops (2 per MAC) of Q K^T and P V over the attended rows of T queries."""
    tot = 0
    for i in range(T):
        t = t0 + i
        keys = (min(k, (t + 1) // m) if k is not None else (t + 1) // m) + min(n_win, t + 1)
        tot += keys
    return 4.0 * tot * H * C


def bench_prefill_1m(stack: Stack, reps: int = 20, T: int = 4096, seed: int = 1005):
    """The stack's 4096-token chunk at 1M context; every rep restarts from the same cache state (median of
    reps, each after a cache-evicting write)."""
    log("building the 4096-token prefill inputs")
    qs, qis, ws = [], [], []
    for spec, tag in zip(stack.specs, STACK_TAGS):
        qs.append(to_dev(S.to_bf16(S.normal(seed, f"{tag}/qp", (1, T, spec.H, C)))))
        if spec.kind == "csa":
            qis.append(to_dev(S.to_bf16(S.normal(seed, f"{tag}/qip", (1, T, spec.H_I, spec.d_I)))))
            ws.append(to_dev(S.normal(seed, f"{tag}/wp", (1, T, spec.H_I), 0.25)))
        else:
            qis.append(None)
            ws.append(None)
    # the chunk needs T rows of scores / idx and prefill-sized workspaces
    for layer in stack.layers:
        layer.reserve_rows(T)
    outs = [torch.empty(1, T, s.H, C, dtype=torch.bfloat16, device="cuda") for s in stack.specs]
    timers = {n: KernelTimer(n) for n in ("indexer_topk", "csa_attn", "hca_attn")}

    def rec(name, fn):
        if name in timers:
            return timers[name](name, fn)
        return fn()

    def chunk(record=None):
        for li, layer in enumerate(stack.layers):
            layer.step(stack.raws[li], stack.t0, qs[li], outs[li], q_idx=qis[li], w=ws[li], record=record)

    chunk()
    torch.cuda.synchronize()
    # each timed rep starts with a 512 MiB write, which evicts the 256 MB Infinity Cache; median of reps
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    times = []
    for r in range(reps):
        flush.fill_(r & 255)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        chunk()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    del flush
    ms = float(np.median(times))
    chunk(record=rec)
    torch.cuda.synchronize()
    kt = {n: t.mean_ms() for n, t in timers.items() if t.pairs}
    # the chunk's CSA selection as separate calls (the indexer kernel alone: its MFMA fraction; the
    # top-k with all its passes), on the same queries and keys
    li = [i for i, sp in enumerate(stack.specs) if sp.kind == "csa"][0]
    layer = stack.layers[li]
    sep = {n: KernelTimer(n) for n in ("indexer_score", "topk_select")}
    for _ in range(3):
        sep["indexer_score"]("indexer_score", lambda: lca.indexer_score(qis[li], ws[li], layer.keys.nope,
                                                                        layer.scores[:, :T], q_pos=stack.t0, m=4))
        sep["topk_select"]("topk_select", lambda: lca.topk_select(layer.scores[:, :T], layer.idx[:, :T],
                                                                  q_pos=stack.t0, m=4, ws=layer.topk_ws))
    torch.cuda.synchronize()
    kt.update({n: t.mean_ms() for n, t in sep.items()})
    # the chunk's indexer call with the QK path in MXFP4 (same queries, keys re-stored as MXFP4)
    k4 = mxfp4_copy(layer.keys)
    f4 = KernelTimer("indexer_mxfp4")
    for _ in range(reps):
        f4("indexer_mxfp4", lambda: lca.indexer_score_mxfp4(qis[li], ws[li], k4, layer.scores[:, :T],
                                                            q_pos=stack.t0, m=layer.spec.m))
    torch.cuda.synchronize()
    kt["indexer_mxfp4"] = f4.mean_ms()
    del k4
    hca_fl = attn_flops(T, stack.t0, 128, 64, 128, None)
    csa_fl = attn_flops(T, stack.t0, 4, 64, 128, 2048)
    idx_fl = 2.0 * 16 * 128 * sum((stack.t0 + i + 1) // 4 for i in range(T))
    tot_fl = 3 * hca_fl + csa_fl + idx_fl
    hca_tf = hca_fl / (kt["hca_attn"] * 1e-3) / 1e12
    return dict(tokens=T, ms=ms, ms_min=min(times), ms_max=max(times), reps=reps,
                tokens_per_s=T / (ms * 1e-3), tflops=tot_fl / (ms * 1e-3) / 1e12,
                mfma_frac=tot_fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, kernel_ms=kt,
                hca_attn=dict(flops=hca_fl, tflops=hca_tf, frac=hca_tf / BF16_PEAK_TFLOPS),
                indexer=dict(flops=idx_fl, tflops=idx_fl / (kt["indexer_score"] * 1e-3) / 1e12,
                             frac=idx_fl / (kt["indexer_score"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS),
                indexer_mxfp4=dict(ms=kt["indexer_mxfp4"], tflops=idx_fl / (kt["indexer_mxfp4"] * 1e-3) / 1e12,
                                   frac=idx_fl / (kt["indexer_mxfp4"] * 1e-3) / 1e12 / FP4_PEAK_TFLOPS),
                csa_attn=dict(flops=csa_fl, tflops=csa_fl / (kt["csa_attn"] * 1e-3) / 1e12))


def bench_prefill_single(kind: str, T: int, reps: int = 10, seed: int = 0):
    """A whole single-layer prefill from position 0 with bf16 storage: CSA at 8,192 tokens (window store,
    compressor, indexer keys, indexer + top-512 (one fused call), attention) or HCA at 65,536 tokens (window store,
    compressor, attention).  Inputs drawn on the GPU (N(0,1), 1 % of channels x20 in the compressor
    streams; w N(0,1)/4); median of reps, each after a cache-evicting write."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    H, m = 64, (4 if kind == "csa" else 128)
    k, n_win = 512, 128
    out_ch = torch.randperm(C, generator=g, device="cuda")[: C // 100]

    def acts(c, oc=None):
        x = torch.randn(1, T, c, device="cuda", generator=g)
        if oc is not None:
            x[..., oc] *= 20.0
        return x.to(torch.bfloat16)

    ca, za, cb, zb = (acts(C, out_ch) for _ in range(4))
    ba = torch.randn(m, C, device="cuda", generator=g) * 0.5
    bb = torch.randn(m, C, device="cuda", generator=g) * 0.5
    gamma = 1.0 + 0.1 * torch.randn(C, device="cuda", generator=g)
    sink = torch.randn(H, device="cuda", generator=g)
    q = torch.randn(1, T, H, C, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty(1, T, H, C, dtype=torch.bfloat16, device="cuda")
    ncap = T // m
    win = lca.KV.empty(lca.BF16, 1, T, 512, 64)
    comp = lca.KV.empty(lca.BF16, 1, ncap, 512, 64)
    if kind == "csa":
        ich = torch.randperm(128, generator=g, device="cuda")[:2]
        ica, iza, icb, izb = (acts(128, ich) for _ in range(4))
        iba = torch.randn(m, 128, device="cuda", generator=g) * 0.5
        ibb = torch.randn(m, 128, device="cuda", generator=g) * 0.5
        keys = lca.KV.empty(lca.BF16, 1, ncap, 128, 0)
        qi = torch.randn(1, T, 16, 128, device="cuda", generator=g).to(torch.bfloat16)
        w = torch.randn(1, T, 16, device="cuda", generator=g) * 0.25
        sc = torch.empty(1, T, ncap, dtype=torch.bfloat16, device="cuda")
        idx = torch.empty(1, T, k, dtype=torch.int32, device="cuda")
        tws = torch.zeros(max(16, lca.indexer_topk_workspace_size(1, T, ncap, k)), dtype=torch.uint8, device="cuda")
    aws = torch.empty(max(16, lca.attn_workspace_size(1, T, H, C, (k if kind == "csa" else ncap) + n_win)),
                      dtype=torch.uint8, device="cuda")

    def run():
        lca.kv_compress(ca, za, None, None, win, m=1, overlap=0, first_pos=0, gamma=gamma, rope_theta=1e4)
        if kind == "csa":
            lca.kv_compress(ca, za, cb, zb, comp, m=m, overlap=1, first_pos=0, bias_a=ba, bias_b=bb, gamma=gamma,
                            rope_theta=1e4)
            lca.kv_compress(ica, iza, icb, izb, keys, m=m, overlap=1, first_pos=0, bias_a=iba, bias_b=ibb)
            lca.indexer_topk(qi, w, keys.nope, sc, idx, q_pos=0, m=m, ws=tws)
            lca.csa_attn(q, out, q_pos=0, comp=comp, m=m, idx=idx, win=win, n_win=n_win, sink=sink,
                         sm_scale=C ** -0.5, rope_theta=1e4, ws=aws)
        else:
            lca.kv_compress(ca, za, None, None, comp, m=m, overlap=0, first_pos=0, bias_a=ba, gamma=gamma,
                            rope_theta=1e4)
            lca.hca_attn(q, out, q_pos=0, comp=comp, m=m, win=win, n_win=n_win, sink=sink, sm_scale=C ** -0.5,
                         rope_theta=1e4, ws=aws)

    run()
    torch.cuda.synchronize()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    times = []
    for r in range(reps):
        flush.fill_(r & 255)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    ms = float(np.median(times))
    att = attn_flops(T, 0, m, H, n_win, k if kind == "csa" else None)
    idx_fl = 2.0 * 16 * 128 * sum((i + 1) // m for i in range(T)) if kind == "csa" else 0.0
    tf = (att + idx_fl) / (ms * 1e-3) / 1e12
    return dict(tokens=T, ms=ms, tokens_per_s=T / (ms * 1e-3), attn_flops=att, indexer_flops=idx_fl, tflops=tf,
                mfma_frac=tf / BF16_PEAK_TFLOPS, storage="bf16", top_k=k if kind == "csa" else None, reps=reps)


def bench_decode_c4(W: int, K: int, seed: int = 1004):
    """CSA decode, 32 sequences at 131,072 tokens (32,768 fp8 entries each), top-k 1024, window 128."""
    B, t0 = 32, 131072
    spec = LayerSpec("csa", 4, k=1024)
    n_pos = W + K + 2
    log("building the 32 x 128K CSA decode state")
    st = Stack([spec], ["c4_csa"], B, t0, n_pos, 1, seed, win_cap=256)
    ms, g = timed_graph_decode([st], W, K, None)
    del g
    call_ms = graph_kernel_ms([st], W, K, "indexer_topk")
    ind_ms = graph_kernel_ms([st], W, K, "indexer_score", unfuse=True)
    vis = (t0 + 1) // 4
    nbytes = indexer_bytes(vis, B)
    call_bytes = indexer_topk_bytes(vis, B, 1024)
    gbs = nbytes / (ind_ms * 1e-3) / 1e9
    step_bytes = decode_step_bytes([spec], t0, B)
    step_gbs = step_bytes / (ms / K * 1e-3) / 1e9
    # the same decode with the indexer's QK path in MXFP4 (keys re-stored as MXFP4 by the compressor)
    keys_to_mxfp4(st.layers[0])
    torch.cuda.synchronize()
    ms4, g = timed_graph_decode([st], W, K, None)
    del g
    call4 = graph_kernel_ms([st], W, K, "indexer_topk")
    ind4 = graph_kernel_ms([st], W, K, "indexer_score", unfuse=True)
    b4 = B * (vis * (64 + 4 + 2) + 16 * 128 * 2 + 16 * 4)
    return dict(batch=B, ctx=t0, ms_per_step=ms / K, tokens_per_s=B * K / (ms * 1e-3),
                step_hbm=dict(bytes_per_step=step_bytes, gbs=step_gbs, frac=step_gbs / HBM_PEAK_GBS),
                indexer_topk=dict(launch_ms=call_ms, bytes=call_bytes, gbs=call_bytes / (call_ms * 1e-3) / 1e9,
                                  frac=call_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS),
                indexer=dict(launch_ms=ind_ms, gbs=gbs, frac=gbs / HBM_PEAK_GBS, bytes=nbytes,
                             note="the plain indexer kernel (indexer_score) on the step's arguments"),
                mxfp4_indexer=dict(ms_per_step=ms4 / K, tokens_per_s=B * K / (ms4 * 1e-3), indexer_topk_ms=call4,
                                   launch_ms=ind4, bytes=b4, gbs=b4 / (ind4 * 1e-3) / 1e9))


def compress_bytes(n_rows: int, m: int, overlap: int, c: int, fmt: int, in_b: int = 2) -> tuple[int, int]:
    """(algorithmic bytes, entries) of one compressor launch over n_rows raw rows (plus the m rows of the
    previous block when overlapping): C and Z of each row read once (and C_b, Z_b), the bias rows and
    gamma, each entry written once."""
    n_in = n_rows + (m if overlap else 0)
    entries = n_rows // m
    row_out = {lca.FP8: 512 + 128 + 16, lca.BF16: 2 * c, lca.F32: 4 * c}[fmt]
    streams = 4 if overlap else 2
    return streams * n_in * c * in_b + (2 if overlap else 1) * m * c * 4 + c * 4 + entries * row_out, entries


def bench_compressor(seed: int = 1007):
    """The compressor's launches timed alone (rows from HBM): an HCA layer's 65,536-token prefill (m' = 128,
    512 entries, bf16 storage), and the 4096-token chunk at 1M of a CSA layer (m = 4 with overlap, 1,024 fp8
    entries) and of an HCA layer (32 fp8 entries).  Each launch reads its own copy of the inputs, the copies
    rotating through more than the 256 MB Infinity Cache; HIP events around a graph of the launches."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    out = {}
    cases = [("hca_prefill_65536", 65536, 128, 0, lca.BF16, 0),
             ("csa_chunk_4096", 4096, 4, 1, lca.FP8, T0_1M),
             ("hca_chunk_4096", 4096, 128, 0, lca.FP8, T0_1M)]
    for name, n, m, ov, fmt, p0 in cases:
        nbytes, entries = compress_bytes(n, m, ov, C, fmt)
        n_in = n + (m if ov else 0)
        copies = max(3, -(-(320 << 20) // max(1, nbytes)))
        streams = []
        for _ in range(copies):
            x = (torch.randn(4 if ov else 2, 1, n_in, C, device="cuda", generator=gen)).to(torch.bfloat16)
            streams.append(x)
        ba = torch.randn(m, C, device="cuda", generator=gen) * 0.5
        bb = torch.randn(m, C, device="cuda", generator=gen) * 0.5
        gamma = 1.0 + 0.1 * torch.randn(C, device="cuda", generator=gen)
        cap = (p0 + n) // m + 2
        kv = lca.KV.empty(fmt, 1, cap, 512, 64)
        first = p0 - (m if ov else 0)
        wsz = lca.compress_workspace_size(lca.BF16, m, ov, 512, 64)  # (as the stack's layers pass it)
        cws = torch.empty(wsz, dtype=torch.uint8, device="cuda") if wsz else None

        def launch(x):
            lca.kv_compress(x[0], x[1], x[2] if ov else None, x[3] if ov else None, kv, m=m, overlap=ov,
                            first_pos=first, bias_a=ba, bias_b=bb if ov else None, gamma=gamma, rope_theta=1e4,
                            ws=cws)

        for x in streams[:2]:
            launch(x)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for x in streams:
                launch(x)
        g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / len(streams)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = dict(rows=n, m=m, overlap=ov, entries=entries, storage={lca.FP8: "fp8", lca.BF16: "bf16"}[fmt],
                         bytes=nbytes, launch_ms=ms, gbs=gbs, hbm_frac=gbs / HBM_PEAK_GBS, copies=len(streams))
        del g, streams, kv
        torch.cuda.empty_cache()
    return out


def bench_projections(reps: int = 5, seed: int = 1006):
    """The linear maps around one attention layer (lca_linear / lca_grouped_out_proj), shaped as the
    pages' smaller model ([R] 4.2.1: hidden 4096, query compression 1024, 64 heads, output projection in
    8 groups of 1024) with this benchmark's heads of 512 + 64 and 16 x 128 indexer: a 4096-token
    chunk (MFMA tiles) and one decode token (weights streamed once).  Weights N(0, 1/fan_in), bf16.  Each
    map is timed as `reps` launches replayed from one captured graph (HIP events around the replay)."""
    d, dq, H, c, HI, dI, g, dg = 4096, 1024, 64, C, 16, 128, 8, 1024
    gen = torch.Generator(device="cuda").manual_seed(seed)

    def wt(n, k):
        return (torch.randn(n, k, device="cuda", generator=gen) * k ** -0.5).to(torch.bfloat16)

    maps = [("q_down", d, dq), ("q_up", dq, H * c), ("kv_ca_za_cb_zb", d, 4 * c), ("idx_keys_4x128", d, 4 * dI),
            ("idx_q", dq, HI * dI), ("idx_w", d, HI)]
    ws = {nm: wt(n, k) for nm, k, n in maps}
    wg = torch.stack([wt(dg, H // g * c) for _ in range(g)])
    wo = wt(d, g * dg)
    res = {}
    for T in (4096, 1):
        xs = {k: torch.randn(T, k, device="cuda", generator=gen).to(torch.bfloat16) for k in (d, dq)}
        o = torch.randn(T, H, c, device="cuda", generator=gen).to(torch.bfloat16)
        mid = torch.empty(T, g * dg, dtype=torch.bfloat16, device="cuda")
        out = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        row = {}
        tot_ms, tot_fl, tot_by = 0.0, 0.0, 0.0
        # one decode token streams each weight once: its reps read distinct copies (the replay touches more
        # than the 256 MB memory-side cache for the large maps)
        ncp = reps if T == 1 else 1
        for nm, k, n in maps + [("grouped_out_proj", H * c, d)]:
            if nm == "grouped_out_proj":
                cps = [(wg, wo)] + [(wg.clone(), wo.clone()) for _ in range(ncp - 1)]
                fns = [lambda a=a, b=b: lca.grouped_out_proj(o, a, b, mid, out, g=g) for a, b in cps]
                fl = 2.0 * T * (g * dg * (H // g) * c + d * g * dg)
                by = 2.0 * (g * dg * (H // g) * c + d * g * dg + T * (H * c + 2 * g * dg + d))
            else:
                y = torch.empty(T, n, dtype=torch.bfloat16, device="cuda")
                cps = [ws[nm]] + [ws[nm].clone() for _ in range(ncp - 1)]
                fns = [lambda x=xs[k], w=w, y=y: lca.linear(x, w, y) for w in cps]
                fl = 2.0 * T * n * k
                by = 2.0 * (n * k + T * (k + n))
            for fn in fns:
                fn()
            torch.cuda.synchronize()
            # the reps as one captured graph: a decode token's launches are a few microseconds each, below
            # the host's cost of an eager launch from Python
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for r in range(reps):
                    fns[r % len(fns)]()
            gr.replay()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            gr.replay()
            e.record()
            torch.cuda.synchronize()
            del gr, cps, fns
            ms = s.elapsed_time(e) / reps
            tot_ms, tot_fl, tot_by = tot_ms + ms, tot_fl + fl, tot_by + by
            row[nm] = dict(ms=ms, tflops=fl / (ms * 1e-3) / 1e12, gbs=by / (ms * 1e-3) / 1e9)
        row["total"] = dict(ms=tot_ms, tflops=tot_fl / (tot_ms * 1e-3) / 1e12,
                            mfma_frac=tot_fl / (tot_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                            gbs=tot_by / (tot_ms * 1e-3) / 1e9, hbm_frac=tot_by / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
        res[f"T{T}"] = row
    return res


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the 1M decode workload
# ----------------------------------------------------------------------------

def _cpu_sample(seed: int, n_steps: int, start_barrier=None):
    """One oracle copy of the 1M stack (random stored cache bytes of the benchmark's shapes) decoding n_steps
    tokens; returns the seconds of the decode steps alone."""
    import oracle as orc
    t0 = T0_1M
    g = S.stream(seed, "cpu/bytes")

    def kv_random(n, fmt=orc.FP8):
        kv = orc.KV.empty(fmt, 1, n, 512, 64)
        codes = g.integers(0, 256, size=kv.nope.shape, dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] &= 0xFE          # no NaN codes
        kv.nope[...] = codes
        kv.scale[...] = np.exp2(g.integers(-9, -4, size=kv.scale.shape)).astype(np.float32)
        kv.rope[...] = S.to_bf16(g.standard_normal(kv.rope.shape).astype(np.float32))
        return kv

    layers = []
    for spec, tag in zip(STACK_SPECS, STACK_TAGS):
        cap = (t0 + n_steps + 8) // spec.m + 2
        d = dict(spec=spec, comp=kv_random(cap), win=kv_random(8192))
        if spec.kind == "csa":
            d["keys"] = S.to_bf16(g.standard_normal((1, cap, 128)).astype(np.float32))
        d["raw"] = [S.to_bf16(S.activations(seed, f"cpu/{tag}/{n}", (1, 2 * spec.m + n_steps, C)))
                    for n in ("ca", "za", "cb", "zb")]
        layers.append(d)
    q = S.to_bf16(S.normal(seed, "cpu/q", (1, 1, 64, C)))
    qi = S.to_bf16(S.normal(seed, "cpu/qi", (1, 1, 16, 128)))
    w = S.normal(seed, "cpu/w", (1, 1, 16), 0.25)
    sink = S.normal(seed, "cpu/sink", (64,))
    gamma = np.ones(C, np.float32)
    orc.lib()
    if start_barrier is not None:
        start_barrier.wait()
    start = time.perf_counter()
    for j in range(n_steps):
        t = t0 + j
        for d in layers:
            spec = d["spec"]
            base = t0 - 2 * spec.m
            r = [x[:, t - base:t - base + 1] for x in d["raw"]]
            orc.kv_compress(r[0], r[1], None, None, d["win"], m=1, overlap=0, first_pos=[t], gamma=gamma,
                            rope_theta=1e4, ring=1)
            if (t + 1) % spec.m == 0:
                lo = t + 1 - (1 + spec.overlap) * spec.m
                rr = [x[:, lo - base:t + 1 - base] for x in d["raw"]]
                orc.kv_compress(rr[0], rr[1], rr[2] if spec.overlap else None, rr[3] if spec.overlap else None,
                                d["comp"], m=spec.m, overlap=spec.overlap, first_pos=[lo], gamma=gamma,
                                rope_theta=1e4)
            if spec.kind == "csa":
                sc = orc.indexer_score(qi, w, d["keys"], q_pos=[t], m=4, score_fmt=orc.BF16)
                idx = orc.topk_select(sc, q_pos=[t], m=4, k=spec.k)
                orc.attention(q, q_pos=[t], comp=d["comp"], m=4, idx=idx, win=d["win"], n_win=128, sink=sink,
                              sm_scale=C ** -0.5, rope_theta=1e4, out_fmt=orc.BF16)
            else:
                orc.attention(q, q_pos=[t], comp=d["comp"], m=128, idx=None, win=d["win"], n_win=128, sink=sink,
                              sm_scale=C ** -0.5, rope_theta=1e4, out_fmt=orc.BF16)
    return time.perf_counter() - start


def _cpu_proc(seed: int, n_steps: int, barrier, results):
    try:
        results.put((seed, _cpu_sample(seed, n_steps, barrier)))
    except BaseException as e:  # (reported by the parent; the barrier is broken so no copy waits forever)
        barrier.abort()
        results.put((seed, repr(e)))


def cpu_baseline(n_steps: int = 4, seed: int = 1005, max_workers: int = 16):
    """The fp64 oracle on the host: one copy of the 1M stack per host core (at most max_workers), each
    decoding n_steps tokens in its own process (the oracle works one query row at a time, so a decode row
    keeps one core busy); tokens/s = copies x n_steps / the slowest copy's decode time.  The copies start
    their decode steps together (a barrier after building their caches)."""
    import multiprocessing as mp
    n = max(1, min(max_workers, os.cpu_count() or 1))
    log(f"cpu baseline: oracle, {n} copies x {n_steps} decode steps of the 1M stack")
    ctx = mp.get_context("spawn")
    env_prev = os.environ.get("OMP_NUM_THREADS")
    os.environ["OMP_NUM_THREADS"] = "1"          # (one row per oracle call: one thread each)
    try:
        barrier = ctx.Barrier(n, timeout=900)
        results = ctx.Queue()
        procs = [ctx.Process(target=_cpu_proc, args=(seed + i, n_steps, barrier, results)) for i in range(n)]
        for pr in procs:
            pr.start()
        got = [results.get(timeout=1800) for _ in procs]
        for pr in procs:
            pr.join()
    finally:
        if env_prev is None:
            os.environ.pop("OMP_NUM_THREADS", None)
        else:
            os.environ["OMP_NUM_THREADS"] = env_prev
    bad = [v for _, v in got if isinstance(v, str)]
    if bad:
        raise RuntimeError(f"cpu baseline copy failed: {bad[0]}")
    els = [v for _, v in got]
    el = max(els)
    return dict(value=n * n_steps / el, unit="tokens/s", cores=n, kind="oracle",
                host=dict(cpu=host_cpu(), nproc=os.cpu_count()),
                sample=f"{n} oracle copies of the 1M-context 4-layer stack, one per host core, each decoding "
                       f"{n_steps} tokens (fp64; random stored cache bytes of the benchmark's shapes); slowest "
                       f"copy {el:.1f} s, fastest {min(els):.1f} s")


# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill and the 32 x 128K decode")
    ap.add_argument("--mxfp4", action="store_true",
                    help="with --no-extra: still time the 1M decode with the MXFP4 indexer (no recall)")
    ap.add_argument("--paged", action="store_true", help="with --no-extra: still time the paged-cache decode")
    ap.add_argument("--prefill-only", action="store_true",
                    help="profiling mode: build the 1M stack, run its 4096-token chunk (3 reps), print nothing else")
    ap.add_argument("--compressor-only", action="store_true",
                    help="profiling mode: time the compressor's three calls, print their figures, nothing else")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (reference for rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lca.lib()  # fail loudly when the HIP library is missing
    torch.cuda.set_device(0)
    K, W, R = args.steps, args.warmup, args.replicas
    if args.calibrate_copy:
        calibrate_copy()
    if args.prefill_only:
        base = Stack(STACK_SPECS, STACK_TAGS, 1, T0_1M, 4, 1, 1005, win_cap=8192, raw_span=4096)
        pf = bench_prefill_1m(base, reps=3)
        log(f"1M prefill chunk: {pf['ms']:.2f} ms ({pf['tokens_per_s']:.0f} tok/s); kernels (ms): "
            + ", ".join(f"{k} {v:.3f}" for k, v in pf['kernel_ms'].items()))
        return
    if args.compressor_only:
        cp = bench_compressor()
        log("compressor: " + ", ".join(f"{k} {v['launch_ms'] * 1e3:.1f} us = {v['gbs']:.0f} GB/s ({v['bytes']} B)"
                                       for k, v in cp.items()))
        return

    d = bench_decode_1m(W, K, R)
    res, stacks = d
    res["roofline"]["copy_ceiling_gbs"] = copy_ceiling_gbs()
    log(f"1M decode: {res['ms_per_step'] * 1e3:.1f} us/step, {res['tokens_per_s']:.0f} tok/s, "
        f"{res['step_hbm']['gbs']:.0f} GB/s over the step ({100 * res['step_hbm']['frac']:.1f} % of HBM peak); "
        f"indexer + top-k {res['indexer_ms'] * 1e3:.1f} us = {res['roofline']['achieved']:.0f} GB/s")
    extra = {}
    if not args.no_extra or args.mxfp4:
        f4 = bench_decode_1m_mxfp4(stacks, W, K, recall=not args.no_extra)
        log(f"1M decode, MXFP4 indexer: {f4['ms_per_step'] * 1e3:.1f} us/step, {f4['tokens_per_s']:.0f} tok/s; "
            f"indexer {f4['indexer']['launch_ms'] * 1e3:.1f} us = {f4['indexer']['gbs']:.0f} GB/s")
        if f4["recall_top2048"]:
            log(f"top-2048 recall vs f32 scores: bf16 {f4['recall_top2048']['bf16_scores_vs_f32']:.4f}, MXFP4 QK "
                f"{f4['recall_top2048']['mxfp4_qk_vs_f32']:.4f}")
        extra["decode_1m_mxfp4_indexer"] = f4
    if not args.no_extra:
        tp = bench_topk_precision(stacks[0])
        log(f"top-2048 selector on the same 1M rows: f32 scores {tp['f32_ms'] * 1e3:.1f} us, bf16 "
            f"{tp['bf16_ms'] * 1e3:.1f} us ({tp['speedup']:.1f}x), recall {tp['recall_bf16_vs_f32']:.4f}")
        extra["topk_bf16_vs_f32_scores"] = tp
    if not args.no_extra or args.paged:
        pf = None
        if not args.no_extra:
            pf = bench_prefill_1m(stacks[0])
            log(f"1M prefill chunk: {pf['ms']:.2f} ms, {pf['tokens_per_s']:.0f} tok/s, {pf['tflops']:.0f} TFLOP/s")
            extra["prefill_1m_chunk4096"] = pf
        extra["decode_1m_paged_cache"] = bench_paged(stacks, W, K, res["ms_per_step"], pf and pf["ms"])
    if not args.no_extra:
        del stacks
        torch.cuda.empty_cache()
        c4 = bench_decode_c4(W, min(K, 64))
        log(f"32 x 128K decode: {c4['ms_per_step'] * 1e3:.1f} us/step, {c4['tokens_per_s']:.0f} tok/s; with the MXFP4 "
            f"indexer {c4['mxfp4_indexer']['ms_per_step'] * 1e3:.1f} us/step, {c4['mxfp4_indexer']['tokens_per_s']:.0f} tok/s")
        extra["decode_csa_b32_128k"] = c4
        torch.cuda.empty_cache()
        for kind, T in (("csa", 8192), ("hca", 65536)):
            r = bench_prefill_single(kind, T)
            log(f"{kind.upper()} prefill of {T} tokens: {r['ms']:.2f} ms, {r['tokens_per_s']:.0f} tok/s, "
                f"{r['tflops']:.0f} TFLOP/s ({100 * r['mfma_frac']:.1f} % of the bf16 MFMA peak)")
            extra[f"prefill_{kind}_{T}"] = r
            torch.cuda.empty_cache()
        cp = bench_compressor()
        log("compressor: " + ", ".join(f"{k} {v['launch_ms'] * 1e3:.1f} us = {v['gbs']:.0f} GB/s" for k, v in cp.items()))
        extra["compressor"] = cp
        torch.cuda.empty_cache()
        pj = bench_projections()
        log(f"layer projections: 4096-token chunk {pj['T4096']['total']['ms']:.2f} ms "
            f"({pj['T4096']['total']['tflops']:.0f} TFLOP/s), one decode token {pj['T1']['total']['ms'] * 1e3:.1f} us "
            f"({pj['T1']['total']['gbs']:.0f} GB/s)")
        extra["layer_projections"] = pj
    else:
        del stacks
    cpu = None if args.no_cpu else cpu_baseline()
    line = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode, 4-layer HCA/HCA/CSA/HCA stack, 1 sequence at 1,048,576 tokens",
                   "global_batch": 1, "seq_len": T0_1M, "layers": "HCA,HCA,CSA,HCA", "csa_entries": 262144,
                   "hca_entries": 8192, "top_k": 2048, "n_win": 128, "heads": 64, "head_dim": "512+64",
                   "kv": "fp8-e4m3 (pow2 scale / 128 dims) + bf16 rope", "indexer": "16x128 bf16, bf16 scores",
                   "replicas": R, "parallelism": "single GPU"},
        "roofline": res["roofline"],
        "step_hbm": res["step_hbm"],
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
