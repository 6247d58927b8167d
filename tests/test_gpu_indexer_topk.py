"""lca_indexer_topk: the decode indexer with the top-k's first histogram pass fused into it.

The fused call must give the scores and selections of lca_indexer_score followed by lca_topk_select
bit for bit (both are checked against the oracle elsewhere), and the top-k of its scores must equal
the oracle's top-k of the same bf16 scores.  The part of its workspace that must start at zero is
cleared again by every call, so calls follow each other (and replays of a captured graph) with no reset: several calls in a row on one workspace,
rows of mixed lengths in one batch (split and trivial rows), the non-split schedule, and a graph
replayed three times with eager work in between.
"""
import numpy as np
import pytest
import torch

import long_context_attention_22_amd as lca
import oracle as orc
from gpu_util import host

pytestmark = pytest.mark.gpu


def _inputs(seed, B, cap, ties=False):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, 1, 16, 128, device="cuda", generator=g).to(torch.bfloat16)
    w = torch.randn(B, 1, 16, device="cuda", generator=g) * 0.25
    if ties:  # every score 0: the whole row ties, the first k indices win
        w.zero_()
    k = torch.randn(B, cap, 128, device="cuda", generator=g).to(torch.bfloat16)
    return q, w, k


def _check_ws(ws, B, T, s_stride, q_pos, m=4):
    """Every call leaves the part of the workspace that must start at zero zeroed again: the first-pass
    histograms at its start, 128 words (16-bit counts) per row and 4096-key chunk when the rows are few
    and long (more than 16384 candidates: the split schedule), else 256 words per row."""
    rows, max_vis = B * T, max((p + T) // m for p in q_pos)
    split = rows < 128 and max_vis > 16384
    nz = rows * (512 * -(-s_stride // 4096) if split else 1024)
    assert nz <= ws.numel()
    assert int(ws[:nz].count_nonzero()) == 0


def _separate(q, w, k, q_pos, m, s_stride, topk):
    B = q.shape[0]
    sc = torch.zeros(B, 1, s_stride, dtype=torch.bfloat16, device="cuda")
    ix = torch.empty(B, 1, topk, dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(16, lca.topk_workspace_size(B, 1, s_stride, topk)), dtype=torch.uint8, device="cuda")
    lca.indexer_score(q, w, k, sc, q_pos=q_pos, m=m)
    lca.topk_select(sc, ix, q_pos=q_pos, m=m, ws=ws)
    return sc, ix


def _vis_cols(sc, q_pos, m):
    """Scores restricted to each row's visible columns (the rest is unspecified)."""
    return [host(sc[b, 0, :(p + 1) // m]) for b, p in enumerate(q_pos)]


@pytest.mark.parametrize("B,cap,topk,pos_list,ties", [
    (1, 262160, 2048, [[(1 << 20) + 3], [(1 << 20) + 7], [(1 << 20) + 11]], False),  # 1M decode, three calls
    (32, 32800, 1024, [[131071 + 4 * b for b in range(32)], [131075] * 32], False),  # 32 x 128K
    (3, 300016, 2048, [[1199995, 20003, 6000], [1200003, 65539, 8191]], False),      # mixed lengths, trivial rows
    (2, 12000, 512, [[40000, 47000]], False),                                         # the row schedule
    (1, 262160, 2048, [[(1 << 20) + 3], [(1 << 20) + 7]], True),                      # a row of equal scores
    (1, 1048600, 2048, [[(1 << 22) + 3]], False),                                     # a 4M-token row, 65 chunks
])
def test_indexer_topk_matches_separate_calls(B, cap, topk, pos_list, ties):
    m = 4
    s_stride = cap
    nbytes = lca.indexer_topk_workspace_size(B, 1, s_stride, topk)
    ws = torch.zeros(max(16, nbytes), dtype=torch.uint8, device="cuda")
    for call, q_pos in enumerate(pos_list):
        q, w, k = _inputs(100 + call, B, cap, ties)
        sc = torch.zeros(B, 1, s_stride, dtype=torch.bfloat16, device="cuda")
        ix = torch.empty(B, 1, topk, dtype=torch.int32, device="cuda")
        lca.indexer_topk(q, w, k, sc, ix, q_pos=q_pos, m=m, ws=ws)
        sc_ref, ix_ref = _separate(q, w, k, q_pos, m, s_stride, topk)
        torch.cuda.synchronize()
        for b, (a, r) in enumerate(zip(_vis_cols(sc, q_pos, m), _vis_cols(sc_ref, q_pos, m))):
            assert np.array_equal(a, r), (call, b)
        assert torch.equal(ix, ix_ref), call
        # the oracle's top-k of the same bf16 scores
        for b, p in enumerate(q_pos):
            n = (p + 1) // m
            row = np.zeros((1, 1, s_stride), np.uint16)
            row[0, 0, :n] = host(sc[b, 0, :n])
            o_ix = orc.topk_select(row, q_pos=[p], m=m, k=topk)
            assert np.array_equal(o_ix[0, 0], host(ix[b, 0])), (call, b)
        _check_ws(ws, B, 1, s_stride, q_pos)


def _inputs_rows(seed, B, T, cap):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, T, 16, 128, device="cuda", generator=g).to(torch.bfloat16)
    w = torch.randn(B, T, 16, device="cuda", generator=g) * 0.25
    k = torch.randn(B, cap, 128, device="cuda", generator=g).to(torch.bfloat16)
    return q, w, k


@pytest.mark.parametrize("B,T,cap,topk,q_pos,sample", [
    (1, 4096, 263200, 2048, [1 << 20], [0, 1, 2, 1365, 4094, 4095]),   # the 1M prefill chunk: row schedule
    (1, 100, 262300, 2048, [(1 << 20) - 50], [0, 49, 50, 99]),        # few long rows, 8 per workgroup: split
    (2, 37, 300100, 1024, [1200003, 65539], [0, 36, 37, 73]),         # few long rows, one per workgroup: split
    (1, 300, 9000, 512, [30000], [0, 1, 150, 299]),                   # short rows: row schedule
])
def test_indexer_topk_prefill_rows(B, T, cap, topk, q_pos, sample):
    """Several query rows per sequence: the indexer counts every row's first radix digit while it stores
    the scores (per chunk for the split schedule, per row for the row schedule); scores and selections
    equal the separate calls bit for bit, the selections of sampled rows equal the oracle's top-k of the
    same scores, and the first-pass histograms are zero again after two calls."""
    m = 4
    nbytes = lca.indexer_topk_workspace_size(B, T, cap, topk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for call in range(2):
        q, w, k = _inputs_rows(300 + call, B, T, cap)
        sc = torch.zeros(B, T, cap, dtype=torch.bfloat16, device="cuda")
        ix = torch.empty(B, T, topk, dtype=torch.int32, device="cuda")
        lca.indexer_topk(q, w, k, sc, ix, q_pos=q_pos, m=m, ws=ws)
        sc_ref = torch.zeros_like(sc)
        ix_ref = torch.empty_like(ix)
        tws = torch.zeros(max(16, lca.topk_workspace_size(B, T, cap, topk)), dtype=torch.uint8, device="cuda")
        lca.indexer_score(q, w, k, sc_ref, q_pos=q_pos, m=m)
        lca.topk_select(sc_ref, ix_ref, q_pos=q_pos, m=m, ws=tws)
        torch.cuda.synchronize()
        assert torch.equal(ix, ix_ref), call
        for r in sample:
            b, i = divmod(r, T)
            n = (q_pos[b] + i + 1) // m
            a_, r_ = host(sc[b, i, :n]), host(sc_ref[b, i, :n])
            assert np.array_equal(a_, r_), (call, r)
            row = np.zeros((1, 1, cap), np.uint16)
            row[0, 0, :n] = a_
            o_ix = orc.topk_select(row, q_pos=[q_pos[b] + i], m=m, k=topk)
            assert np.array_equal(o_ix[0, 0], host(ix[b, i])), (call, r)
        del sc, sc_ref
        _check_ws(ws, B, T, cap, q_pos)


def test_indexer_topk_mxfp4_prefill_rows():
    B, T, cap, topk, m = 1, 200, 262300, 2048, 4
    q_pos = [(1 << 20) - 150]
    k = _mxfp4_keys(11, B, cap)
    nbytes = lca.indexer_topk_workspace_size(B, T, cap, topk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    q, w, _ = _inputs_rows(12, B, T, 16)
    sc = torch.zeros(B, T, cap, dtype=torch.bfloat16, device="cuda")
    ix = torch.empty(B, T, topk, dtype=torch.int32, device="cuda")
    lca.indexer_topk_mxfp4(q, w, k, sc, ix, q_pos=q_pos, m=m, ws=ws)
    sc_ref, ix_ref = torch.zeros_like(sc), torch.empty_like(ix)
    tws = torch.zeros(max(16, lca.topk_workspace_size(B, T, cap, topk)), dtype=torch.uint8, device="cuda")
    lca.indexer_score_mxfp4(q, w, k, sc_ref, q_pos=q_pos, m=m)
    lca.topk_select(sc_ref, ix_ref, q_pos=q_pos, m=m, ws=tws)
    torch.cuda.synchronize()
    assert torch.equal(ix, ix_ref)
    for i in (0, 99, 199):
        n = (q_pos[0] + i + 1) // m
        assert np.array_equal(host(sc[0, i, :n]), host(sc_ref[0, i, :n])), i
    _check_ws(ws, B, T, cap, q_pos)


def test_indexer_topk_graph_replays():
    B, cap, topk, m = 1, 262160, 2048, 4
    s_stride = cap
    ws = torch.zeros(lca.indexer_topk_workspace_size(B, 1, s_stride, topk), dtype=torch.uint8, device="cuda")
    q, w, k = _inputs(7, B, cap)
    pos = [(1 << 20) + 1, (1 << 20) + 2, (1 << 20) + 3]
    outs = [(torch.zeros(B, 1, s_stride, dtype=torch.bfloat16, device="cuda"),
             torch.empty(B, 1, topk, dtype=torch.int32, device="cuda")) for _ in pos]
    refs = [_separate(q, w, k, [p], m, s_stride, topk) for p in pos]
    lca.indexer_topk(q, w, k, outs[0][0], outs[0][1], q_pos=pos[0], m=m, ws=ws)  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for p, (sc, ix) in zip(pos, outs):
            lca.indexer_topk(q, w, k, sc, ix, q_pos=p, m=m, ws=ws)
    for rep in range(3):
        for sc, ix in outs:
            ix.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for (sc, ix), (_, ix_ref) in zip(outs, refs):
            assert torch.equal(ix, ix_ref), rep
        _separate(q, w, k, [pos[rep]], m, s_stride, topk)  # eager work between replays
        torch.cuda.synchronize()
        _check_ws(ws, B, 1, s_stride, pos)


def _mxfp4_keys(seed, B, cap):
    g = torch.Generator(device="cuda").manual_seed(seed)
    kv = lca.KV.empty(lca.MXFP4, B, cap, 128, 0)
    kv.nope.copy_(torch.randint(0, 256, kv.nope.shape, dtype=torch.uint8, device="cuda", generator=g))
    kv.scale.copy_(torch.randint(118, 128, kv.scale.shape, dtype=torch.uint8, device="cuda", generator=g))
    return kv


@pytest.mark.parametrize("B,cap,topk,pos_list", [
    (1, 262160, 2048, [[(1 << 20) + 3], [(1 << 20) + 7]]),
    (32, 32800, 1024, [[131071 + 4 * b for b in range(32)]]),
])
def test_indexer_topk_mxfp4_matches_separate_calls(B, cap, topk, pos_list):
    m, s_stride = 4, cap
    ws = torch.zeros(lca.indexer_topk_workspace_size(B, 1, s_stride, topk), dtype=torch.uint8, device="cuda")
    k = _mxfp4_keys(5, B, cap)
    tws = torch.zeros(max(16, lca.topk_workspace_size(B, 1, s_stride, topk)), dtype=torch.uint8, device="cuda")
    for call, q_pos in enumerate(pos_list):
        q, w, _ = _inputs(200 + call, B, 16)
        sc = torch.zeros(B, 1, s_stride, dtype=torch.bfloat16, device="cuda")
        ix = torch.empty(B, 1, topk, dtype=torch.int32, device="cuda")
        lca.indexer_topk_mxfp4(q, w, k, sc, ix, q_pos=q_pos, m=m, ws=ws)
        sc_ref = torch.zeros_like(sc)
        ix_ref = torch.empty_like(ix)
        lca.indexer_score_mxfp4(q, w, k, sc_ref, q_pos=q_pos, m=m)
        lca.topk_select(sc_ref, ix_ref, q_pos=q_pos, m=m, ws=tws)
        torch.cuda.synchronize()
        for b, (a, r) in enumerate(zip(_vis_cols(sc, q_pos, m), _vis_cols(sc_ref, q_pos, m))):
            assert np.array_equal(a, r), (call, b)
        assert torch.equal(ix, ix_ref), call
        _check_ws(ws, B, 1, s_stride, q_pos)
