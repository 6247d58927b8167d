"""End-to-end decode parity of the paths the benchmark times beyond the per-workload tests.

* CSA decode with MXFP4 indexer keys through Layer.step (the fused indexer_topk_mxfp4 call), at the
  shapes of the 32 x 131,072-token decode, against the oracle's MXFP4 keys, MXFP4 scores, top-k
  and attention ("DeepSeek-V4 中文翻译" section 5.2.1: the indexer's QK path in FP4).
* The graph-replayed decode the benchmark times: bench.timed_graph_decode captures K steps of the
  1M-context 4-layer stack over rotating replicas and replays the graph; every captured step's
  outputs and CSA selection are compared with the oracle, after the benchmark's two replays and
  again after a third replay with unrelated eager work in between (bit-identical to the second).
* NaN poisoning of the CSA side: NaN in entries no row selects, in indexer keys past vis(t), and
  index lists that name entries a row cannot see (block-level causality, section 2.3.1) or ids past
  the cache change no visible score, no selection and no output bit.

Bars as the other end-to-end tests: selections equal on decided rows and recall >= 99.9 %;
outputs within 2e-2 (bf16 outputs: plus one bf16 step) on rows whose selections agree.
"""
import numpy as np
import pytest
import torch

import lca_synth as S
import long_context_attention_22_amd as lca
import oracle as orc
from gpu_util import dev, host, kv_dev
from test_gpu_configs import _check_rows, _oracle_attend, _oracle_layer, _oracle_step, _queries

pytestmark = pytest.mark.gpu
C = 576


def _oracle_mxfp4_keys(L, cap):
    """The oracle's MXFP4 copy of a layer's bf16 indexer keys: each row quantised on its own, as
    bench.keys_to_mxfp4 stores them through the library's compressor (m = 1, no norm)."""
    kb = L["keys"]
    k4 = orc.KV.empty(orc.MXFP4, kb.shape[0], cap, 128, 0)
    orc.kv_compress(kb, np.zeros_like(kb), None, None, k4, m=1, overlap=0, first_pos=[0] * kb.shape[0])
    return k4


@pytest.mark.slow
def test_mxfp4_keys_csa_decode_b32_128k():
    """32 sequences at 131,072 tokens with MXFP4 indexer keys: decode steps 0..4 (an entry and its
    MXFP4 key complete at step 3) through indexer_topk_mxfp4, sampled sequences against the oracle."""
    import bench
    seed, B, t0, W, tag = 1004, 32, 131072, 5, "c4_csa"
    spec = bench.LayerSpec("csa", 4, k=1024)
    st = bench.Stack([spec], [tag], B, t0, W, 1, seed, win_cap=256)
    layer = st.layers[0]
    bench.keys_to_mxfp4(layer)
    assert layer.keys.fmt == lca.MXFP4 and layer.fuse_topk
    bseqs = [0, 13, 31]
    L = _oracle_layer(seed, spec, tag, B, t0, 256, layer.comp.cap, bseqs, st.raws[0].c_a.shape[1])
    L["k4"] = _oracle_mxfp4_keys(L, layer.comp.cap)
    q, qi, w = _queries(seed, tag, spec, W, B)
    calls = []
    gi, go, oi, os32, oo = [], [], [], [], []
    for j in range(W):
        st.decode(j, record=lambda name, fn: (calls.append(name), fn()))
        torch.cuda.synchronize()
        t = t0 + j
        _oracle_step(L, spec, t, 1)
        ix, s32, o = _oracle_attend(L, spec, t, q[j][bseqs], qi[j][bseqs], w[j][bseqs])
        gi += list(host(layer.idx)[bseqs, 0])
        go += list(host(st.out[0])[bseqs, 0])
        oi += list(ix[:, 0])
        os32 += list(s32[:, 0])
        oo += list(o[:, 0])
    assert calls.count("indexer_topk") == W and "indexer_score" not in calls
    # the MXFP4 keys the decode stored (entry 32768 at step 3) equal the oracle's bytes
    e = (t0 + 4) // 4 - 1
    g4n, g4s = host(layer.keys.nope)[bseqs, e], host(layer.keys.scale)[bseqs, e]
    np.testing.assert_array_equal(g4s, L["k4"].scale[:, e])
    np.testing.assert_array_equal(g4n, L["k4"].nope[:, e])
    _check_rows("config4 mxfp4 keys", gi, oi, os32, go, oo, lambda r: (t0 + r // len(bseqs) + 1) // 4, spec.k)


class _StepCopies:
    """Record hook for bench.timed_graph_decode: after each attention launch, copy the layer's output
    (and the CSA layer's selection) into a buffer of its own, so every captured step can be read back
    after a replay."""

    def __init__(self, stacks, W, K):
        self.pairs = []
        self.stacks, self.W = stacks, W
        nl = len(stacks[0].layers)
        self.out = {(i, li): torch.empty_like(stacks[0].out[li]) for i in range(W, W + K) for li in range(nl)}
        self.idx = {(i, li): torch.empty(1, 1, ly.spec.k, dtype=torch.int32, device="cuda")
                    for i in range(W, W + K) for li, ly in enumerate(stacks[0].layers) if ly.spec.kind == "csa"}
        self.n = 0

    def __call__(self, name, fn):
        fn()
        if name not in ("csa_attn", "hca_attn"):
            return
        nl = len(self.stacks[0].layers)
        i, li = self.W + self.n // nl, self.n % nl
        self.n += 1
        st = self.stacks[i % len(self.stacks)]
        self.out[(i, li)].copy_(st.out[li])
        if (i, li) in self.idx:
            self.idx[(i, li)].copy_(st.layers[li].idx.view(-1)[:st.layers[li].spec.k].view(1, 1, -1))

    def snapshot(self):
        return ({k: host(v) for k, v in self.out.items()}, {k: host(v) for k, v in self.idx.items()})


@pytest.mark.slow
def test_graph_replayed_1m_decode_matches_oracle():
    import bench
    seed, t0, R, W, K = 1005, 1 << 20, 2, 2, 8
    specs, tags = bench.STACK_SPECS, bench.STACK_TAGS
    n_pos = (W + K + R - 1) // R + 2
    base = bench.Stack(specs, tags, 1, t0, n_pos, 1, seed, win_cap=8192, raw_span=4096)
    stacks = [base] + [base.replicate() for _ in range(R - 1)]
    rec = _StepCopies(stacks, W, K)
    _, g = bench.timed_graph_decode(stacks, W, K, rec)
    assert rec.n == K * len(specs)
    torch.cuda.synchronize()
    outs, idxs = rec.snapshot()
    # a third replay after unrelated eager work: the same bits
    x = torch.randn(2048, 2048, device="cuda")
    (x @ x).sum().item()
    g.replay()
    torch.cuda.synchronize()
    outs3, idxs3 = rec.snapshot()
    for key in outs:
        assert np.array_equal(outs[key], outs3[key]), f"replay 3 output differs at {key}"
    for key in idxs:
        assert np.array_equal(idxs[key], idxs3[key]), f"replay 3 selection differs at {key}"
    del g
    # the oracle, advanced position by position (step i ran position t0 + i // R on replica i % R)
    Ls = [_oracle_layer(seed, sp, tg, 1, t0, 8192, ly.comp.cap, [0], base.raws[li].c_a.shape[1])
          for li, (sp, tg, ly) in enumerate(zip(specs, tags, base.layers))]
    qs = [_queries(seed, tg, sp, n_pos, 1) for sp, tg in zip(specs, tags)]
    res = {li: ([], [], [], [], [], []) for li in range(len(specs))}
    for i in range(W, W + K):
        j = i // R
        t = t0 + j
        for li, (sp, L) in enumerate(zip(specs, Ls)):
            if t + 1 > L["done"]:
                _oracle_step(L, sp, L["done"], t + 1 - L["done"])
                L["done"] = t + 1
            q, qi, w = qs[li]
            ix, s32, o = _oracle_attend(L, sp, t, q[j], None if qi is None else qi[j], None if w is None else w[j])
            gi, go, oi, os32, oo, vis = res[li]
            go.append(outs[(i, li)][0, 0])
            oo.append(o[0, 0])
            vis.append((t + 1) // sp.m)
            if sp.kind == "csa":
                gi.append(idxs[(i, li)][0, 0]), oi.append(ix[0, 0]), os32.append(s32[0, 0])
    for li, sp in enumerate(specs):
        gi, go, oi, os32, oo, vis = res[li]
        _check_rows(f"graph replay layer {li} ({sp.kind})", gi, oi, os32, go, oo, lambda r: vis[r], sp.k)


# ---------------------------------------------------------------------------
# NaN poisoning of the CSA side
# ---------------------------------------------------------------------------

BF16_NAN = 0x7FC0


def _csa_case(seed, B, T, q_pos, k, fmt):
    """Caches, indexer inputs and queries of a CSA launch (m = 4, window 128)."""
    m, n_win, H = 4, 128, 64
    vis_last = [(p + T) // m for p in q_pos]
    cap = max(vis_last) + 40                       # rows past every visible count exist
    x = np.stack([S.block_scaled(seed, "ent", b, cap, C) for b in range(B)])
    comp = orc.KV.empty(fmt, B, cap, 512, 64)
    orc.kv_compress(x, np.zeros_like(x), None, None, comp, m=1, overlap=0, first_pos=[0] * B)
    wcap = 512
    xw = np.stack([S.block_scaled(seed, "win", b, wcap, C) for b in range(B)])
    win = orc.KV.empty(fmt, B, wcap, 512, 64)
    orc.kv_compress(xw, np.zeros_like(xw), None, None, win, m=1, overlap=0, first_pos=[0] * B, ring=1)
    keys = S.to_bf16(S.normal(seed, "keys", (B, cap, 128)))
    qi = S.to_bf16(S.normal(seed, "qi", (B, T, 16, 128)))
    w = S.normal(seed, "w", (B, T, 16), 0.25)
    q = S.to_bf16(S.normal(seed, "q", (B, T, H, C)))
    sink = S.normal(seed, "sink", (H,))
    return dict(m=m, n_win=n_win, H=H, cap=cap, vis_last=vis_last, comp=comp, win=win, keys=keys, qi=qi, w=w, q=q,
                sink=sink, k=k, q_pos=q_pos, B=B, T=T)


def _select(c, keys_dev, decode):
    """Scores and selection on the GPU: the fused decode call, or indexer_score + topk_select."""
    B, T, cap, k = c["B"], c["T"], c["cap"], c["k"]
    sc = torch.zeros(B, T, cap, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(B, T, k, dtype=torch.int32, device="cuda")
    if decode:
        ws = torch.zeros(max(16, lca.indexer_topk_workspace_size(B, 1, cap, k)), dtype=torch.uint8, device="cuda")
        if keys_dev.fmt == lca.MXFP4:
            lca.indexer_topk_mxfp4(dev(c["qi"]), dev(c["w"]), keys_dev, sc, idx, q_pos=c["q_pos"], m=c["m"], ws=ws)
        else:
            lca.indexer_topk(dev(c["qi"]), dev(c["w"]), keys_dev.nope, sc, idx, q_pos=c["q_pos"], m=c["m"], ws=ws)
    else:
        ws = torch.zeros(max(16, lca.topk_workspace_size(B, T, cap, k)), dtype=torch.uint8, device="cuda")
        lca.indexer_score(dev(c["qi"]), dev(c["w"]), keys_dev.nope, sc, q_pos=c["q_pos"], m=c["m"])
        lca.topk_select(sc, idx, q_pos=c["q_pos"], m=c["m"], ws=ws)
    torch.cuda.synchronize()
    return host(sc), host(idx)


def _attend(c, comp, win, idx):
    B, T, H = c["B"], c["T"], c["H"]
    k2 = idx.shape[2]
    out = torch.zeros(B, T, H, C, dtype=torch.float32, device="cuda")
    lse = torch.zeros(B, T, H, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(16, lca.attn_workspace_size(B, T, H, C, k2 + c["n_win"])), dtype=torch.uint8, device="cuda")
    lca.csa_attn(dev(c["q"]), out, q_pos=c["q_pos"], comp=comp, m=c["m"], idx=dev(idx), win=win, n_win=c["n_win"],
                 sink=dev(c["sink"]), sm_scale=C ** -0.5, rope_theta=1e4, lse=lse, ws=ws)
    torch.cuda.synchronize()
    return host(out), host(lse)


@pytest.mark.parametrize("case", ["decode_bf16keys", "decode_mxfp4keys", "prefill"])
def test_csa_nan_poison_and_invisible_ids(case):
    decode = case.startswith("decode")
    if decode:
        c = _csa_case(77, 3, 1, [5000, 3001, 1302], 256, orc.FP8)
    else:
        c = _csa_case(78, 2, 37, [2100, 640], 64, orc.FP8)
    B, T, cap, k = c["B"], c["T"], c["cap"], c["k"]
    fp4 = case == "decode_mxfp4keys"
    # clean run
    kb = lca.KV(dev(c["keys"]), None, None, lca.BF16, 128, 0, cap)
    if fp4:
        k4 = lca.KV.empty(lca.MXFP4, B, cap, 128, 0)
        lca.kv_compress(kb.nope, torch.zeros_like(kb.nope), None, None, k4, m=1, overlap=0, first_pos=0)
        kb = k4
    sc0, idx0 = _select(c, kb, decode)
    # room for ids a row cannot see: k + 8 columns, the extra ones -1 in the clean list
    ext = np.concatenate([idx0, np.full((B, T, 8), -1, np.int32)], -1)
    comp0, win0 = kv_dev(c["comp"]), kv_dev(c["win"])
    out0, lse0 = _attend(c, comp0, win0, ext)
    assert np.isfinite(out0).all()

    # poisoned: keys past the launch's last visible count NaN (MXFP4: E8M0 NaN scale bytes), entries no
    # row of the sequence selects NaN (scale), and the extra columns naming invisible entries / ids past
    # the cache
    kp = c["keys"].copy()
    for b in range(B):
        kp[b, c["vis_last"][b]:] = BF16_NAN
    kbp = lca.KV(dev(kp), None, None, lca.BF16, 128, 0, cap)
    if fp4:
        kbp = lca.KV(kb.nope.clone(), None, kb.scale.clone(), lca.MXFP4, 128, 0, cap)
        for b in range(B):
            kbp.scale[b, c["vis_last"][b]:] = 0xFF
    sc1, idx1 = _select(c, kbp, decode)
    for b in range(B):
        for i in range(T):
            vis = min((c["q_pos"][b] + i + 1) // c["m"], cap)
            np.testing.assert_array_equal(sc1[b, i, :vis], sc0[b, i, :vis])
    np.testing.assert_array_equal(idx1, idx0)
    cp = orc.KV(c["comp"].nope.copy(), c["comp"].rope.copy(), c["comp"].scale.copy(), orc.FP8, 512, 64, cap)
    for b in range(B):
        used = np.zeros(cap, bool)
        sel = idx0[b][idx0[b] >= 0]
        used[sel] = True
        cp.scale[b, ~used] = np.nan
    bad = ext.copy()
    for b in range(B):
        for i in range(T):
            vis = min((c["q_pos"][b] + i + 1) // c["m"], cap)
            bad[b, i, k:] = [vis, vis + 1, cap - 1, cap, cap + 3, 1 << 20, (1 << 31) - 1, vis + 7]
    out1, lse1 = _attend(c, kv_dev(cp), win0, bad)
    np.testing.assert_array_equal(out1, out0)
    np.testing.assert_array_equal(lse1, lse0)
    # and the clean output against the oracle on the clean caches
    oo, _ = orc.attention(c["q"], q_pos=c["q_pos"], comp=c["comp"], m=c["m"], idx=idx0, win=c["win"],
                          n_win=c["n_win"], sink=c["sink"], sm_scale=C ** -0.5, rope_theta=1e4)
    err = float(np.abs(out0 - oo).max())
    assert err <= 2e-2, err
    print(f"{case}: poisoned run bit-identical, max-abs vs oracle {err:.2e}")
