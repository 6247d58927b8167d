"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/lca.h declares, and rejects bad arguments before launching.

Only error paths are exercised: a call that passed validation would launch a
kernel, which needs a GPU.  Device pointers are fake aligned addresses, never
dereferenced on the host.
"""
import ctypes as C
import os
import re

import pytest

import long_context_attention_22_amd as lca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
FAKE2 = 0x7F0000100000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lca.LIB_PATH):
        import long_context_attention_22_amd.build as bld
        bld.build()
    return lca.lib()


@pytest.fixture(scope="module")
def no_gpu():
    """Calls that pass validation launch a kernel on the fake pointers: only where no GPU is visible
    (the launch then fails with LCA_EHIP)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: a valid call would launch on fake pointers")


def _declared():
    txt = "".join(open(os.path.join(ROOT, "include", f)).read() for f in sorted(os.listdir(os.path.join(ROOT, "include")))
                  if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(lca_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) >= {"lca_kv_compress", "lca_indexer_score", "lca_topk_select", "lca_csa_attn",
                          "lca_hca_attn", "lca_attn_workspace_size", "lca_topk_workspace_size",
                          "lca_last_error", "lca_version", "lca_cache_create", "lca_cache_fork"}
    for n in names:
        assert hasattr(L, n), n
    assert L.lca_version() == 1


def kv(fmt=lca.BF16, d_nope=512, d_rope=64, cap=64, scale=True):
    return lca._KV(FAKE, FAKE2, FAKE + 4096 if (fmt == lca.FP8 and scale) else 0, fmt, d_nope, d_rope, cap)


def pos(*v):
    return (C.c_int64 * len(v))(*v)


def compress(L, **kw):
    a = dict(c_a=FAKE, z_a=FAKE, c_b=FAKE, z_b=FAKE, in_dtype=lca.BF16, bias_a=None, bias_b=None,
             gamma=None, eps=1e-6, theta=0.0, m=4, overlap=1, B=1, n_rows=64, in_stride=0,
             first_pos=pos(0), out=kv(), ring=0)
    a.update(kw)
    return L.lca_kv_compress(a["c_a"], a["z_a"], a["c_b"], a["z_b"], a["in_dtype"], a["bias_a"], a["bias_b"],
                             a["gamma"], a["eps"], a["theta"], a["m"], a["overlap"], a["B"], a["n_rows"],
                             a["in_stride"], a["first_pos"], a["out"], a["ring"], None)


def test_kv_compress_validation(L):
    assert compress(L, c_a=None) == 1
    assert compress(L, m=0) == 1
    assert compress(L, overlap=2) == 1
    assert compress(L, c_b=None) == 1                       # overlap needs the b-set
    assert compress(L, in_dtype=2) == 3
    assert compress(L, B=0, first_pos=pos()) == 2
    assert compress(L, B=65, first_pos=pos(*([0] * 65))) == 2
    assert compress(L, first_pos=pos(-4)) == 2
    assert compress(L, out=kv(lca.FP8, d_nope=96, d_rope=32)) == 2      # fp8 needs d_nope % 128
    assert compress(L, out=kv(lca.FP8, scale=False)) == 1
    assert compress(L, out=kv(d_rope=63)) == 2
    assert compress(L, out=kv(fmt=7)) == 3
    assert compress(L, c_a=FAKE + 8) == 4
    # 64 rows at m=4 make entries 0..15: does not fit cap 8 without a ring
    assert compress(L, out=kv(cap=8)) == 2
    assert b"cap" in L.lca_last_error()
    assert compress(L, theta=-1.0) == 1
    assert compress(L, in_stride=63) == 2


def compress_ws(L, ws=FAKE, ws_bytes=0, **kw):
    a = dict(c_a=FAKE, z_a=FAKE, c_b=None, z_b=None, in_dtype=lca.BF16, bias_a=None, bias_b=None,
             gamma=None, eps=1e-6, theta=0.0, m=128, overlap=0, B=1, n_rows=4096, in_stride=0,
             first_pos=pos(0), out=kv(cap=64), ring=0)
    a.update(kw)
    return L.lca_kv_compress_ws(a["c_a"], a["z_a"], a["c_b"], a["z_b"], a["in_dtype"], a["bias_a"], a["bias_b"],
                                a["gamma"], a["eps"], a["theta"], a["m"], a["overlap"], a["B"], a["n_rows"],
                                a["in_stride"], a["first_pos"], a["out"], a["ring"], ws, ws_bytes, None)


def test_kv_compress_ws_validation(L):
    """The split compressor's workspace: its size for long blocks, 0 where calls never split, and the call's
    own need (32 entries x 8 parts x 3 x 576 floats) checked before any launch."""
    size = L.lca_compress_workspace_size
    assert size(lca.BF16, 128, 0, 512, 64) == 256 * 3 * 576 * 4
    assert size(lca.BF16, 32, 1, 512, 64) == 256 * 3 * 576 * 4     # 64 rows per entry with the b-block
    assert size(lca.BF16, 4, 1, 512, 64) == 0                      # 8 rows per entry: never split
    assert size(lca.F32, 128, 0, 512, 64) == 0                     # f32 inputs take the per-channel kernel
    assert size(lca.BF16, 128, 0, 600, 0) == 0                     # wider than the pooling kernel's 576
    assert size(lca.BF16, 0, 0, 512, 64) == 0
    need = 32 * 8 * 3 * 576 * 4
    assert compress_ws(L, ws_bytes=need - 1) == lca.EWORKSPACE
    assert b"workspace" in L.lca_last_error()
    assert compress_ws(L, ws=FAKE + 8, ws_bytes=need) == 4
    assert compress_ws(L, ws_bytes=need, m=0) == 1                 # the plain call's checks still apply
    assert compress_ws(L, ws_bytes=need, out=kv(cap=8)) == 2


def indexer(L, **kw):
    a = dict(q=FAKE, w=None, k=FAKE, dt=lca.BF16, k_cap=100, H=16, d=128, B=1, T=8, q_pos=pos(0), m=4,
             s=FAKE2, sdt=lca.BF16, stride=100)
    a.update(kw)
    return L.lca_indexer_score(a["q"], a["w"], a["k"], a["dt"], a["k_cap"], a["H"], a["d"], a["B"], a["T"],
                               a["q_pos"], a["m"], a["s"], a["sdt"], a["stride"], None)


def test_indexer_validation(L):
    assert indexer(L, q=None) == 1
    assert indexer(L, m=0) == 1
    assert indexer(L, dt=2) == 3
    assert indexer(L, sdt=2) == 3
    assert indexer(L, H=8) == 2                 # bf16 path is 16 heads x 128
    assert indexer(L, q_pos=pos(400)) == 2      # (400 + 8) / 4 = 102 visible > k_cap
    assert indexer(L, stride=1) == 2
    assert indexer(L, k=FAKE + 2) == 4


def topk(L, **kw):
    a = dict(s=FAKE, sdt=lca.BF16, stride=128, B=1, T=4, q_pos=pos(0), m=4, k=16, idx=FAKE2)
    a.update(kw)
    return L.lca_topk_select(a["s"], a["sdt"], a["stride"], a["B"], a["T"], a["q_pos"], a["m"], a["k"],
                             a["idx"], None, 0, None)


def test_topk_validation(L):
    assert topk(L, s=None) == 1
    assert topk(L, k=0) == 1
    assert topk(L, sdt=2) == 3
    assert topk(L, q_pos=pos(600)) == 2
    assert topk(L, idx=FAKE2 + 4) == 4
    assert L.lca_topk_workspace_size(1, 1, 1024, 16) == 0


def attn(L, csa=True, **kw):
    a = dict(q=FAKE, qdt=lca.BF16, H=64, B=1, T=4, q_pos=pos(100), comp=kv(), m=4, idx=FAKE2, k=16,
             win=kv(cap=256), n_win=128, sink=None, scale=0.04, theta=0.0, out=FAKE2, odt=lca.F32,
             lse=None, ws=None, wsb=0)
    a.update(kw)
    if csa:
        return L.lca_csa_attn(a["q"], a["qdt"], a["H"], a["B"], a["T"], a["q_pos"], a["comp"], a["m"],
                              a["idx"], a["k"], a["win"], a["n_win"], a["sink"], a["scale"], a["theta"],
                              a["out"], a["odt"], a["lse"], a["ws"], a["wsb"], None)
    return L.lca_hca_attn(a["q"], a["qdt"], a["H"], a["B"], a["T"], a["q_pos"], a["comp"], a["m"], a["win"],
                          a["n_win"], a["sink"], a["scale"], a["theta"], a["out"], a["odt"], a["lse"],
                          a["ws"], a["wsb"], None)


def test_attn_validation(L):
    assert attn(L, idx=None) == 1
    assert attn(L, k=0) == 1
    assert attn(L, n_win=-1) == 1
    assert attn(L, odt=2) == 3
    assert attn(L, qdt=lca.F32) == 3                              # bf16 cache with f32 queries
    assert attn(L, H=72) == 2                                     # MFMA path: at most 64 heads
    assert attn(L, comp=kv(d_nope=256)) == 2                      # MFMA path: 512 + 64
    assert attn(L, win=kv(cap=100)) == 2                          # min(n_win - 1, q_pos) + T > cap
    assert attn(L, q_pos=pos(0), T=100, win=kv(cap=99)) == 2
    assert attn(L, win=kv(fmt=lca.FP8, cap=256)) == 2             # window format differs
    assert attn(L, csa=False, comp=kv(cap=10)) == 2               # 26 visible entries > cap
    assert attn(L, out=FAKE2 + 4) == 4
    # decode-sized launches need a workspace for the split partials
    need = L.lca_attn_workspace_size(1, 1, 64, 576, 1152)
    assert need > 0
    assert attn(L, T=1, q_pos=pos(4000), k=1024) == 5
    assert attn(L, T=1, q_pos=pos(4000), k=1024, ws=FAKE2, wsb=64) == 5

    # prefill: one split per row; the size covers the optional bf16 expansion of a dense launch's
    # rows (2 max_keys + T rows of 1152 bytes)
    assert L.lca_attn_workspace_size(1, 4096, 64, 576, 2176) == (2 * 2176 + 4096) * 1152


@pytest.mark.parametrize("B,T,H", [(1, 1, 64), (1, 1, 16), (32, 1, 64), (3, 5, 48), (1, 127, 64), (2, 3, 24)])
def test_attn_workspace_covers_smaller_launches(L, no_gpu, B, T, H):
    """lca_attn_workspace_size(..., M) covers every launch with at most M attended rows per query: no
    such launch is refused for its workspace (it passes validation and only then fails to launch,
    here without a GPU).  The split count is not monotone in the row count; the size is."""
    m, n_win, M = 4, 128, 4224
    need = L.lca_attn_workspace_size(B, T, H, 576, M)
    sizes = []
    for qp in range(0, 4 * (M - n_win) - T, 37):          # HCA: vis + window grows with the position
        rc = attn(L, csa=False, B=B, T=T, H=H, q_pos=pos(*([qp] * B)), m=m, comp=kv(cap=M), win=kv(cap=512),
                  ws=FAKE2, wsb=need)
        assert rc != 5, (qp, L.lca_last_error())
        sizes.append(L.lca_attn_workspace_size(B, T, H, 576, min(M, (qp + T) // m + n_win)))
    for k in list(range(1, 300, 7)) + [1024, 2048, M - n_win]:   # CSA: k + window
        rc = attn(L, B=B, T=T, H=H, q_pos=pos(*([100000] * B)), k=k, comp=kv(cap=1 << 16), win=kv(cap=512),
                  ws=FAKE2, wsb=need)
        assert rc != 5, (k, L.lca_last_error())
    assert max(sizes) <= need
    assert sizes == sorted(sizes)


def test_indexer_mxfp4_validation(L):
    """Every rejection happens on the host, before anything is launched (no GPU needed)."""
    V = FAKE
    good = lca._KV(FAKE, 0, FAKE2, lca.MXFP4, 128, 0, 1024)
    q_pos = pos(100)

    def call(k=good, H=16, d=128, m=4, sdt=lca.BF16, stride=1024, q=V, s=V):
        return L.lca_indexer_score_mxfp4(q, None, k, H, d, 1, 1, q_pos, m, s, sdt, stride, None)
    assert call(q=None) == 1 and call(m=0) == 1
    assert call(k=lca._KV(FAKE, 0, FAKE2, lca.BF16, 128, 0, 1024)) == 3
    assert call(sdt=lca.FP8) == 3
    assert call(H=8) == 2 and call(d=64) == 2
    assert call(k=lca._KV(FAKE, 0, FAKE2, lca.MXFP4, 128, 64, 1024)) == 2     # MXFP4 has no rope dims
    assert call(k=lca._KV(FAKE, 0, FAKE2, lca.MXFP4, 128, 0, 10)) == 2        # vis(100) = 25 > cap
    assert call(stride=10) == 2
    assert call(k=lca._KV(FAKE, 0, 0, lca.MXFP4, 128, 0, 1024)) == 1       # scales missing
    assert call(s=FAKE + 2) == 4
    # MXFP4 storage is for indexer keys: the attention calls reject it
    comp = lca._KV(FAKE, 0, FAKE2, lca.MXFP4, 512, 0, 64)
    assert attn(L, comp=comp) == 3
    assert b"MXFP4" in L.lca_last_error()
    # the compressor writes it only without rope dims and with d_nope % 32 == 0
    assert compress(L, out=lca._KV(FAKE, FAKE2, FAKE2, lca.MXFP4, 512, 64, 64), in_dtype=lca.BF16) == 2
    assert compress(L, out=lca._KV(FAKE, 0, FAKE2, lca.MXFP4, 80, 0, 64), in_dtype=lca.BF16) == 2


def test_attn_append_validation(L):
    """The appending calls reject a missing row source, an empty window and bad row dtypes on the host."""
    def call(csa=True, x=FAKE, xdt=lca.BF16, n_win=128, eps=1e-6, xs=0):
        a = dict(q=FAKE, qdt=lca.BF16, H=64, B=1, T=1, q_pos=pos(100), comp=kv(), m=4, idx=FAKE2, k=16,
                 win=kv(cap=256), sink=None, scale=0.04, theta=0.0, out=FAKE2, odt=lca.F32, lse=None, ws=None,
                 wsb=0)
        if csa:
            return L.lca_csa_attn_append(a["q"], a["qdt"], a["H"], a["B"], a["T"], a["q_pos"], a["comp"], a["m"],
                                         a["idx"], a["k"], a["win"], n_win, x, xdt, xs, None, eps, a["sink"],
                                         a["scale"], a["theta"], a["out"], a["odt"], a["lse"], a["ws"], a["wsb"],
                                         None)
        return L.lca_hca_attn_append(a["q"], a["qdt"], a["H"], a["B"], a["T"], a["q_pos"], a["comp"], a["m"],
                                     a["win"], n_win, x, xdt, xs, None, eps, a["sink"], a["scale"], a["theta"],
                                     a["out"], a["odt"], a["lse"], a["ws"], a["wsb"], None)
    for csa in (True, False):
        assert call(csa, x=None) == 1
        assert call(csa, n_win=0) == 1
        assert call(csa, xdt=lca.FP8) == 3
        assert call(csa, eps=-1.0) == 1
        assert call(csa, x=FAKE + 4) == 4
        assert call(csa, xs=-1) == 2


def test_linear_validation(L):
    def call(x=FAKE, ldx=64, sx=0, w=FAKE2, ldw=64, sw=0, ydt=lca.F32, ldy=32, M=4, N=32, K=64, bt=1):
        return L.lca_linear(x, ldx, sx, w, ldw, sw, FAKE2, ydt, ldy, 0, M, N, K, bt, None)
    assert call(x=None) == 1
    assert call(ydt=lca.FP8) == 3
    assert call(K=60) == 2 and call(K=0) == 2 and call(N=0) == 2 and call(bt=0) == 2
    assert call(ldx=32) == 2 and call(ldy=16) == 2
    assert call(ldx=68) == 4 and call(sx=4, bt=2) == 4
    assert call(x=FAKE + 8) == 4
    assert L.lca_grouped_out_proj(FAKE, 4, 6, 64, 4, FAKE2, 64, FAKE2, 96, FAKE2, FAKE2, lca.F32, None) == 2  # H % g
    assert L.lca_grouped_out_proj(FAKE, 4, 8, 63, 4, FAKE2, 64, FAKE2, 96, FAKE2, FAKE2, lca.F32, None) == 2  # (H/g) c % 8
    # one batch entry's rows are addressed with 32-bit element offsets: 2^32 elements or more are refused
    assert call(M=1 << 20, ldx=4096, ldw=4096, K=4096) == 2          # x: (2^20 - 1) 4096 + 4096 = 2^32
    assert b"2^32" in L.lca_last_error()
    assert call(N=1 << 20, ldx=4096, ldw=4096, K=4096, ldy=1 << 20) == 2
    assert b"2^32" in L.lca_last_error()
    assert L.lca_grouped_out_proj(FAKE, 1 << 17, 64, 576, 8, FAKE2, 1024, FAKE2, 4096, FAKE2, FAKE2,
                                  lca.F32, None) == 2              # o: 2^17 tokens x 36,864


def test_cache_validation(L):
    """Plane rules of lca_cache_create, checked before the runtime is asked for anything."""
    from long_context_attention_22_amd import cache as pc
    Lc = pc._lib()

    def create(planes, max_seqs=2, page=65536, pool=4):
        arr = (pc._Plane * len(planes))(*[pc._Plane(*p) for p in planes])
        h = C.c_void_p()
        return Lc.lca_cache_create(arr, len(planes), max_seqs, page, pool, C.byref(h))

    csa = (512, 1024, 4, 0)                            # fp8 nope rows of a CSA stream
    assert create([csa], max_seqs=0) == lca.EINVAL
    assert create([csa], max_seqs=lca.MAX_BATCH + 1) == lca.EINVAL
    assert create([(512, 1024, -1, 0)]) == lca.EINVAL
    assert create([(512, 1024, 4, 1)]) == lca.EINVAL  # reserved field
    assert create([csa], page=0) == lca.ESHAPE
    assert create([(768, 1024, 4, 0)]) == lca.ESHAPE  # rows do not tile the page
    assert create([(512, 1000, 4, 0)]) == lca.ESHAPE  # a slot is not whole pages
    # a page must cover a multiple of lcm(m) raw tokens: 4096 B of 512 B rows at m = 4 is 32 tokens,
    # not a multiple of lcm(4, 128)
    assert create([csa, (512, 1024, 128, 0)], page=4096) == lca.ESHAPE
    assert b"lcm" in L.lca_last_error()
    assert create([(4, 9, 0, 0)]) == lca.ESHAPE        # state plane of 36 bytes per slot
    assert Lc.lca_cache_destroy(None) == lca.OK


def test_indexer_topk_validation(L):
    """lca_indexer_topk rejects bad arguments before launching (the two calls' rules plus its workspace)."""
    L.lca_indexer_topk.restype = C.c_int
    vp = C.c_void_p

    def call(**kw):
        a = dict(q=FAKE, w=None, k=FAKE2, k_cap=300000, H_I=16, d_I=128, B=1, T=1, q_pos=pos(1 << 20), m=4,
                 scores=FAKE, s_stride=300000, topk=2048, idx=FAKE2, ws=FAKE, ws_bytes=1 << 20)
        a.update(kw)
        return L.lca_indexer_topk(vp(a["q"]), vp(a["w"]) if a["w"] else None, vp(a["k"]), C.c_int64(a["k_cap"]),
                                  C.c_int32(a["H_I"]), C.c_int32(a["d_I"]), C.c_int32(a["B"]), C.c_int32(a["T"]),
                                  a["q_pos"],
                                  C.c_int32(a["m"]), vp(a["scores"]), C.c_int64(a["s_stride"]), C.c_int32(a["topk"]),
                                  vp(a["idx"]), vp(a["ws"]) if a["ws"] else None, C.c_size_t(a["ws_bytes"]), None)

    assert call(q=0) == lca.EINVAL
    assert call(idx=0) == lca.EINVAL
    assert call(m=0) == lca.EINVAL
    assert call(topk=0) == lca.EINVAL
    assert call(H_I=8) == lca.ESHAPE
    assert call(B=0, q_pos=pos(0)) == lca.ESHAPE
    assert call(k_cap=1000) == lca.ESHAPE            # 262,144 visible entries do not fit
    assert call(idx=FAKE2 + 4) == lca.EALIGN
    assert call(T=-1) == lca.ESHAPE
    assert call(T=40000, k_cap=262200, s_stride=262200) == lca.ESHAPE   # the last row sees past the cache
    need = L.lca_indexer_topk_workspace_size(1, 1, 300000, 2048)
    assert need > 0
    assert call(ws=0, ws_bytes=0) == lca.EWORKSPACE
    assert call(ws_bytes=need - 1) == lca.EWORKSPACE
    # short rows (the row schedule): one 256-bin histogram per row; many rows: likewise
    assert L.lca_indexer_topk_workspace_size(1, 1, 10000, 2048) == 1024
    assert L.lca_indexer_topk_workspace_size(2, 4096, 300000, 2048) == 2 * 4096 * 1024
    rows_need = L.lca_indexer_topk_workspace_size(1, 4096, 300000, 2048)
    assert call(T=4096, ws_bytes=rows_need - 1) == lca.EWORKSPACE
