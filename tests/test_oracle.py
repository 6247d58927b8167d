"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with a retyped copy of itself: every check is
a closed form, an invariant, a special case that reduces to a textbook or
library routine (numpy / torch / scipy), or a published format table.
Pages: "DeepSeek-V4 中文翻译" (cnblogs translation of the report), section 2.3;
"DeepSeek-V4：百万 token 上下文，真正可供 Agent 使用" (HF blog translation).
"""
import math
import os

import numpy as np
import pytest
import torch

import lca_synth as S

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# codecs
# --------------------------------------------------------------------------

def test_fp8_points_match_ocp_table(orc):
    for line in open(os.path.join(GOLD, "ocp_e4m3_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = orc.fp8_to_f64(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_fp8_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.fp8_to_f64(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # monotone magnitudes over codes 0..126, round trip on every finite code
    mags = got[:127]
    assert np.all(np.diff(mags) > 0)
    for c in range(256):
        if not np.isnan(got[c]):
            assert orc.f64_to_fp8(got[c]) == c


def test_fp8_encode_matches_torch_rne(orc):
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(4000) * 30, g.standard_normal(2000) * 1e-2,
                        g.uniform(-448, 448, 2000)])
    # exact midpoints between neighbouring codes exercise ties-to-even
    vals = np.array([orc.fp8_to_f64(c) for c in range(127)])
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.f64_to_fp8(v) for v in x], np.uint8)
    assert np.array_equal(got, ref)
    # saturation (the library's stated behaviour; torch gives NaN there)
    assert orc.f64_to_fp8(1e6) == 0x7E and orc.f64_to_fp8(-500.0) == 0xFE


def test_bf16_round_matches_torch(orc):
    g = np.random.default_rng(1)
    x = g.standard_normal(5000).astype(np.float32) * 100
    # exact ties: lower half exactly 0x8000
    u = g.integers(0, 2**31, 2000, dtype=np.uint32) & 0x7F7F0000 | 0x00008000
    x = np.concatenate([x, u.view(np.float32)])
    ref = S.to_bf16(x)
    got = np.array([orc.f32_to_bf16(v) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    assert orc.bf16_to_f64(0x3F80) == 1.0 and orc.bf16_to_f64(0xC000) == -2.0


# --------------------------------------------------------------------------
# compressor
# --------------------------------------------------------------------------

def _f32(*shape, seed=0, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _compress_f32(orc, ca, za, cb, zb, m, overlap, d_nope, d_rope, first_pos=0, cap=None, **kw):
    B, n, c = ca.shape
    cap = cap or (first_pos + n) // m + 1
    out = orc.KV.empty(orc.F32, B, cap, d_nope, d_rope)
    cnt = orc.kv_compress(ca, za, cb, zb, out, m=m, overlap=overlap, first_pos=[first_pos] * B, **kw)
    return out, cnt


def test_compress_m1_is_identity(orc):
    """m=1, no overlap: the softmax over a single logit is 1, whatever the gate."""
    ca, za = _f32(2, 37, 24, seed=1), _f32(2, 37, 24, seed=2, scale=50)
    out, cnt = _compress_f32(orc, ca, za, None, None, 1, 0, 16, 8,
                             bias_a=_f32(1, 24, seed=3, scale=9))
    assert cnt == 2 * 37
    assert np.array_equal(out.nope[:, :37], ca[:, :, :16])
    assert np.array_equal(out.rope[:, :37], ca[:, :, 16:])


@pytest.mark.parametrize("m,overlap", [(4, 1), (4, 0), (8, 1), (128, 0)])
def test_compress_zero_gate_is_mean_pooling(orc, m, overlap):
    n = 3 * m + 1  # ragged tail: the partial last block is not compressed
    ca, cb = _f32(1, n, 12, seed=4), _f32(1, n, 12, seed=5)
    z = np.zeros_like(ca)
    out, cnt = _compress_f32(orc, ca, z, cb, z, m, overlap, 12, 0)
    assert cnt == 3
    for s in range(3):
        blk = ca[0, s * m:(s + 1) * m].astype(np.float64)
        if overlap and s >= 1:
            blk = np.concatenate([blk, cb[0, (s - 1) * m:s * m].astype(np.float64)])
        np.testing.assert_allclose(out.nope[0, s], blk.mean(0), rtol=1e-6, atol=1e-6)


def test_compress_overlap_closed_form_m1(orc):
    ca, cb = _f32(1, 9, 8, seed=6), _f32(1, 9, 8, seed=7)
    z = np.zeros_like(ca)
    out, _ = _compress_f32(orc, ca, z, cb, z, 1, 1, 8, 0)
    np.testing.assert_array_equal(out.nope[0, 0], ca[0, 0])
    for s in range(1, 9):
        np.testing.assert_allclose(out.nope[0, s], 0.5 * (ca[0, s].astype(np.float64) + cb[0, s - 1]),
                                   rtol=1e-7)


def test_compress_constant_block_and_dominant_gate(orc):
    m = 4
    c = np.repeat(_f32(1, 1, 10, seed=8), 4 * m, axis=1)   # same value on every row
    za, zb = _f32(1, 4 * m, 10, seed=9, scale=3), _f32(1, 4 * m, 10, seed=10, scale=3)
    out, _ = _compress_f32(orc, c, za, c, zb, m, 1, 10, 0)
    np.testing.assert_allclose(out.nope[0, :4], np.broadcast_to(c[0, 0], (4, 10)), rtol=1e-6)
    # a gate far above the others picks that row's value
    ca, cb = _f32(1, 4 * m, 10, seed=11), _f32(1, 4 * m, 10, seed=12)
    za = np.zeros_like(ca)
    zb = np.zeros_like(ca)
    za[0, 2 * m + 3, :] = 200.0          # block 2, position 3 of the a-set
    zb[0, 2 * m + 1, :] = 200.0          # block 2 of the b-set feeds entry 3
    out, _ = _compress_f32(orc, ca, za, cb, zb, m, 1, 10, 0)
    np.testing.assert_allclose(out.nope[0, 2], ca[0, 2 * m + 3], rtol=1e-6)
    np.testing.assert_allclose(out.nope[0, 3], cb[0, 2 * m + 1], rtol=1e-6)


def test_compress_bias_is_per_position_and_shift_invariant(orc):
    m = 4
    ca, cb = _f32(1, 3 * m, 6, seed=13), _f32(1, 3 * m, 6, seed=14)
    z = np.zeros_like(ca)
    ba = np.zeros((m, 6), np.float32)
    ba[1, :] = 300.0                      # position 1 inside every block
    bb = np.zeros((m, 6), np.float32)
    out, _ = _compress_f32(orc, ca, z, cb, z, m, 1, 6, 0, bias_a=ba, bias_b=bb)
    for s in range(3):
        np.testing.assert_allclose(out.nope[0, s], ca[0, s * m + 1], rtol=1e-6)
    # adding one per-channel constant to every logit of an entry changes nothing
    za, zb = _f32(1, 3 * m, 6, seed=15), _f32(1, 3 * m, 6, seed=16)
    shift = _f32(1, 1, 6, seed=17, scale=7)
    o1, _ = _compress_f32(orc, ca, za, cb, zb, m, 1, 6, 0)
    o2, _ = _compress_f32(orc, ca, za + shift, cb, zb + shift, m, 1, 6, 0)
    np.testing.assert_allclose(o1.nope[0, :3], o2.nope[0, :3], rtol=1e-5, atol=1e-6)


def test_compress_entry_range_and_ring(orc):
    """Only entries whose rows are all present are produced; ring rows are s mod cap."""
    m = 4
    ca = _f32(1, 10, 4, seed=18)
    z = np.zeros_like(ca)
    # rows at positions 6..15: block 2 (8..11) needs block 1 (4..7) -> absent; block 3 ok
    out, cnt = _compress_f32(orc, ca, z, ca, z, m, 1, 4, 0, first_pos=6, cap=8)
    assert cnt == 1
    exp = np.concatenate([ca[0, 6:10], ca[0, 2:6]]).astype(np.float64).mean(0)  # block 3 + block 2
    np.testing.assert_allclose(out.nope[0, 3], exp, rtol=1e-6)
    assert not out.nope[0, 2].any()
    ring = orc.KV.empty(orc.F32, 1, 3, 4, 0)
    orc.kv_compress(ca, z, None, None, ring, m=1, overlap=0, first_pos=[6], ring=1)
    for p in range(13, 16):
        np.testing.assert_array_equal(ring.nope[0, p % 3], ca[0, p - 6])


def test_compress_rmsnorm_and_rope(orc):
    m, dn, dr = 4, 24, 8
    ca, za = _f32(1, 5 * m, dn + dr, seed=19, scale=4), _f32(1, 5 * m, dn + dr, seed=20)
    gamma = np.ones(dn + dr, np.float32)
    out, _ = _compress_f32(orc, ca, za, ca, za, m, 1, dn, dr, gamma=gamma, eps=0.0)
    y = np.concatenate([out.nope[0, :5], out.rope[0, :5]], -1).astype(np.float64)
    # RMS over all dims is 1 (RoPE preserves each pair's norm)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(-1)), 1.0, rtol=1e-6)
    g2 = np.linspace(0.5, 2.0, dn + dr).astype(np.float32)
    out2, _ = _compress_f32(orc, ca, za, ca, za, m, 1, dn, dr, gamma=g2, eps=0.0)
    np.testing.assert_allclose(out2.nope[0, :5], out.nope[0, :5] * g2[:dn], rtol=1e-6)
    # RoPE: the pair (i, i + dr/2) of entry s turns by s*m*theta^(-2i/dr); entry 0 unturned
    theta = 10000.0
    out3, _ = _compress_f32(orc, ca, za, ca, za, m, 1, dn, dr, gamma=gamma, eps=0.0, rope_theta=theta)
    np.testing.assert_array_equal(out3.nope[0, :5], out.nope[0, :5])
    np.testing.assert_allclose(out3.rope[0, 0], out.rope[0, 0], rtol=1e-6)
    for s in range(1, 5):
        for i in range(dr // 2):
            a0 = math.atan2(out.rope[0, s, i + dr // 2], out.rope[0, s, i])
            a1 = math.atan2(out3.rope[0, s, i + dr // 2], out3.rope[0, s, i])
            want = (s * m * theta ** (-2 * i / dr)) % (2 * math.pi)
            d = (a1 - a0 - want + math.pi) % (2 * math.pi) - math.pi
            assert abs(d) < 1e-5
            assert math.hypot(out3.rope[0, s, i], out3.rope[0, s, i + dr // 2]) == pytest.approx(
                math.hypot(out.rope[0, s, i], out.rope[0, s, i + dr // 2]), rel=1e-6)


def test_compress_rmsnorm_epsilon(orc):
    """epsilon joins the mean square under the root: a row of ones with eps = 3 becomes 1 / sqrt(1 + 3)
    = 0.5 in every dim, a row of twos 2 / sqrt(4 + 3); an all-zero row stays zero (no division by 0)."""
    dn = 16
    x = np.ones((1, 3, dn), np.float32)
    x[0, 1] = 2.0
    x[0, 2] = 0.0
    out = orc.KV.empty(orc.F32, 1, 3, dn, 0)
    orc.kv_compress(x, np.zeros_like(x), None, None, out, m=1, overlap=0, first_pos=[0],
                    gamma=np.ones(dn, np.float32), eps=3.0)
    np.testing.assert_array_equal(out.nope[0, 0], np.full(dn, 0.5, np.float32))
    np.testing.assert_allclose(out.nope[0, 1], 2.0 / math.sqrt(7.0), rtol=1e-7)
    np.testing.assert_array_equal(out.nope[0, 2], np.zeros(dn, np.float32))


def test_compress_store_formats(orc):
    m, dn, dr = 1, 256, 64
    x = S.block_scaled(3, "x", 0, 40, dn + dr)[None]
    x[0, 5, :128] = 0.0                         # an all-zero group: scale 1, codes 0
    z = np.zeros_like(x)
    f8 = orc.KV.empty(orc.FP8, 1, 40, dn, dr)
    orc.kv_compress(x, z, None, None, f8, m=1, overlap=0, first_pos=[0])
    bf = orc.KV.empty(orc.BF16, 1, 40, dn, dr)
    orc.kv_compress(x, z, None, None, bf, m=1, overlap=0, first_pos=[0])
    # bf16 planes are the nearest-even rounding of the fp32 inputs
    assert np.array_equal(bf.nope[0], S.to_bf16(x[0, :, :dn]))
    assert np.array_equal(f8.rope[0], S.to_bf16(x[0, :, dn:]))
    # fp8: power-of-two scales with amax/scale in (224, 448]; codes are torch's e4m3fn of x/scale
    assert f8.scale[0, 5, 0] == 1.0 and not f8.nope[0, 5, :128].any()
    for r in range(40):
        for g in range(dn // 128):
            blk = x[0, r, g * 128:(g + 1) * 128].astype(np.float64)
            a = np.abs(blk).max()
            if a == 0:
                continue
            sc = float(f8.scale[0, r, g])
            assert math.log2(sc) == int(math.log2(sc))
            assert 224 < a / sc <= 448
            ref = torch.from_numpy(blk / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(f8.nope[0, r, g * 128:(g + 1) * 128], ref)
    dec = f8.decode(0)
    assert np.all(np.abs(dec[:, :dn] - x[0, :, :dn]) <= np.abs(x[0, :, :dn]) * 2 ** -4 + 1e-30)


# --------------------------------------------------------------------------
# lightning indexer
# --------------------------------------------------------------------------

def test_indexer_single_head_is_matrix_product(orc):
    """H_I = 1, w = 1, q, k >= 0: ReLU is inactive and S = Q K^T."""
    m, T, N, d = 4, 40, 10, 16
    q = np.abs(_f32(1, T, 1, d, seed=21))
    k = np.abs(_f32(1, N, d, seed=22))
    s = orc.indexer_score(q, None, k, q_pos=[0], m=m, score_fmt=orc.F32)
    ref = (q[0, :, 0].astype(np.float64) @ k[0].astype(np.float64).T).astype(np.float32)
    for t in range(T):
        vis = (t + 1) // m
        np.testing.assert_array_equal(s[0, t, :vis], ref[t, :vis])
        assert not s[0, t, vis:].any()          # invisible columns untouched


def test_indexer_relu_weights_and_heads(orc):
    m, T, N, d, H = 1, 6, 6, 8, 3
    q, k = _f32(1, T, H, d, seed=23), _f32(1, N, d, seed=24)
    w = _f32(1, T, H, seed=25)
    s = orc.indexer_score(q, w, k, q_pos=[0], m=m, score_fmt=orc.F32).astype(np.float64)
    # per-head contributions: head h alone (w = e_h) is w_h * relu(q_h . k) via matmul
    tot = np.zeros((T, N))
    for h in range(H):
        wh = np.zeros_like(w)
        wh[0, :, h] = w[0, :, h]
        sh = orc.indexer_score(q, wh, k, q_pos=[0], m=m, score_fmt=orc.F32).astype(np.float64)
        dots = q[0, :, h].astype(np.float64) @ k[0].astype(np.float64).T
        exp = w[0, :, h:h + 1].astype(np.float64) * np.maximum(dots, 0.0)
        for t in range(T):
            np.testing.assert_allclose(sh[0, t, :t + 1], exp[t, :t + 1], rtol=1e-6, atol=1e-7)
        tot += sh[0]
    for t in range(T):
        np.testing.assert_allclose(s[0, t, :t + 1], tot[t, :t + 1], rtol=1e-5, atol=1e-6)
    s2 = orc.indexer_score(q, 2 * w, k, q_pos=[0], m=m, score_fmt=orc.F32)
    np.testing.assert_array_equal(s2, 2 * s.astype(np.float32))


def test_indexer_bf16_scores_and_positions(orc):
    m, T, N, d, H = 4, 12, 64, 16, 4
    q, k = _f32(2, T, H, d, seed=26), _f32(2, N, d, seed=27)
    w = _f32(2, T, H, seed=28)
    pos = [200, 17]
    f = orc.indexer_score(q, w, k, q_pos=pos, m=m, score_fmt=orc.F32)
    b = orc.indexer_score(q, w, k, q_pos=pos, m=m, score_fmt=orc.BF16)
    for bi in range(2):
        for t in range(T):
            vis = min(N, (pos[bi] + t + 1) // m)
            assert np.array_equal(b[bi, t, :vis], S.to_bf16(f[bi, t, :vis] + np.float32(0.0)))
            assert not np.any(b[bi, t, :vis] == 0x8000)   # no negative zero
            assert not b[bi, t, vis:].any()


# --------------------------------------------------------------------------
# top-k selector
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_topk_matches_lexsort(orc, fmt):
    m, T, N, k = 4, 50, 48, 7
    g = np.random.default_rng(30)
    raw = np.round(g.standard_normal((2, T, N)) * 4).astype(np.float32) / 4   # many ties
    sc = raw if fmt == "f32" else S.to_bf16(raw)
    val = raw if fmt == "f32" else S.from_bf16(sc)
    pos = [0, 150]
    idx = orc.topk_select(sc, q_pos=pos, m=m, k=k)
    for b in range(2):
        for t in range(T):
            vis = min(N, (pos[b] + t + 1) // m)
            K = min(k, vis)
            order = np.lexsort((np.arange(vis), -val[b, t, :vis].astype(np.float64)))
            want = np.sort(order[:K])
            assert np.array_equal(idx[b, t, :K], want)
            assert np.all(idx[b, t, K:] == -1)
            if K and vis > K:
                sel = val[b, t, idx[b, t, :K]]
                rest = np.delete(val[b, t, :vis], idx[b, t, :K])
                assert sel.min() >= rest.max()


def test_topk_negative_zero_ties_positive_zero(orc):
    sc = np.zeros((1, 1, 6), np.float32)
    sc[0, 0, [0, 2, 4]] = -0.0
    idx = orc.topk_select(sc, q_pos=[23], m=4, k=3)
    assert idx[0, 0].tolist() == [0, 1, 2]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _causal_mqa(q, kv, scale):
    """Textbook causal softmax attention, one KV head shared by all query heads."""
    T, H, c = q.shape
    lg = np.einsum("thd,sd->ths", q.astype(np.float64), kv.astype(np.float64)) * scale
    mask = np.tril(np.ones((T, T), bool))
    lg = np.where(mask[:, None, :], lg, -np.inf)
    lg -= lg.max(-1, keepdims=True)
    p = np.exp(lg)
    p /= p.sum(-1, keepdims=True)
    return np.einsum("ths,sd->thd", p, kv.astype(np.float64))


def _rows_kv(orc, x, fmt=None, m=1):
    """Store raw rows x [B][n][c] as a KV with the identity compressor (m=1)."""
    fmt = orc.F32 if fmt is None else fmt
    B, n, c = x.shape
    kv = orc.KV.empty(fmt, B, n, c - 8, 8)
    orc.kv_compress(x, np.zeros_like(x), None, None, kv, m=1, overlap=0, first_pos=[0] * B)
    return kv


def test_window_only_is_causal_mqa(orc):
    T, H, c = 20, 3, 24
    x, q = _f32(1, T, c, seed=31), _f32(1, T, H, c, seed=32)
    win = _rows_kv(orc, x)
    comp = orc.KV.empty(orc.F32, 1, 1, c - 8, 8)   # m larger than the sequence: nothing visible
    o, _ = orc.attention(q, q_pos=[0], comp=comp, m=64, idx=None, win=win, n_win=T, sm_scale=0.3)
    np.testing.assert_allclose(o[0], _causal_mqa(q[0], x[0], 0.3), rtol=1e-5, atol=1e-6)


def test_identity_compressor_full_topk_is_causal_mqa(orc):
    T, H, c = 18, 2, 24
    x, q = _f32(1, T, c, seed=33), _f32(1, T, H, c, seed=34)
    comp = _rows_kv(orc, x)
    sc = orc.indexer_score(_f32(1, T, 1, 4, seed=35), None, _f32(1, T, 4, seed=36), q_pos=[0], m=1,
                           score_fmt=orc.F32)
    idx = orc.topk_select(sc, q_pos=[0], m=1, k=T + 3)
    ref = _causal_mqa(q[0], x[0], 0.25)
    o, _ = orc.attention(q, q_pos=[0], comp=comp, m=1, idx=idx, sm_scale=0.25)
    np.testing.assert_allclose(o[0], ref, rtol=1e-5, atol=1e-6)
    # and with the whole-sequence window as well: every key twice, same softmax
    o2, _ = orc.attention(q, q_pos=[0], comp=comp, m=1, idx=idx, win=comp, n_win=T, sm_scale=0.25)
    np.testing.assert_allclose(o2[0], ref, rtol=1e-5, atol=1e-6)
    # CSA with k >= vis equals HCA over the same cache
    o3, _ = orc.attention(q, q_pos=[0], comp=comp, m=1, idx=None, sm_scale=0.25)
    np.testing.assert_allclose(o3, o, rtol=1e-6, atol=1e-7)


def test_sink_single_key_and_lse(orc):
    c = 16
    x = _f32(1, 1, c, seed=37)
    kv = _rows_kv(orc, x)
    q = _f32(1, 1, 2, c, seed=38)
    sink = np.array([0.7, -1e30], np.float32)
    o, lse = orc.attention(q, q_pos=[0], comp=kv, m=1, idx=None, sink=sink, sm_scale=0.5)
    l = 0.5 * (q[0, 0].astype(np.float64) @ x[0, 0].astype(np.float64))
    # one key plus a sink: o = v * sigmoid(l - z); without a sink o = v
    sig = 1.0 / (1.0 + np.exp(sink[0] - l[0]))
    np.testing.assert_allclose(o[0, 0, 0], x[0, 0] * sig, rtol=1e-6)
    np.testing.assert_allclose(o[0, 0, 1], x[0, 0], rtol=1e-6)
    np.testing.assert_allclose(lse[0, 0, 0], np.logaddexp(l[0], sink[0]), rtol=1e-6)
    np.testing.assert_allclose(lse[0, 0, 1], l[1], rtol=1e-6)


def test_invisible_and_future_rows_never_read(orc):
    """NaN in entries beyond vis(t), in unselected entries and in future window rows changes nothing."""
    m, T, H, c, n_win = 4, 16, 2, 24, 5
    q = _f32(1, T, H, c, seed=39)
    ent = _rows_kv(orc, _f32(1, 8, c, seed=40))
    win = _rows_kv(orc, _f32(1, T, c, seed=41))
    idx = np.full((1, T, 2), -1, np.int32)
    for t in range(T):
        vis = (t + 1) // m
        if vis:
            idx[0, t, 0] = vis - 1
    o_h, _ = orc.attention(q, q_pos=[0], comp=ent, m=m, win=win, n_win=n_win, sm_scale=0.2)
    o_c, _ = orc.attention(q, q_pos=[0], comp=ent, m=m, idx=idx, win=win, n_win=n_win, sm_scale=0.2)
    for t in range(T):
        vis = (t + 1) // m
        e2, w2 = orc.KV(ent.nope.copy(), ent.rope.copy(), None, ent.fmt, ent.d_nope, ent.d_rope, ent.cap), \
            orc.KV(win.nope.copy(), win.rope.copy(), None, win.fmt, win.d_nope, win.d_rope, win.cap)
        e2.nope[0, vis:] = np.nan
        w2.nope[0, t + 1:] = np.nan
        w2.nope[0, :max(0, t - n_win + 1)] = np.nan
        qt = q[:, t:t + 1]
        a, _ = orc.attention(qt, q_pos=[t], comp=e2, m=m, win=w2, n_win=n_win, sm_scale=0.2)
        np.testing.assert_array_equal(a[0, 0], o_h[0, t])
        e3 = orc.KV(e2.nope.copy(), e2.rope.copy(), None, ent.fmt, ent.d_nope, ent.d_rope, ent.cap)
        e3.nope[0, :max(0, vis - 1)] = np.nan      # unselected entries
        b_, _ = orc.attention(qt, q_pos=[t], comp=e3, m=m, idx=idx[:, t:t + 1], win=w2, n_win=n_win,
                              sm_scale=0.2)
        np.testing.assert_array_equal(b_[0, 0], o_c[0, t])


def _windowed_mqa(q, kv, scale, n_win):
    """Textbook sliding-window softmax attention: query t attends keys p in [t - n_win + 1, t]."""
    T, H, c = q.shape
    lg = np.einsum("thd,sd->ths", q.astype(np.float64), kv.astype(np.float64)) * scale
    t, p = np.arange(T)[:, None], np.arange(T)[None, :]
    mask = (p <= t) & (p > t - n_win)
    lg = np.where(mask[:, None, :], lg, -np.inf)
    lg -= lg.max(-1, keepdims=True)
    w = np.exp(lg)
    w /= w.sum(-1, keepdims=True)
    return np.einsum("ths,sd->thd", w, kv.astype(np.float64))


def test_window_ring_wrap_is_sliding_window_mqa(orc):
    """A window ring smaller than the sequence (cap 7 < T = 30), written by the compressor's ring rule
    (row p mod cap) one chunk at a time, read at row p mod cap: each query's output equals the textbook
    sliding-window attention over the raw rows."""
    T, H, c, n_win, cap = 30, 2, 24, 5, 7
    x, q = _f32(1, T, c, seed=84), _f32(1, T, H, c, seed=85)
    ref = _windowed_mqa(q[0], x[0], 0.3, n_win)
    ring = orc.KV.empty(orc.F32, 1, cap, c - 8, 8)
    comp = orc.KV.empty(orc.F32, 1, 1, c - 8, 8)   # m larger than the sequence: nothing visible
    z = np.zeros_like(x)
    for t in range(T):                              # store row t, then attend from t (decode order)
        orc.kv_compress(x[:, t:t + 1], z[:, t:t + 1], None, None, ring, m=1, overlap=0, first_pos=[t], ring=1)
        o, _ = orc.attention(q[:, t:t + 1], q_pos=[t], comp=comp, m=64, idx=None, win=ring, n_win=n_win,
                             sm_scale=0.3)
        np.testing.assert_allclose(o[0, 0], ref[t], rtol=1e-5, atol=1e-6)


def test_csa_listed_future_entries_not_attended(orc):
    """Block-level causality holds at the attention step: an index list naming every entry, future ones
    included (their rows NaN), and ids past the cache still gives textbook causal attention
    (identity compressor, m = 1)."""
    T, H, c = 14, 2, 24
    x, q = _f32(1, T, c, seed=86), _f32(1, T, H, c, seed=87)
    comp = _rows_kv(orc, x)
    ref = _causal_mqa(q[0], x[0], 0.25)
    idx = np.tile(np.arange(T + 2, dtype=np.int32), (1, T, 1))   # ids T, T + 1 lie past the cache
    for t in range(T):
        poisoned = orc.KV(comp.nope.copy(), comp.rope.copy(), None, comp.fmt, comp.d_nope, comp.d_rope, comp.cap)
        poisoned.nope[0, t + 1:] = np.nan
        o, _ = orc.attention(q[:, t:t + 1], q_pos=[t], comp=poisoned, m=1, idx=idx[:, t:t + 1], sm_scale=0.25)
        np.testing.assert_allclose(o[0, 0], ref[t], rtol=1e-5, atol=1e-6)


def test_output_rope_makes_position_relative(orc):
    """One visible entry at position p and rotation by -t: the output's RoPE pair is turned by p - t."""
    c, dr, theta, m = 24, 8, 10000.0, 4
    x = _f32(1, 2 * m, c, seed=42)
    kv = orc.KV.empty(orc.F32, 1, 2, c - dr, dr)
    z = np.zeros_like(x)
    orc.kv_compress(x, z, None, None, kv, m=m, overlap=0, first_pos=[0], rope_theta=theta)
    kv0 = orc.KV.empty(orc.F32, 1, 2, c - dr, dr)
    orc.kv_compress(x, z, None, None, kv0, m=m, overlap=0, first_pos=[0])
    q = _f32(1, 1, 1, c, seed=43)
    for t in (4, 7):   # only entry 0 (position 0) visible; the pair turns by 0 - t
        idx = np.array([[[0]]], np.int32)
        o, _ = orc.attention(q, q_pos=[t], comp=kv, m=m, idx=idx, sm_scale=0.1, rope_theta=theta)
        v = kv0.decode(0, 0, 1)[0]
        for i in range(dr // 2):
            ang = -t * theta ** (-2 * i / dr)
            a, b = v[c - dr + i], v[c - dr + dr // 2 + i]
            np.testing.assert_allclose(o[0, 0, 0, c - dr + i], a * math.cos(ang) - b * math.sin(ang),
                                       rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(o[0, 0, 0, c - dr + dr // 2 + i],
                                       a * math.sin(ang) + b * math.cos(ang), rtol=1e-5, atol=1e-6)
    # entry 1 at position 4, query t = 7 -> relative turn 4 - 7 applied to the unrotated vector
    o, _ = orc.attention(q, q_pos=[7], comp=kv, m=m, idx=np.array([[[1]]], np.int32), sm_scale=0.1,
                         rope_theta=theta)
    v = kv0.decode(0, 1, 1)[0]
    for i in range(dr // 2):
        ang = (4 - 7) * theta ** (-2 * i / dr)
        a, b = v[c - dr + i], v[c - dr + dr // 2 + i]
        np.testing.assert_allclose(o[0, 0, 0, c - dr + i], a * math.cos(ang) - b * math.sin(ang),
                                   rtol=1e-5, atol=1e-6)


def test_fp8_cache_reads_decoded_values(orc):
    """Attention over an fp8 cache equals attention over the same decoded values held in f32."""
    T, H, dn, dr = 6, 2, 128, 8
    x = S.block_scaled(44, "kv", 0, T, dn + dr)[None]
    f8 = orc.KV.empty(orc.FP8, 1, T, dn, dr)
    orc.kv_compress(x, np.zeros_like(x), None, None, f8, m=1, overlap=0, first_pos=[0])
    dec = f8.decode(0).astype(np.float32)[None]
    f32 = orc.KV.empty(orc.F32, 1, T, dn, dr)
    orc.kv_compress(dec, np.zeros_like(dec), None, None, f32, m=1, overlap=0, first_pos=[0])
    q = _f32(1, T, H, dn + dr, seed=45)
    a, la = orc.attention(q, q_pos=[0], comp=f8, m=1, sm_scale=0.05)
    b, lb = orc.attention(q, q_pos=[0], comp=f32, m=1, sm_scale=0.05)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# --------------------------------------------------------------------------
# MXFP4 QK path ("DeepSeek-V4 中文翻译" section 5.2.1: the indexer's QK
# activations are cached, loaded and multiplied in FP4 (MXFP4))
# --------------------------------------------------------------------------

def _e2m1_grid():
    """The 16 E2M1 values built from the format's fields (bias 1, 1 mantissa bit, subnormals)."""
    out = []
    for code in range(16):
        s, e, mt = code >> 3, (code >> 1) & 3, code & 1
        v = mt * 0.5 if e == 0 else (1 + mt / 2) * 2.0 ** (e - 1)
        out.append(-v if s else v)
    return np.array(out)


def test_e2m1_decode_matches_ocp_table(orc):
    rows = [l.split() for l in open(os.path.join(GOLD, "ocp_e2m1_values.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) == 16
    grid = _e2m1_grid()
    for code, val in rows:
        got = orc.e2m1_to_f64(int(code, 16))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
        assert got == grid[int(code, 16)] and math.copysign(1, got) == math.copysign(1, grid[int(code, 16)])


def test_e2m1_encode_is_nearest_ties_even_saturating(orc):
    """Brute force over the 16 codes: nearest value, exact ties to the code with mantissa bit 0."""
    grid = _e2m1_grid()
    g = np.random.default_rng(71)
    mids = (grid[:7] + grid[1:8]) / 2
    x = np.concatenate([g.uniform(-7, 7, 3000), g.standard_normal(500) * 0.3, mids, -mids,
                        grid[:8], -grid[:8], [6.5, 100.0, -1e9, 5.999, 0.2500001, 0.2499999]])
    for v in x:
        c = orc.f64_to_e2m1(v)
        mag = min(abs(v), 6.0)
        d = np.abs(grid[:8] - mag)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c & 7 == want, (v, c)
        assert (c >> 3) == (1 if math.copysign(1, v) < 0 else 0)


def test_mxfp4_block_scale_rule_and_codes(orc):
    """Scale 2^(floor(log2 amax) - 2) puts amax/X in [4, 8); codes are nearest of v/X (brute force)."""
    grid = _e2m1_grid()
    g = np.random.default_rng(72)
    for trial in range(300):
        sc = 2.0 ** g.integers(-30, 30)
        v = g.standard_normal(32) * sc
        if trial % 7 == 0:
            v[g.integers(0, 32)] = 2.0 ** g.integers(-20, 20)    # amax exactly a power of two
        e, codes = orc.mxfp4_block(v)
        X = 2.0 ** (e - 127)
        amax = np.abs(v).max()
        assert 4 <= amax / X < 8
        for j in range(32):
            mag = min(abs(v[j]) / X, 6.0)
            d = np.abs(grid[:8] - mag)
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert codes[j] & 7 == want
    # an all-zero block: scale byte 127 (2^0), zero codes
    e, codes = orc.mxfp4_block(np.zeros(32))
    assert e == 127 and not codes.any()
    # values in [6, 8) x X saturate to +-6 X
    v = np.zeros(32)
    v[0], v[1] = 7.5, -7.0
    e, codes = orc.mxfp4_block(v)
    assert e == 127 and codes[0] == 7 and codes[1] == 15


def test_mxfp4_block_roundtrip_exact_on_grid(orc):
    """A block of E2M1 grid values times a common power of two is stored exactly."""
    grid = _e2m1_grid()
    g = np.random.default_rng(73)
    for _ in range(200):
        k = int(g.integers(-40, 40))
        v = grid[g.integers(0, 16, 32)] * 2.0 ** k
        if not np.any(v):
            continue
        e, codes = orc.mxfp4_block(v)
        dec = np.array([orc.e2m1_to_f64(c) for c in codes]) * 2.0 ** (e - 127)
        np.testing.assert_array_equal(np.abs(dec), np.abs(v))


def test_compress_mxfp4_store_is_nearest_grid(orc):
    """MXFP4 rows of the compressor: per 32-block, the decoded value is the nearest point of the
    block's grid X * E2M1 to the fp32 row (ties excepted), X from the block's amax."""
    dn, N = 128, 48
    x = S.block_scaled(74, "kv", 0, N, dn)[None]
    x[0, 3, 32:64] = 0.0
    z = np.zeros_like(x)
    f4 = orc.KV.empty(orc.MXFP4, 1, N, dn, 0)
    orc.kv_compress(x, z, None, None, f4, m=1, overlap=0, first_pos=[0])
    assert f4.scale[0, 3, 1] == 127 and not f4.nope[0, 3, 16:32].any()
    dec = f4.decode(0)
    grid = _e2m1_grid()
    for r in range(N):
        for blk in range(dn // 32):
            v = x[0, r, 32 * blk:32 * blk + 32].astype(np.float64)
            a = np.abs(v).max()
            if a == 0:
                continue
            X = 2.0 ** (math.floor(math.log2(a)) - 2)
            assert f4.scale[0, r, blk] == 127 + round(math.log2(X))
            cand = np.sign(v)[:, None] * grid[None, :8] * X
            dist = np.abs(cand - v[:, None])
            got = dec[r, 32 * blk:32 * blk + 32]
            assert np.all(np.abs(got - v) <= dist.min(1) * (1 + 1e-12) + 1e-300)
    # byte packing: even element in the low nibble
    e0 = orc.e2m1_to_f64(f4.nope[0, 0, 0] & 15) * 2.0 ** (int(f4.scale[0, 0, 0]) - 127)
    e1 = orc.e2m1_to_f64(f4.nope[0, 0, 0] >> 4) * 2.0 ** (int(f4.scale[0, 0, 0]) - 127)
    assert dec[0, 0] == e0 and dec[0, 1] == e1


def _mxfp4_keys(orc, k):
    """[B][N][d] f32 keys stored MXFP4 through the compressor at m = 1."""
    B, N, d = k.shape
    kv = orc.KV.empty(orc.MXFP4, B, N, d, 0)
    orc.kv_compress(k, np.zeros_like(k), None, None, kv, m=1, overlap=0, first_pos=[0] * B)
    return kv


def test_indexer_mxfp4_on_grid_is_matrix_formula(orc):
    """q and keys already on MXFP4 grids: the scores are the plain formula (numpy, fp64)."""
    grid = _e2m1_grid()
    g = np.random.default_rng(75)
    B, T, H, d, m, N = 2, 9, 3, 64, 2, 12
    eq = 2.0 ** g.integers(-3, 3, (B, T, H, d // 32))
    q = (grid[g.integers(0, 16, (B, T, H, d))] * eq.repeat(32, -1)).astype(np.float32)
    q[..., ::32] = 6.0 * eq                      # every block reaches its grid's top value
    ek = 2.0 ** g.integers(-4, 4, (B, N, d // 32))
    k = (grid[g.integers(0, 16, (B, N, d))] * ek.repeat(32, -1)).astype(np.float32)
    k[..., ::32] = -4.0 * ek
    w = _f32(B, T, H, seed=76)
    kv = _mxfp4_keys(orc, k)
    np.testing.assert_array_equal(kv.decode(0), k[0])
    pos = [5, 20]
    s = orc.indexer_score_mxfp4(q, w, kv, q_pos=pos, m=m, score_fmt=orc.F32)
    for b in range(B):
        dots = np.einsum("thd,nd->thn", q[b].astype(np.float64), k[b].astype(np.float64))
        ref = np.einsum("th,thn->tn", w[b].astype(np.float64), np.maximum(dots, 0.0)).astype(np.float32)
        for t in range(T):
            vis = min(N, (pos[b] + t + 1) // m)
            np.testing.assert_array_equal(s[b, t, :vis], ref[t, :vis] + np.float32(0))
            assert not s[b, t, vis:].any()


def test_indexer_mxfp4_quantises_q_per_head_block(orc):
    """General bf16 q: the scores equal the formula on q quantised block by block (each block's
    quantisation pinned above) and the stored keys; bf16 scores are RNE of the f32 ones."""
    B, T, H, d, m, N = 1, 7, 4, 128, 1, 7
    q = S.to_bf16(_f32(B, T, H, d, seed=77) * 3)
    k = _f32(B, N, d, seed=78)
    w = _f32(B, T, H, seed=79)
    kv = _mxfp4_keys(orc, k)
    qf = np.array([orc.bf16_to_f64(h) for h in q.reshape(-1)]).reshape(q.shape)
    codes, scales = orc.mxfp4_quantize(qf)
    grid = _e2m1_grid()
    qd = grid[codes] * (2.0 ** (scales.astype(np.float64) - 127)).repeat(32, -1)
    kd = kv.decode(0)
    s = orc.indexer_score_mxfp4(q, w, kv, q_pos=[0], m=m, score_fmt=orc.F32)
    sb = orc.indexer_score_mxfp4(q, w, kv, q_pos=[0], m=m, score_fmt=orc.BF16)
    dots = np.einsum("thd,nd->thn", qd[0], kd)
    ref = np.einsum("th,thn->tn", w[0].astype(np.float64), np.maximum(dots, 0.0))
    for t in range(T):
        np.testing.assert_allclose(s[0, t, :t + 1], ref[t, :t + 1], rtol=1e-6, atol=1e-6)
        assert np.array_equal(sb[0, t, :t + 1], S.to_bf16(s[0, t, :t + 1] + np.float32(0)))
    # and the MXFP4 scores track the full-precision scores of the same inputs
    k2 = _f32(1, 512, d, seed=80)
    e = orc.indexer_score(q, w, S.to_bf16(k2), q_pos=[600], m=m, score_fmt=orc.F32)
    f = orc.indexer_score_mxfp4(q, w, _mxfp4_keys(orc, k2), q_pos=[600], m=m, score_fmt=orc.F32)
    for t in range(T):
        assert np.corrcoef(e[0, t], f[0, t])[0, 1] > 0.95


# --------------------------------------------------------------------------
# linear maps around the path ("DeepSeek-V4 中文翻译" section 2.3.1: projections of
# the hidden state; grouped output projection)
# --------------------------------------------------------------------------

def test_linear_small_integers_brute_force(orc):
    """Small-integer inputs: every product and sum is exact; checked against Python integer loops."""
    g = np.random.default_rng(81)
    bt, M, N, K = 2, 5, 7, 9
    x = g.integers(-8, 9, (bt, M, K)).astype(np.float32)
    w = g.integers(-8, 9, (bt, N, K))
    y = orc.linear(x, S.to_bf16(w.astype(np.float32)))
    for b in range(bt):
        for m in range(M):
            for n in range(N):
                assert y[b, m, n] == sum(int(x[b, m, k]) * int(w[b, n, k]) for k in range(K))


def test_linear_identity_permutation_and_strides(orc):
    g = np.random.default_rng(82)
    x = S.to_bf16(g.standard_normal((6, 16)).astype(np.float32))
    eye = S.to_bf16(np.eye(16, dtype=np.float32))
    np.testing.assert_array_equal(orc.linear(x, eye), S.from_bf16(x))          # W = I: Y = X exactly
    perm = g.permutation(16)
    pw = S.to_bf16(np.eye(16, dtype=np.float32)[perm])                          # row n picks column perm[n]
    np.testing.assert_array_equal(orc.linear(x, pw), S.from_bf16(x)[:, perm])
    # bf16 output = nearest-even rounding of the f32 result
    w = S.to_bf16(g.standard_normal((5, 16)).astype(np.float32))
    np.testing.assert_array_equal(orc.linear(x, w, y_fmt=orc.BF16), S.to_bf16(orc.linear(x, w) + np.float32(0)))


def test_grouped_out_proj_is_block_diagonal_then_dense(orc):
    """g groups projected separately then concatenated equals one map with the block-diagonal weight,
    and g = 1 is two plain maps (numpy fp64 on the same rounded intermediate)."""
    g_ = np.random.default_rng(83)
    T, H, c, g, d_g, d = 3, 8, 12, 4, 5, 7
    o = g_.standard_normal((T, H, c)).astype(np.float32)
    wg = S.to_bf16(g_.standard_normal((g, d_g, H // g * c)).astype(np.float32))
    wo = S.to_bf16(g_.standard_normal((d, g * d_g)).astype(np.float32))
    for mid_fmt in (orc.F32, orc.BF16):
        out = orc.grouped_out_proj(o, wg, wo, g=g, mid_fmt=mid_fmt)
        blk = np.zeros((g * d_g, H * c))
        for j in range(g):
            blk[j * d_g:(j + 1) * d_g, j * (H // g) * c:(j + 1) * (H // g) * c] = S.from_bf16(wg[j])
        mid = o.reshape(T, H * c).astype(np.float64) @ blk.T
        mid = mid.astype(np.float32) if mid_fmt == orc.F32 else S.from_bf16(S.to_bf16(mid.astype(np.float32)))
        ref = (mid.astype(np.float64) @ S.from_bf16(wo).astype(np.float64).T).astype(np.float32)
        np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)
