// attn.hip -- core attention of the DeepSeek-V4 hybrid attention
// ("DeepSeek-V4 中文翻译" sections 2.3.1 - 2.3.3): shared-KV MQA (each stored
// row is both key and value, one KV head for every query head) over
//   CSA: the top-k selected compressed entries, or
//   HCA: every visible compressed entry,
// plus the sliding window of raw rows, with a per-head sink logit and RoPE
// applied to the output by -t.
//
// bf16 / fp8 caches, c = 512 + 64, H a multiple of 16 (up to 64): MFMA path.
//   One workgroup (4 waves) per (query row, key split).  The attended rows are
//   a list of "slots": compressed slots (idx entries, or 0..vis-1) followed by
//   window slots.  Per tile of 32 slots the workgroup gathers the rows from HBM
//   (fp8 codes are expanded to bf16 exactly: the scale is a power of two) into
//   one row-major LDS tile.  It serves both operands: the K operand of Q.K^T
//   (16 contiguous bytes of one key per lane, ds_read_b128) and the V operand
//   of P.V (8 consecutive keys of one dim per lane) through gfx950's
//   transposing LDS read ds_read_b64_tr_b16: within each 16-lane group, lane i
//   receives element i mod 4 of the 8-byte rows addressed by lanes i/4 + 4e,
//   so lanes addressing (key r/4, dims 4(r mod 4)..+3) hand lane i four
//   consecutive keys of dim i.  The next tile's rows are fetched into
//   registers while the current tile is computed.  Wave w owns heads [16w, 16w+16): S = Q K^T with
//   v_mfma_f32_16x16x32_bf16 (M = heads, N = keys, K = 576 in 18 steps, Q kept
//   in registers), online softmax in the accumulator layout (row max / sum over
//   16 lanes), P goes through a small per-wave LDS buffer into A-operand
//   layout as a bf16 hi + lo pair, O += P V (N = 576 dims in 36 blocks, O
//   kept in registers).
//   Decode-sized launches split the slot list across workgroups; a second
//   kernel merges the partial (O, max, sum) triples in a fixed order.
// f32 caches: one wave per (query row, head), f32 FMA, for fp32 workloads.
#include "device.h"
#include "kernels.h"

namespace lca {

constexpr int kDN = 512, kDR = 64, kC = 576;
constexpr int kKT = 32;             // slots per tile
constexpr int kKS = kC + 8;         // row stride of the row-major tile (bf16 elements)
constexpr int kVS = kKT + 8;        // row stride of the per-wave P tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SlotMap {
    int64_t ncs;    // compressed slots
    int64_t w_lo;   // first window position
    int64_t nslots;
};

__device__ __forceinline__ SlotMap slot_map(const AttnArgs& a, int64_t t) {
    SlotMap s;
    const int64_t vis = min((t + 1) / a.m, a.comp.cap);
    s.ncs = a.idx ? (int64_t)a.k : vis;
    s.w_lo = t - a.n_win + 1 < 0 ? 0 : t - a.n_win + 1;
    const int64_t nw = a.n_win > 0 ? t - s.w_lo + 1 : 0;
    s.nslots = s.ncs + nw;
    return s;
}

// source row of a slot: 0 = invalid, 1 = compressed row, 2 = window row
__device__ __forceinline__ int slot_row(const AttnArgs& a, const SlotMap& sm, int64_t rowid, int b,
                                        int64_t slot, int64_t s_end, int64_t* row) {
    if (slot >= s_end) return 0;
    if (slot < sm.ncs) {
        int64_t e = a.idx ? (int64_t)a.idx[rowid * a.k + slot] : slot;
        if (e < 0 || e >= a.comp.cap) return 0;
        *row = (int64_t)b * a.comp.cap + e;
        return 1;
    }
    const int64_t p = sm.w_lo + (slot - sm.ncs);
    *row = (int64_t)b * a.win.cap + p % a.win.cap;
    return 2;
}

// The gathered tile's 16-byte chunks held by one thread: thread (slot j = tid % 32, chunk group
// cg = tid / 32 in [0, 16)).  fp8 rows: nope chunks of 16 codes cg and cg + 16, plus RoPE chunk cg
// (8 bf16) when cg < 8; bf16 rows: nope chunks of 8 dims cg + 16u (u < 4), plus RoPE chunk cg.
template <int FMT>
struct Gather {
    static constexpr int kN = FMT == LCA_FP8 ? 2 : 4;  // nope chunks per thread
    u32x4 v[kN + 1];
    float sc[FMT == LCA_FP8 ? 2 : 1];
    int src;

    __device__ __forceinline__ void load(const AttnArgs& a, const SlotMap& sm, int64_t rowid, int b,
                                         int64_t slot, int64_t s_end, int cg) {
        int64_t row = 0;
        src = slot_row(a, sm, rowid, b, slot, s_end, &row);
        const lca_kv& kv = src == 2 ? a.win : a.comp;
#pragma unroll
        for (int u = 0; u <= kN; ++u) v[u] = u32x4{0u, 0u, 0u, 0u};
        if (!src) return;
        if constexpr (FMT == LCA_FP8) {
            const u32x4* np = (const u32x4*)((const uint8_t*)kv.nope + row * kDN);
            v[0] = np[cg];
            v[1] = np[cg + 16];
            // 16-code chunk c covers dims 16c .. 16c+15: scale group c / 8
            sc[0] = kv.scale[row * 4 + (cg >> 3)];
            sc[1] = kv.scale[row * 4 + 2 + (cg >> 3)];
        } else {
            const u32x4* np = (const u32x4*)((const uint16_t*)kv.nope + row * kDN);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = np[cg + 16 * u];
        }
        if (cg < 8) v[kN] = ((const u32x4*)((const uint16_t*)kv.rope + row * kDR))[cg];
    }
};

__device__ __forceinline__ void put8(uint16_t* Kt, int j, int d0, u32x4 v) {
    *(u32x4*)(Kt + j * kKS + d0) = v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// transposing LDS read (see the header comment)
__device__ __forceinline__ s16x4 lds_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)p);
}

// two fp8 codes (low 16 bits when !high_half) -> packed bf16 bits of code * scale.  The hardware
// conversion decodes OCP e4m3fn exactly; the power-of-two scale keeps the product exact and a
// 4-significant-bit value loses nothing when the low 16 bits are dropped.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t codes, float sc) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, kHigh);
    const uint32_t lo = __float_as_uint(v[0] * sc), hi = __float_as_uint(v[1] * sc);
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

template <int FMT>
__device__ __forceinline__ void store_tile(const Gather<FMT>& g, uint16_t* Kt, int j, int cg) {
    if constexpr (FMT == LCA_FP8) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int d0 = 16 * (cg + 16 * u);
            u32x4 lo, hi;
            lo[0] = fp8x2_bf16<false>(g.v[u][0], g.sc[u]);
            lo[1] = fp8x2_bf16<true>(g.v[u][0], g.sc[u]);
            lo[2] = fp8x2_bf16<false>(g.v[u][1], g.sc[u]);
            lo[3] = fp8x2_bf16<true>(g.v[u][1], g.sc[u]);
            hi[0] = fp8x2_bf16<false>(g.v[u][2], g.sc[u]);
            hi[1] = fp8x2_bf16<true>(g.v[u][2], g.sc[u]);
            hi[2] = fp8x2_bf16<false>(g.v[u][3], g.sc[u]);
            hi[3] = fp8x2_bf16<true>(g.v[u][3], g.sc[u]);
            if (!g.src) lo = hi = u32x4{0u, 0u, 0u, 0u};
            put8(Kt, j, d0, lo);
            put8(Kt, j, d0 + 8, hi);
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) put8(Kt, j, 8 * (cg + 16 * u), g.v[u]);
    }
    if (cg < 8) put8(Kt, j, kDN + 8 * cg, g.v[Gather<FMT>::kN]);
}

// Eight waves: wave w owns heads [16 (w % 4), +16) and output dims [288 (w / 4), +288).
// Q.K^T: each wave of a pair contracts its 288 dims (9 MFMA k-steps per 16-slot block); the two
// partial score tiles are exchanged through LDS and summed in the same order by both waves, so
// both hold identical scores and run the identical online softmax.  P.V fills the wave's half
// of O (18 column blocks).  Per wave: Q fragments 36 VGPRs, O 72 VGPRs -> two waves per SIMD.
constexpr int kHalf = kC / 2;  // 288
template <int FMT>
__global__ void __launch_bounds__(512) attn_mfma(AttnArgs a, int64_t split_len, int nsplit) {
    __shared__ __attribute__((aligned(16))) uint16_t Kt[kKT * kKS];
    __shared__ __attribute__((aligned(16))) f32x4 Sx[8][2][64];           // partial scores
    __shared__ __attribute__((aligned(16))) uint16_t Ps[8][32 * kVS];     // P hi / lo, per wave
    __shared__ int valid[kKT];

    const int64_t rowid = blockIdx.x;
    const int split = blockIdx.y;
    const int b = (int)(rowid / a.T);
    const int64_t t = a.q_pos.v[b] + rowid % a.T;
    const SlotMap sm = slot_map(a, t);
    const int64_t s_begin = (int64_t)split * split_len;
    const int64_t s_end = min(sm.nslots, s_begin + split_len);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int hrow = lane & 15, kgrp = lane >> 4;
    const int hg = wv & 3, dh = wv >> 2;      // head group, dim half
    const int h0 = 16 * hg, dbase = kHalf * dh;

    // Q fragments of this wave: A[row = head h0 + hrow][k = dbase + 32 ks + 8 kgrp + e]
    bf16x8 qf[9];
    {
        const bool hv = h0 + hrow < a.H;
        const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + (rowid * a.H + h0 + hrow) * kC + dbase);
#pragma unroll
        for (int ks = 0; ks < 9; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, hv ? qp[4 * ks + kgrp] : u32x4{0u, 0u, 0u, 0u});
    }
    f32x4 o[18];
#pragma unroll
    for (int nb = 0; nb < 18; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun[4], lrun[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mrun[r] = -INFINITY;
        lrun[r] = 0.0f;
    }
    const float qk_scale = a.sm_scale * kLog2e;

    const int gj = tid & 31, gcg = tid >> 5;  // gather role: slot gj, chunk group gcg (0..15)
    Gather<FMT> g;
    if (s_begin < s_end) g.load(a, sm, rowid, b, s_begin + gj, s_end, gcg);

    uint16_t* pw = Ps[wv];
    const uint16_t* kr0 = Kt + hrow * kKS + dbase + 8 * kgrp;
    const uint16_t* kr1 = Kt + (16 + hrow) * kKS + dbase + 8 * kgrp;
    const uint16_t* vr = Kt + (8 * kgrp + (hrow >> 2)) * kKS + dbase + 4 * (hrow & 3);

    for (int64_t s0 = s_begin; s0 < s_end; s0 += kKT) {
        __syncthreads();  // previous tile fully consumed
        store_tile<FMT>(g, Kt, gj, gcg);
        if (gcg == 0) valid[gj] = g.src != 0;
        __syncthreads();
        if (s0 + kKT < s_end) g.load(a, sm, rowid, b, s0 + kKT + gj, s_end, gcg);

        // partial S over this wave's 288 dims, two 16-slot blocks
        f32x4 s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int ks = 0; ks < 9; ++ks) {
            const bf16x8 k0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr0 + 32 * ks));
            const bf16x8 k1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr1 + 32 * ks));
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], k0, s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], k1, s[1], 0, 0, 0);
        }
        Sx[wv][0][lane] = s[0];
        Sx[wv][1][lane] = s[1];
        __syncthreads();
        {
            const int pv = wv ^ 4;  // the partner wave (same heads, other dim half)
            const f32x4 o0 = Sx[pv][0][lane], o1 = Sx[pv][1][lane];
            // dim half 0 + dim half 1 in both waves (the same additions, the same results)
            s[0] = dh == 0 ? s[0] + o0 : o0 + s[0];
            s[1] = dh == 0 ? s[1] + o1 : o1 + s[1];
        }

        // online softmax; lane holds rows (heads) 4 kgrp + r, columns (slots) hrow and 16 + hrow.
        // The reference max moves only when a row's max exceeds it by more than 2^8 (weights stay
        // <= 256), so O is rescaled on few tiles instead of every tile.
        const bool v0 = valid[hrow], v1 = valid[16 + hrow];
        float p0[4], p1[4], x0[4], x1[4], mx[4];
        bool grow = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x0[r] = v0 ? s[0][r] * qk_scale : -INFINITY;
            x1[r] = v1 ? s[1][r] * qk_scale : -INFINITY;
            mx[r] = row_max16(fmaxf(x0[r], x1[r]));
            grow |= mx[r] > mrun[r] + 8.0f;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform
            float corr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mnew = fmaxf(mrun[r], mx[r]);
                corr[r] = mnew == -INFINITY ? 1.0f : exp2f(mrun[r] - mnew);
                lrun[r] *= corr[r];
                mrun[r] = mnew;
            }
#pragma unroll
            for (int nb = 0; nb < 18; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[nb][r] *= corr[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float muse = mrun[r] == -INFINITY ? 0.0f : mrun[r];
            p0[r] = exp2f(x0[r] - muse);
            p1[r] = exp2f(x1[r] - muse);
            lrun[r] += row_sum16(p0[r] + p1[r]);
        }
        // P through this wave's LDS buffer into A layout, A[row = head hrow][k = slot 8 kgrp + e], as
        // two bf16 terms P = hi + lo (hi = bf16(P), lo = bf16(P - hi)): both multiply the same V
        // fragment, so P V keeps ~16 mantissa bits at no extra LDS traffic.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint16_t h0b = f2bf(p0[r]), h1b = f2bf(p1[r]);
            pw[(4 * kgrp + r) * kVS + hrow] = h0b;
            pw[(4 * kgrp + r) * kVS + 16 + hrow] = h1b;
            pw[(16 + 4 * kgrp + r) * kVS + hrow] = f2bf(p0[r] - bf2f(h0b));
            pw[(16 + 4 * kgrp + r) * kVS + 16 + hrow] = f2bf(p1[r] - bf2f(h1b));
        }
        // the buffer is this wave's own: order its LDS writes before its reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const bf16x8 pa = __builtin_bit_cast(bf16x8, *(const u32x4*)(pw + hrow * kVS + 8 * kgrp));
        const bf16x8 pl = __builtin_bit_cast(bf16x8, *(const u32x4*)(pw + (16 + hrow) * kVS + 8 * kgrp));
        // O += P V over this wave's dims: B[k = slot 8 kgrp + e][n = dim dbase + 16 nb + hrow], two
        // transposing reads of four slots each (this lane addresses slot 8 kgrp + hrow / 4 (+4))
#pragma unroll
        for (int nb = 0; nb < 18; ++nb) {
            const s16x4 w0 = lds_tr16(vr + 16 * nb);
            const s16x4 w1 = lds_tr16(vr + 4 * kKS + 16 * nb);
            const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7));
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[nb], 0, 0, 0);
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[nb], 0, 0, 0);
        }
    }

    // epilogue: this wave's heads h0 + 4 kgrp + r and dims dbase + 16 nb + hrow
    const int64_t nrows = (int64_t)gridDim.x;
    if (nsplit > 1) {
        float* wo = (float*)a.ws;
        float* wml = wo + (int64_t)nsplit * nrows * a.H * kC;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = h0 + 4 * kgrp + r;
            if (h >= a.H) continue;
            const int64_t pr = ((int64_t)split * nrows + rowid) * a.H + h;
            float* dst = wo + pr * kC + dbase + hrow;
#pragma unroll
            for (int nb = 0; nb < 18; ++nb) dst[16 * nb] = o[nb][r];
            if (hrow == 0 && dh == 0) {
                wml[2 * pr] = mrun[r];
                wml[2 * pr + 1] = lrun[r];
            }
        }
        return;
    }
    // output RoPE: dims 512 + i and 544 + i (i < 32) sit in this half's blocks 14 + q2 and 16 + q2
    float sn[2] = {0.0f, 0.0f}, cs[2] = {1.0f, 1.0f};
    const bool rot = a.rope_theta != 0.0 && dh == 1;
    if (rot) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) rope_sincos(a.rope.inv, 16 * q2 + hrow, -(double)t, &sn[q2], &cs[q2]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = h0 + 4 * kgrp + r;
        if (h >= a.H) continue;
        float mu = mrun[r];
        float den = lrun[r];
        if (a.sink) {
            const float z = a.sink[h] * kLog2e;
            mu = fmaxf(mrun[r], z);
            den = (mrun[r] == -INFINITY ? 0.0f : lrun[r] * exp2f(mrun[r] - mu)) + exp2f(z - mu);
        }
        const float f = den > 0.0f && mrun[r] != -INFINITY ? exp2f(mrun[r] - mu) / den : 0.0f;
        float ov[18];
#pragma unroll
        for (int nb = 0; nb < 18; ++nb) ov[nb] = o[nb][r] * f;
        if (rot) {
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const float x0 = ov[14 + q2], x1 = ov[16 + q2];
                ov[14 + q2] = x0 * cs[q2] - x1 * sn[q2];
                ov[16 + q2] = x0 * sn[q2] + x1 * cs[q2];
            }
        }
        const int64_t orow = (rowid * a.H + h) * kC + dbase + hrow;
        if (a.out_dtype == LCA_F32) {
            float* dst = (float*)a.out + orow;
#pragma unroll
            for (int nb = 0; nb < 18; ++nb) dst[16 * nb] = ov[nb];
        } else {
            uint16_t* dst = (uint16_t*)a.out + orow;
#pragma unroll
            for (int nb = 0; nb < 18; ++nb) dst[16 * nb] = f2bf(ov[nb]);
        }
        if (a.lse && hrow == 0 && dh == 0)
            a.lse[rowid * a.H + h] = den > 0.0f ? (mu + log2f(den)) * kLn2 : -INFINITY;
    }
}

// Merge nsplit partial (O, m, l) triples of one (row, head) in split order.
// Block (row, head, dim chunk of 192): wave 0 turns the splits' (m, l) into
// weights in LDS, then every thread reduces its dim over the splits.
constexpr int kCombDims = 192;
__global__ void __launch_bounds__(kCombDims) attn_combine(AttnArgs a, int nsplit, int c, int d_nope,
                                                          int d_rope) {
    const int64_t rowid = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int d = blockIdx.z * kCombDims + tid;
    const int64_t nrows = gridDim.x;
    const float* wo = (const float*)a.ws;
    const float* wml = wo + (int64_t)nsplit * nrows * a.H * c;
    const int b = (int)(rowid / a.T);
    const int64_t t = a.q_pos.v[b] + rowid % a.T;
    __shared__ float wsp[1024];
    __shared__ float s_mu, s_den;
    if (tid < 64) {
        float M = -INFINITY;
        for (int j = lane; j < nsplit; j += 64) M = fmaxf(M, wml[2 * ((j * nrows + rowid) * a.H + h)]);
        M = wave_max(M);
        float mu = M;
        const float z = a.sink ? a.sink[h] * kLog2e : -INFINITY;
        if (a.sink) mu = fmaxf(M, z);
        const float muse = mu == -INFINITY ? 0.0f : mu;
        float den = 0.0f;
        for (int j = lane; j < nsplit; j += 64) {
            const int64_t pr = (j * nrows + rowid) * a.H + h;
            const float wgt = exp2f(wml[2 * pr] - muse);
            wsp[j] = wgt;
            den += wml[2 * pr + 1] * wgt;
        }
        den = wave_sum(den) + (a.sink ? exp2f(z - muse) : 0.0f);
        if (lane == 0) {
            s_mu = mu;
            s_den = den;
        }
    }
    __syncthreads();
    const float den = s_den, mu = s_mu;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    if (a.lse && blockIdx.z == 0 && tid == 0)
        a.lse[rowid * a.H + h] = den > 0.0f ? (mu + log2f(den)) * kLn2 : -INFINITY;
    if (d >= c) return;
    // this thread's dim, and its RoPE partner when the output is rotated
    const int half = d_rope / 2;
    const bool rot = a.rope_theta != 0.0 && d >= d_nope;
    const int r = d - d_nope;
    const int dp = !rot ? d : (r < half ? d + half : d - half);
    const int64_t stride = nrows * a.H * c;  // between splits
    const float* p0 = wo + (rowid * a.H + h) * c;
    float acc = 0.0f, accp = 0.0f;
    int j = 0;
    for (; j + 16 <= nsplit; j += 16) {
        float v[16], vp[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            v[u] = p0[(j + u) * stride + d];
            vp[u] = rot ? p0[(j + u) * stride + dp] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            acc = fmaf(v[u], wsp[j + u], acc);
            accp = fmaf(vp[u], wsp[j + u], accp);
        }
    }
    for (; j < nsplit; ++j) {
        acc = fmaf(p0[j * stride + d], wsp[j], acc);
        if (rot) accp = fmaf(p0[j * stride + dp], wsp[j], accp);
    }
    float v = acc * inv;
    if (rot) {
        float sn, cs;
        rope_sincos(a.rope.inv, r < half ? r : r - half, -(double)t, &sn, &cs);
        const float vp = accp * inv;
        v = r < half ? v * cs - vp * sn : vp * sn + v * cs;
    }
    const int64_t oi = (rowid * a.H + h) * c + d;
    if (a.out_dtype == LCA_F32) ((float*)a.out)[oi] = v;
    else ((uint16_t*)a.out)[oi] = f2bf(v);
}

// f32 caches: one wave per (row, head); lane owns dims lane + 64 u.
__global__ void __launch_bounds__(64) attn_f32(AttnArgs a) {
    const int64_t rowid = blockIdx.x;
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int b = (int)(rowid / a.T);
    const int64_t t = a.q_pos.v[b] + rowid % a.T;
    const SlotMap sm = slot_map(a, t);
    const int d_nope = a.comp.d_nope, d_rope = a.comp.d_rope, c = d_nope + d_rope;
    constexpr int U = 16;  // c <= 1024
    __shared__ float osh[1024];

    const float* q = (const float*)a.q + (rowid * a.H + h) * c;
    float qv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int d = lane + 64 * u;
        qv[u] = d < c ? q[d] : 0.0f;
        ov[u] = 0.0f;
    }
    float mrun = -INFINITY, lrun = 0.0f;
    const float qk_scale = a.sm_scale * kLog2e;
    for (int64_t slot = 0; slot < sm.nslots; ++slot) {
        int64_t row = 0;
        const int src = slot_row(a, sm, rowid, b, slot, sm.nslots, &row);
        if (!src) continue;
        const lca_kv& kv = src == 2 ? a.win : a.comp;
        const float* np = (const float*)kv.nope + row * d_nope;
        const float* rp = (const float*)kv.rope + row * d_rope;
        float kvv[U];
        float dot = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int d = lane + 64 * u;
            kvv[u] = d < d_nope ? np[d] : (d < c ? rp[d - d_nope] : 0.0f);
            dot = fmaf(qv[u], kvv[u], dot);
        }
        const float x = wave_sum(dot) * qk_scale;
        const float mnew = fmaxf(mrun, x);
        const float corr = exp2f(mrun - mnew);
        const float p = exp2f(x - mnew);
        lrun = lrun * corr + p;
#pragma unroll
        for (int u = 0; u < U; ++u) ov[u] = fmaf(p, kvv[u], ov[u] * corr);
        mrun = mnew;
    }
    float mu = mrun, den = lrun;
    if (a.sink) {
        const float z = a.sink[h] * kLog2e;
        mu = fmaxf(mrun, z);
        den = (mrun == -INFINITY ? 0.0f : lrun * exp2f(mrun - mu)) + exp2f(z - mu);
    }
    const float f = den > 0.0f && mrun != -INFINITY ? exp2f(mrun - mu) / den : 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int d = lane + 64 * u;
        if (d < c) osh[d] = ov[u] * f;
    }
    __syncthreads();
    const int half = d_rope / 2;
    for (int d = lane; d < c; d += 64) {
        float v = osh[d];
        if (a.rope_theta != 0.0 && d >= d_nope) {
            const int r = d - d_nope;
            float sn, cs;
            rope_sincos(a.rope.inv, r < half ? r : r - half, -(double)t, &sn, &cs);
            v = r < half ? v * cs - osh[d + half] * sn : osh[d - half] * sn + v * cs;
        }
        const int64_t oi = (rowid * a.H + h) * c + d;
        if (a.out_dtype == LCA_F32) ((float*)a.out)[oi] = v;
        else ((uint16_t*)a.out)[oi] = f2bf(v);
    }
    if (a.lse && lane == 0) a.lse[rowid * a.H + h] = den > 0.0f ? (mu + log2f(den)) * kLn2 : -INFINITY;
}

// Split policy: decode-sized launches split the slot list so that the grid
// covers the chip; prefill-sized launches use one split per row.
#ifndef LCA_SPLIT_TARGET
#define LCA_SPLIT_TARGET 256   // workgroups a decode-sized launch aims for (one per CU)
#endif
#ifndef LCA_SPLIT_MIN_SLOTS
#define LCA_SPLIT_MIN_SLOTS 128  // fewest slots per split
#endif
int attn_num_splits(int64_t rows, int64_t max_keys, int32_t c) {
    if (c != kC || rows >= 128 || max_keys <= LCA_SPLIT_MIN_SLOTS) return 1;
    int64_t want = (LCA_SPLIT_TARGET + rows - 1) / rows;
    int64_t most = (max_keys + LCA_SPLIT_MIN_SLOTS - 1) / LCA_SPLIT_MIN_SLOTS;
    if (want > most) want = most;
    if (want > 1024) want = 1024;           // combine keeps the split weights in LDS
    if (want < 1) want = 1;
    int64_t len = (max_keys + want - 1) / want;
    len = (len + kKT - 1) / kKT * kKT;
    return (int)((max_keys + len - 1) / len);
}

static int64_t split_len_of(int64_t max_keys, int nsplit) {
    int64_t len = (max_keys + nsplit - 1) / nsplit;
    return (len + kKT - 1) / kKT * kKT;
}

size_t attn_ws_bytes(int64_t rows, int32_t H, int32_t c, int64_t max_keys) {
    const int ns = attn_num_splits(rows, max_keys, c);
    if (ns <= 1) return 0;
    return (size_t)ns * rows * H * (c + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.T;
    if (rows <= 0) return hipSuccess;
    const int c = a.comp.d_nope + a.comp.d_rope;
    if (a.comp.fmt == LCA_F32) {
        hipLaunchKernelGGL(attn_f32, dim3((unsigned)rows, (unsigned)a.H), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    const int ns = attn_num_splits(rows, a.max_keys, c);
    const int64_t len = ns > 1 ? split_len_of(a.max_keys, ns) : (a.max_keys + kKT - 1) / kKT * kKT;
    dim3 grid((unsigned)rows, (unsigned)ns);
    if (a.comp.fmt == LCA_FP8) hipLaunchKernelGGL((attn_mfma<LCA_FP8>), grid, dim3(512), 0, st, a, len, ns);
    else hipLaunchKernelGGL((attn_mfma<LCA_BF16>), grid, dim3(512), 0, st, a, len, ns);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns <= 1) return e;
    hipLaunchKernelGGL(attn_combine, dim3((unsigned)rows, (unsigned)a.H, (unsigned)((c + kCombDims - 1) / kCombDims)),
                       dim3(kCombDims), 0, st, a, ns, c, a.comp.d_nope, a.comp.d_rope);
    return hipGetLastError();
}

}  // namespace lca
