// attn.hip -- core attention of the DeepSeek-V4 hybrid attention
// ("DeepSeek-V4 中文翻译" sections 2.3.1 - 2.3.3): shared-KV MQA (each stored
// row is both key and value, one KV head for every query head) over
//   CSA: the top-k selected compressed entries, or
//   HCA: every visible compressed entry,
// plus the sliding window of raw rows, with a per-head sink logit and RoPE
// applied to the output by -t.
//
// bf16 / fp8 caches, c = 512 + 64, H up to 64 (taken 16 heads at a time; the heads of a last
// partial group past H have zero queries and store nothing): MFMA path.
//   One workgroup (8 waves) per (query row, key split).  The attended rows are
//   a list of "slots": compressed slots (idx entries, or 0..vis-1) followed by
//   window slots.  Per tile of 32 slots the workgroup gathers the rows from HBM
//   (fp8 codes are expanded to bf16 exactly: the scale is a power of two) into
//   one row-major LDS tile (three tiles rotate, see the pipeline below).  The
//   tile serves both operands: the K operand of the score product (16
//   contiguous bytes of one key per lane, ds_read_b128) and the V operand of
//   the value product (four keys of one dim per lane) through gfx950's
//   transposing LDS read ds_read_b64_tr_b16: within each 16-lane group, lane i
//   receives element i mod 4 of the 8-byte rows addressed by lanes i/4 + 4e,
//   so lanes addressing (key r/4, dims 4(r mod 4)..+3) hand lane i four keys of
//   dim i.
//   Wave w owns heads [16 (w % 4), +16) and dims [288 (w / 4), +288).  Scores
//   are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16, rows =
//   slots, columns = heads, Q^T fragments in registers), so each lane holds one
//   head: the softmax row statistics are per-lane values, and the bf16 weights
//   (as a hi + lo pair) go from the accumulator registers straight into the
//   B operand of O^T += V^T P^T.  The two waves of a head group exchange their
//   288-dim partial scores through LDS and add them in the same order.
//   Decode-sized launches split the slot list across workgroups; a second
//   kernel merges the partial (O, max, sum) triples in a fixed order.
// f32 caches: one wave per (query row, head), f32 FMA, for fp32 workloads.
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "rowstore.h"
#include "trace.h"

namespace lca {

constexpr int kDN = 512, kDR = 64, kC = 576;
constexpr int kKT = 32;             // slots per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SlotMap {
    int64_t vis;     // visible compressed entries, min(floor((t + 1) / m), comp.cap)
    int64_t ncs;     // compressed slots
    int64_t w_lo;    // first window position
    int64_t w_row;   // its ring row, w_lo mod win.cap
    int64_t nslots;
};

// Row i of sequence b (position t = q_pos[b] + i).  No 64-bit division: the window ring row of
// the first window position comes from the host's per-sequence base (i < T <= win.cap, so one
// subtraction wraps it), and m is a shift when it is a power of two.
__device__ __forceinline__ SlotMap slot_map(const AttnArgs& a, int b, int i, int64_t* tp) {
    SlotMap s;
    const int64_t t = a.q_pos.v[b] + i;
    *tp = t;
    const int64_t q1 = a.m_shift >= 0 ? (t + 1) >> a.m_shift : (t + 1) / a.m;
    const int64_t vis = min(q1, a.comp.cap);
    s.vis = vis;
    s.ncs = a.idx ? (int64_t)a.k : vis;
    const int64_t d = a.q_pos.v[b] - a.n_win + 1;  // first window position of row 0
    const int64_t wl = d + i;
    s.w_lo = wl < 0 ? 0 : wl;
    const int64_t nw = a.n_win > 0 ? t - s.w_lo + 1 : 0;
    int64_t wr = 0;
    if (nw > 0 && wl > 0) {
        if (d < 0) wr = wl;  // below win.cap: i < T <= win.cap
        else {
            wr = a.w_base.v[b] + i;
            if (wr >= a.win.cap) wr -= a.win.cap;
        }
    }
    s.w_row = wr;
    s.nslots = s.ncs + nw;
    return s;
}

// (rowid = b * T + i, 32-bit)
__device__ __forceinline__ void row_coords(const AttnArgs& a, int64_t rowid, int* b, int* i) {
    const uint32_t r = (uint32_t)rowid, T = (uint32_t)a.T;
    *b = (int)(r / T);
    *i = (int)(r - (uint32_t)*b * T);
}

// source row of a slot: 0 = invalid, 1 = compressed row, 2 = window row.  A listed entry id is
// attended only when it is visible, 0 <= e < vis(t): an entry whose block ends after t never is
// (block-level causality), whatever the index list says.  Window slots are consecutive positions,
// fewer than win.cap of them, so their ring rows wrap at most once.
__device__ __forceinline__ int slot_row(const AttnArgs& a, const SlotMap& sm, int64_t rowid, int b,
                                        int64_t slot, int64_t s_end, int64_t* row) {
    if (slot >= s_end) return 0;
    if (slot < sm.ncs) {
        int64_t e = a.idx ? (int64_t)a.idx[rowid * a.k + slot] : slot;
        if (e < 0 || e >= sm.vis) return 0;
        *row = (int64_t)b * a.comp.cap + e;
        return 1;
    }
    int64_t r = sm.w_row + (slot - sm.ncs);
    if (r >= a.win.cap) r -= a.win.cap;
    *row = (int64_t)b * a.win.cap + r;
    return 2;
}

// Kernel-argument pointers pinned in scalar registers.  A per-lane choice between two of them
// must be a choice between register values: written as a choice between struct fields, the
// compiler turns it into a per-lane load of the chosen field from the argument segment, which
// puts a dependent memory round trip in front of every gathered row.
// (global address space kept explicit: through the integer round trip it would be lost and
// the loads would become flat loads)
#define GMEM __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const GMEM T* sptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const GMEM T*)(((uint64_t)hi << 32) | lo);
}
struct KvPtrs {  // rows of one sequence: [0] compressed rows, [1] window rows
    const GMEM uint8_t* nope[2];
    const GMEM uint16_t* rope[2];
    const GMEM float* scale[2];
};

// The gather: half-wave h = tid / 32 (16 of them) moves tile rows h and h + 16, one whole row
// per load instruction (fp8 rows: 32 lanes x 16 codes; bf16 rows: 32 lanes x 8 dims, twice),
// RoPE chunk c (8 bf16) by lane c < 8.  An invalid slot loads nothing; its tile row is zeros.
// DENSE (HCA): compressed slot s is entry s.  Otherwise (CSA) the entry ids come from idx and are
// fetched one tile ahead of the rows (fetch_idx), so the row loads never wait on them.
template <int FMT, bool DENSE>
struct Gather {
    static constexpr int kN = FMT == LCA_FP8 ? 1 : 2;              // nope chunks per row and thread
    static constexpr uint32_t kRow = FMT == LCA_FP8 ? kDN : 2 * kDN;  // nope bytes per row
    u32x4 v[2][kN + 1];
    float sc[2];
    int src[2];
    int32_t ent[2];  // entry ids of the next tile's rows (CSA)
    // byte offsets of row h, chunk c from a tile's first row (row h + 16 adds 16 rows)
    uint32_t on, os, orp;
    int h, c;

    __device__ __forceinline__ void init(int h_, int c_) {
        h = h_;
        c = c_;
        on = h * kRow + 16u * c;
        os = h * 16u + 4u * (c >> 3);  // 16-code chunk c covers dims 16c .. 16c+15: scale group c / 8
        orp = h * 128u + 16u * c;
    }

    __device__ __forceinline__ void fetch_idx(const SlotMap& sm, const GMEM int32_t* irow, int64_t s0, int64_t s_end) {
        const int64_t lim = min(sm.ncs, s_end);
        const GMEM int32_t* ip = irow + s0 + h;  // this lane's slots of the tile
        if (s0 + kKT <= lim) {                   // wave-uniform
            ent[0] = ip[0];
            ent[1] = ip[16];
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) ent[u] = s0 + h + 16 * u < lim ? ip[16 * u] : -1;
        }
    }

    // Common case, decided per tile (wave-uniform): every slot of the tile is a compressed slot.
    // Rows are addressed from a per-tile scalar base (dense) or from 32-bit row offsets (CSA;
    // off32: the sequence's rows span less than 4 GiB).
    __device__ __forceinline__ void load_comp(const SlotMap& sm, const KvPtrs& P, int64_t s0) {
        if constexpr (DENSE) {
            const GMEM uint8_t* bn = P.nope[0] + s0 * kRow;
            const GMEM uint8_t* bs = (const GMEM uint8_t*)P.scale[0] + s0 * 16;
            const GMEM uint8_t* br = (const GMEM uint8_t*)P.rope[0] + s0 * 128;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                src[u] = 1;
                v[u][0] = *(const GMEM u32x4*)(bn + (on + 16u * kRow * u));
                if constexpr (FMT == LCA_FP8) sc[u] = *(const GMEM float*)(bs + (os + 256u * u));
                else v[u][1] = *(const GMEM u32x4*)(bn + (on + 16u * kRow * u + 512u));
                if (c < 8) v[u][kN] = *(const GMEM u32x4*)(br + (orp + 2048u * u));
            }
        } else {
            bool ok[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) ok[u] = ent[u] >= 0 && ent[u] < sm.vis;  // visible entries only
            const bool all = !__builtin_amdgcn_ballot_w64(!(ok[0] && ok[1]));  // wave-uniform
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                src[u] = ok[u];
                if (!all) {
#pragma unroll
                    for (int q = 0; q <= kN; ++q) v[u][q] = u32x4{0u, 0u, 0u, 0u};
                    sc[u] = 0.0f;
                    if (!ok[u]) continue;
                }
                const uint32_t eu = (uint32_t)ent[u];
                v[u][0] = *(const GMEM u32x4*)(P.nope[0] + (eu * kRow + 16u * c));
                if constexpr (FMT == LCA_FP8) sc[u] = *(const GMEM float*)((const GMEM uint8_t*)P.scale[0] + (eu * 16u + 4u * (c >> 3)));
                else v[u][1] = *(const GMEM u32x4*)(P.nope[0] + (eu * kRow + 16u * c + 512u));
                if (c < 8) v[u][kN] = *(const GMEM u32x4*)((const GMEM uint8_t*)P.rope[0] + (eu * 128u + 16u * c));
            }
        }
    }

    // General case: window slots, slots past the end, or rows beyond 32-bit offsets.
    __device__ __forceinline__ void load(const AttnArgs& a, const SlotMap& sm, const KvPtrs& P, bool off32,
                                         int64_t s0, int64_t s_end) {
        if (off32 && s0 + kKT <= min(sm.ncs, s_end)) {  // wave-uniform
            load_comp(sm, P, s0);
            return;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t slot = s0 + h + 16 * u;
            // source row: compressed slot (entry id, or the slot itself when dense) or window slot;
            // window slots are consecutive positions, fewer than win.cap, wrapping at most once
            int64_t row = 0;
            int sr = 0;
            if (slot < s_end) {
                if (slot < sm.ncs) {
                    const int64_t e = DENSE ? slot : (int64_t)ent[u];
                    if (e >= 0 && e < sm.vis) {
                        row = e;
                        sr = 1;
                    }
                } else {
                    int64_t r = sm.w_row + (slot - sm.ncs);
                    if (r >= a.win.cap) r -= a.win.cap;
                    row = r;
                    sr = 2;
                }
            }
            src[u] = sr;
            const int w = sr == 2;
            const GMEM uint8_t* nope = w ? P.nope[1] : P.nope[0];
            const GMEM uint16_t* rope = w ? P.rope[1] : P.rope[0];
#pragma unroll
            for (int q = 0; q <= kN; ++q) v[u][q] = u32x4{0u, 0u, 0u, 0u};
            sc[u] = 0.0f;
            if (!sr) continue;
            if constexpr (FMT == LCA_FP8) {
                const GMEM float* scale = w ? P.scale[1] : P.scale[0];
                v[u][0] = ((const GMEM u32x4*)(nope + row * kDN))[c];
                sc[u] = scale[row * 4 + (c >> 3)];
            } else {
                const GMEM u32x4* np = (const GMEM u32x4*)(nope + row * kDN * 2);
                v[u][0] = np[c];
                v[u][1] = np[c + 32];
            }
            if (c < 8) v[u][kN] = ((const GMEM u32x4*)(rope + row * kDR))[c];
        }
    }
};

// Tile layout: row r (slot) at r * kKS, dims contiguous.  The 16-element pad (row stride
// 1184 bytes) keeps both reads near the conflict-free LDS rate on gfx950: the 16 rows of one
// ds_read_b128 phase and the four 32-byte row pieces of one transposing read fall on
// different banks (measured against other strides and XOR swizzles).
constexpr int kKS = kC + 16;

__device__ __forceinline__ void put8(uint16_t* Kt, int j, int chunk, u32x4 v) {
    *(u32x4*)(Kt + j * kKS + 8 * chunk) = v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// transposing LDS read (see the header comment) at an LDS byte address
__device__ __forceinline__ s16x4 lds_tr16(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(uintptr_t)addr);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// two fp8 codes (low 16 bits when !kHigh) -> packed bf16 bits of code * scale, in one gfx950
// scaled conversion (v_cvt_scalef32_pk_bf16_fp8).  It decodes OCP e4m3fn exactly and applies the
// power-of-two scale; a 4-significant-bit product is exact in bf16.  (Checked bit for bit against
// decode, multiply and truncation to bf16 for every code pair and the scales 2^-20 .. 2^9.)
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t codes, float sc) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, sc, kHigh));
}

// Expand and store one tile; flags[r] = slot r valid (read back as 32-bit words of 4 slots).
template <int FMT, bool DENSE>
__device__ __forceinline__ void store_tile(const Gather<FMT, DENSE>& g, uint16_t* Kt, uint8_t* flags) {
    const int h = g.h, c = g.c;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = h + 16 * u;
        if constexpr (FMT == LCA_FP8) {
            u32x4 lo, hi;
            lo[0] = fp8x2_bf16<false>(g.v[u][0][0], g.sc[u]);
            lo[1] = fp8x2_bf16<true>(g.v[u][0][0], g.sc[u]);
            lo[2] = fp8x2_bf16<false>(g.v[u][0][1], g.sc[u]);
            lo[3] = fp8x2_bf16<true>(g.v[u][0][1], g.sc[u]);
            hi[0] = fp8x2_bf16<false>(g.v[u][0][2], g.sc[u]);
            hi[1] = fp8x2_bf16<true>(g.v[u][0][2], g.sc[u]);
            hi[2] = fp8x2_bf16<false>(g.v[u][0][3], g.sc[u]);
            hi[3] = fp8x2_bf16<true>(g.v[u][0][3], g.sc[u]);
            put8(Kt, r, 2 * c, lo);
            put8(Kt, r, 2 * c + 1, hi);
        } else {
            put8(Kt, r, c, g.v[u][0]);
            put8(Kt, r, c + 32, g.v[u][1]);
        }
        if (c < 8) put8(Kt, r, kDN / 8 + c, g.v[u][Gather<FMT, DENSE>::kN]);
        if (c == 0) flags[r] = g.src[u] != 0;
    }
}


__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};  // nearest-even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint32_t, v);
}

// Eight waves: wave w owns heads [16 (w % 4), +16) and output dims [288 (w / 4), +288).
// Per wave: Q^T fragments 36 VGPRs, O^T 72 VGPRs -> two waves per SIMD.
//
// The tile loop is software-pipelined over three LDS tiles so that every phase has both matrix
// and vector work:
//   phase 1 (tile t):  S^T partial = K Q^T over the wave's dims  |  expand + store tile t+1,
//                      fetch tile t+2 into registers
//   phase 2:           O^T += V^T P^T of tile t-1               |  exchange + softmax of tile t
// The running max can move in phase 2 of tile t; O is rescaled at the end of that phase, after
// tile t-1's product has been added and before tile t's is.
constexpr int kHalf = kC / 2;  // 288
constexpr int kTileElems = kKT * kKS;
template <int FMT, bool DENSE>
__global__ void __launch_bounds__(512) attn_mfma(AttnArgs a, int64_t split_len, int nsplit) {
    __shared__ __attribute__((aligned(16))) uint16_t Kt[3][kTileElems];
    __shared__ __attribute__((aligned(16))) f32x4 Sx[8][2][64];  // partial scores
    __shared__ uint32_t vflag[3][kKT / 4];                         // slot valid flags, per tile

    const int64_t rowid = blockIdx.x;
    const int split = blockIdx.y;
    int b, ri;
    row_coords(a, rowid, &b, &ri);
    int64_t t;
    const SlotMap sm = slot_map(a, b, ri, &t);
    const int64_t s_begin = (int64_t)split * split_len;
    const int64_t s_end = min(sm.nslots, s_begin + split_len);
    const int ntile = s_end > s_begin ? (int)((s_end - s_begin + kKT - 1) / kKT) : 0;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, g4 = lane >> 4;  // MFMA lane coordinates
    const int hg = wv & 3, dh = wv >> 2;      // head group, dim half
    const int h0 = 16 * hg, dbase = kHalf * dh;
    const bool active = h0 < a.H;             // wave-uniform
    const bool hv = h0 + n < a.H;             // this lane's head exists (H need not be a multiple of 16:
                                              // a missing head has zero queries and stores nothing)

    // Q^T fragments: B[k = dim dbase + 32 ks + 8 g4 + e][n = head h0 + n]
    bf16x8 qf[9];
    {
        const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + (rowid * a.H + (hv ? h0 + n : 0)) * kC + dbase);
#pragma unroll
        for (int ks = 0; ks < 9; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, hv ? qp[4 * ks + g4] : u32x4{0u, 0u, 0u, 0u});
    }
    // O^T: lane holds dims dbase + 16 nb + 4 g4 + i (i < 4) of head h0 + n
    f32x4 o[18];
#pragma unroll
    for (int nb = 0; nb < 18; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = -INFINITY;  // running max (log2 domain) of head h0 + n
    float lpart = 0.0f;      // this lane's share of the running sum
    const float qk_scale = a.sm_scale * kLog2e;

    // K operand: rows n and 16 + n, dims dbase + 32 ks + 8 g4
    const int koff = n * kKS + dbase + 8 * g4;
    // V operand: rows 4 g4 + n / 4 and 16 + that (slots 4 g4 + e, 16 + 4 g4 + e), dims
    // dbase + 16 nb + 4 (n & 3)
    const int voff = (4 * g4 + (n >> 2)) * kKS + dbase + 4 * (n & 3);

    constexpr int64_t kRowBytes = FMT == LCA_FP8 ? kDN : 2 * kDN;
    KvPtrs P;  // this sequence's rows
    P.nope[0] = sptr<uint8_t>(a.comp.nope) + (int64_t)b * a.comp.cap * kRowBytes;
    P.nope[1] = sptr<uint8_t>(a.win.nope) + (int64_t)b * a.win.cap * kRowBytes;
    P.rope[0] = sptr<uint16_t>(a.comp.rope) + (int64_t)b * a.comp.cap * kDR;
    P.rope[1] = sptr<uint16_t>(a.win.rope) + (int64_t)b * a.win.cap * kDR;
    P.scale[0] = FMT == LCA_FP8 ? sptr<float>(a.comp.scale) + (int64_t)b * a.comp.cap * 4 : nullptr;
    P.scale[1] = FMT == LCA_FP8 ? sptr<float>(a.win.scale) + (int64_t)b * a.win.cap * 4 : nullptr;
    const GMEM int32_t* irow = DENSE ? nullptr : sptr<int32_t>(a.idx) + rowid * a.k;  // this row's entry ids
    const bool off32 = a.comp.cap * kRowBytes < (int64_t)1 << 32;
    Gather<FMT, DENSE> g;
    g.init(tid >> 5, tid & 31);
    if (ntile > 0) {
        if constexpr (!DENSE) g.fetch_idx(sm, irow, s_begin, s_end);
        g.load(a, sm, P, off32, s_begin, s_end);
        if constexpr (!DENSE) g.fetch_idx(sm, irow, s_begin + kKT, s_end);
        store_tile(g, Kt[0], (uint8_t*)vflag[0]);
        if (ntile > 1) {
            g.load(a, sm, P, off32, s_begin + kKT, s_end);
            if constexpr (!DENSE) g.fetch_idx(sm, irow, s_begin + 2 * kKT, s_end);
        }
    }
    // The Q loads were issued before tile 0's, which store_tile has waited for.  Consume them
    // here, on every path into the loop, so that the waits inside the loop cover only the gather
    // loads in flight (otherwise the first Q use in the loop waits for every load).
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) asm volatile("" ::"v"(qf[ks]));

    // O^T += V^T P^T over one tile: A[row = dim dbase + 16 nb + n][k = slot pi(8 g4 + e)], two
    // transposing reads (slots 4 g4 + e and 16 + 4 g4 + e); P as bf16 hi + lo
    // (tile buffers are addressed by uniform byte offsets that rotate every tile, so that every
    // read is one base register plus an immediate offset)
    const uint32_t vbase = lds_addr(&Kt[0][0]) + 2 * voff;
    auto pv = [&](uint32_t boff, const bf16x8& pa, const bf16x8& pb) {
        const uint32_t vr = vbase + boff;
#pragma unroll
        for (int nb = 0; nb < 18; ++nb) {
            const s16x4 w0 = lds_tr16(vr + 32 * nb);
            const s16x4 w1 = lds_tr16(vr + 32 * kKS + 32 * nb);
            const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7));
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pa, o[nb], 0, 0, 0);
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[nb], 0, 0, 0);
        }
    };

    bf16x8 pa = {}, pb = {};  // P^T of the previous tile (B operand, hi / lo)
    constexpr uint32_t kTileBytes = 2 * kTileElems;
    uint32_t bq = 0, bs = kTileBytes, bp = 2 * kTileBytes;  // byte offsets: tiles it, it + 1, it - 1
    int fq = 0, fs = 1;                                      // their flag sets
    for (int it = 0; it < ntile; ++it) {
        __syncthreads();  // tile it stored; tile it - 2 (this phase's store target) consumed
        // ---- phase 1 ----
        const uint16_t* K = (const uint16_t*)((const char*)&Kt[0][0] + bq);
        f32x4 s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        {  // (every wave: with H < 64 an idle wave multiplies zero queries; no branch here lets
           // the tile store below fill the waits of these reads)
            const uint16_t* kr = K + koff;
#pragma unroll
            for (int ks = 0; ks < 9; ++ks) {
                const bf16x8 k0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr + 32 * ks));
                const bf16x8 k1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr + 16 * kKS + 32 * ks));
                s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s[1], 0, 0, 0);
            }
        }
        // Tile it + 1 (after the last tile: a harmless store of stale rows into the free buffer;
        // unconditional so that its VALU work can fill the waits of the score product).
        store_tile(g, (uint16_t*)((char*)&Kt[0][0] + bs), (uint8_t*)vflag[fs]);
        {
            if (it + 2 < ntile) {
                g.load(a, sm, P, off32, s_begin + (int64_t)(it + 2) * kKT, s_end);
                if constexpr (!DENSE) g.fetch_idx(sm, irow, s_begin + (int64_t)(it + 3) * kKT, s_end);
            }
        }
        if (active) {
            // invalid slots (zero rows) get -inf in both partial sums; lane holds slots
            // 16 kb + 4 g4 + i of head h0 + n
            const uint32_t f0 = vflag[fq][g4], f1 = vflag[fq][4 + g4];
            if (__builtin_amdgcn_ballot_w64((f0 & f1) != 0x01010101u)) {  // wave-uniform
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!((f0 >> (8 * i)) & 1u)) s[0][i] = -INFINITY;
                    if (!((f1 >> (8 * i)) & 1u)) s[1][i] = -INFINITY;
                }
            }
            Sx[wv][0][lane] = s[0];
            Sx[wv][1][lane] = s[1];
        }
        __syncthreads();
        // ---- phase 2 ----
        if (active) {
            if (it > 0) pv(bp, pa, pb);  // tile it - 1
            {
                const int pw = wv ^ 4;  // the partner wave (same heads, other dim half)
                const f32x4 o0 = Sx[pw][0][lane], o1 = Sx[pw][1][lane];
                // dim half 0 + dim half 1 in both waves (the same additions, the same results)
                s[0] = dh == 0 ? s[0] + o0 : o0 + s[0];
                s[1] = dh == 0 ? s[1] + o1 : o1 + s[1];
            }
            const float smax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
            const float tmax = max4g(smax) * qk_scale;
            // The reference max moves only when the tile max exceeds it by more than 2^8 (weights
            // stay <= 256), so O is rescaled on few tiles instead of every tile.
            const bool grow = __builtin_amdgcn_ballot_w64(tmax > mrun + 8.0f) != 0;  // wave-uniform
            const float mnew = grow ? fmaxf(mrun, tmax) : mrun;
            const float corr = mnew == mrun ? 1.0f : exp2f(mrun - mnew);  // mrun = -inf -> 0
            mrun = mnew;
            const float mneg = mrun == -INFINITY ? 0.0f : -mrun;
            float p[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], qk_scale, mneg));
            lpart = lpart * corr +
                    (((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
            // B operand P^T as hi + lo = bf16(P) + bf16(P - hi): k-slot 8 g4 + e is slot 4 g4 + e
            // (e < 4) or 16 + 4 g4 + e - 4
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float x0 = p[kb][2 * q], x1 = p[kb][2 * q + 1];
                    const uint32_t hb = pk_bf16(x0, x1);
                    ph[2 * kb + q] = hb;
                    pl[2 * kb + q] = pk_bf16(x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u));
                }
            pa = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
            pb = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
            if (grow) {  // after tile it - 1's product, before tile it's
                // (the empty asm keeps this a branch: if-converted, the 72 products would run on
                // every tile)
                asm volatile("");
#pragma unroll
                for (int nb = 0; nb < 18; ++nb) o[nb] *= corr;
            }
        }
        const uint32_t bt = bp;  // tile it - 1's buffer takes tile it + 2
        bp = bq;
        bq = bs;
        bs = bt;
        fq = fs;
        fs = fs == 2 ? 0 : fs + 1;
    }
    if (!active) return;
    if (ntile > 0) pv(bp, pa, pb);  // the last tile (after the final rotation bp is its buffer)
    const float lrun = sum4g(lpart);

    // epilogue: head h = h0 + n, dims dbase + 16 nb + 4 g4 + i
    const int h = h0 + n;
    const int64_t nrows = (int64_t)gridDim.x;
    if (!hv) return;
    if (nsplit > 1) {
        // partial O (unnormalised, f32), then the (max, sum) pairs
        float* wo = (float*)a.ws;
        float* wml = wo + (int64_t)nsplit * nrows * a.H * kC;
        const int64_t pr = ((int64_t)split * nrows + rowid) * a.H + h;
        float* dst = wo + pr * kC + dbase + 4 * g4;
#pragma unroll
        for (int nb = 0; nb < 18; ++nb) __builtin_nontemporal_store(o[nb], (f32x4*)(dst + 16 * nb));
        if (g4 == 0 && dh == 0) {
            __builtin_nontemporal_store(mrun, wml + 2 * pr);
            __builtin_nontemporal_store(lrun, wml + 2 * pr + 1);
        }
        return;
    }
    float mu = mrun, den = lrun;
    if (a.sink) {
        const float z = a.sink[h] * kLog2e;
        mu = fmaxf(mrun, z);
        den = (mrun == -INFINITY ? 0.0f : lrun * exp2f(mrun - mu)) + exp2f(z - mu);
    }
    const float f = den > 0.0f && mrun != -INFINITY ? exp2f(mrun - mu) / den : 0.0f;
#pragma unroll
    for (int nb = 0; nb < 18; ++nb) o[nb] *= f;
    // output RoPE by -t: dims 512 + j and 544 + j (j < 32) are blocks 14 + q2 and 16 + q2 of the
    // upper half, j = 16 q2 + 4 g4 + i
    if (a.rope_theta != 0.0 && dh == 1) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sn, cs;
                rope_sincos(a.rope.inv, 16 * q2 + 4 * g4 + i, -(double)t, &sn, &cs);
                const float x0 = o[14 + q2][i], x1 = o[16 + q2][i];
                o[14 + q2][i] = x0 * cs - x1 * sn;
                o[16 + q2][i] = x0 * sn + x1 * cs;
            }
    }
    const int64_t orow = (rowid * a.H + h) * kC + dbase + 4 * g4;
    if (a.out_dtype == LCA_F32) {
        float* dst = (float*)a.out + orow;
#pragma unroll
        for (int nb = 0; nb < 18; ++nb) *(f32x4*)(dst + 16 * nb) = o[nb];
    } else {
        uint16_t* dst = (uint16_t*)a.out + orow;
#pragma unroll
        for (int nb = 0; nb < 18; ++nb) {
            uint2 w;
            w.x = (uint32_t)f2bf(o[nb][0]) | ((uint32_t)f2bf(o[nb][1]) << 16);
            w.y = (uint32_t)f2bf(o[nb][2]) | ((uint32_t)f2bf(o[nb][3]) << 16);
            *(uint2*)(dst + 16 * nb) = w;
        }
    }
    if (a.lse && g4 == 0 && dh == 0)
        a.lse[rowid * a.H + h] = den > 0.0f ? (mu + log2f(den)) * kLn2 : -INFINITY;
}

// Merge nsplit partial (O, m, l) triples of one (row, head).  Grid (T, H x 4, B): row i =
// blockIdx.x of sequence b = blockIdx.z, head h and dim quarter z from blockIdx.y.  ng x 36 threads
// (ng = one split group per 8 splits, at most 8): split group q = tid / 36 sums splits q, q + ng,
// ... for dims 144 z + 4 (tid % 36) .. +3 (and, for RoPE dims, their rotation partners, which lie
// in the same quarter); the group sums are added in group order.  The merge is bound by load
// latency: the arguments, each thread's first eight partials and wave 0's (m, l) pairs are all
// fetched in one round, before the weights are formed (wave 0, through LDS).
constexpr int kCombGroups = 8, kCombQuarters = 4, kCombPer = kC / 4 / kCombQuarters;  // 36 threads x 4 dims
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kCombThreads = kCombGroups * kCombPer;
// (as many groups as eight prefetched splits each need, so that few prefetch slots are padding)
static int comb_groups(int nsplit) { return nsplit <= 8 ? 1 : min(kCombGroups, (nsplit + 7) / 8); }
// quad = 0: one workgroup per (row, head, dim quarter), ng groups of 36 threads splitting the splits;
// quad = 1 (few splits): one workgroup per (row, head), its four groups of 36 threads the four dim
// quarters, so the head's split weights are formed once and there are four times fewer workgroups.
__global__ void __launch_bounds__(kCombThreads) attn_combine(AttnArgs a, int nsplit, int quad) {
    const int ng = quad ? 1 : blockDim.x / kCombPer;  // blockDim.x = max(64, ng x 36): wave 0 is whole
    const int ri = blockIdx.x, b = blockIdx.z;
    const int h = quad ? (int)blockIdx.y : (int)(blockIdx.y >> 2);
    const int qz = quad ? (int)threadIdx.x / kCombPer : (int)(blockIdx.y & 3);
    const int64_t nrows = (int64_t)gridDim.x * gridDim.z;
    const int64_t rowid = (int64_t)b * gridDim.x + ri;
    const int tid = threadIdx.x, lane = tid & 63;
    const int H = a.H;
    const float* wo = (const float*)a.ws;
    const float* sink = a.sink;
    const int64_t t = a.q_pos.v[b] + ri;
    asm volatile("" ::"s"(H), "s"(wo), "s"(sink), "s"(t));
    const float* wml = wo + (int64_t)nsplit * nrows * H * kC;
    __shared__ float wsp[1024];
    __shared__ float s_mu, s_den;
    __shared__ f32x4 part[kCombGroups - 1][kCombPer][2];
    const int el = tid % kCombPer;  // this thread's slot in the group exchange
    const int q = quad ? 0 : tid / kCombPer;
    const int e = qz * kCombPer + el;  // float4 index in the row
    const int d = 4 * e;
    // RoPE dims 512 + j pair with 544 + j (j < 32)
    const bool rot = a.rope_theta != 0.0 && d >= kDN;
    const int r = d - kDN;
    const int dp = !rot ? d : (r < kDR / 2 ? d + kDR / 2 : d - kDR / 2);
    const int64_t stride = nrows * H * kC / 4;  // between splits, in f32x4
    const f32x4* p0 = (const f32x4*)(wo + (rowid * H + h) * kC);
    // this group's first eight splits q + ng u (indices past the end read split q; weight 0)
    constexpr int kPre = 8;
    f32x4 v0[kPre], vp0[kPre];
    const bool grp = q < ng;  // (the padding lanes of a one-group block hold no split)
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int jx = q + ng * u < nsplit && grp ? q + ng * u : 0;
        v0[u] = p0[jx * stride + e];
        vp0[u] = p0[jx * stride + dp / 4];
    }
    if (tid < 64) {
        // (m, l) of splits lane, lane + 64, ..: split `lane`'s pair is loaded once, in the same round
        // as the partials, and kept for the weights (one round trip, not two, for up to 64 splits)
        f32x2 ml0 = {-INFINITY, 0.0f};
        if (lane < nsplit) ml0 = *(const f32x2*)(wml + 2 * (((int64_t)lane * nrows + rowid) * H + h));
        float M = ml0[0];
        for (int j = lane + 64; j < nsplit; j += 64) M = fmaxf(M, wml[2 * ((j * nrows + rowid) * H + h)]);
        M = wave_max_dpp(M);
        float mu = M;
        const float z = sink ? sink[h] * kLog2e : -INFINITY;
        if (sink) mu = fmaxf(M, z);
        const float muse = mu == -INFINITY ? 0.0f : mu;
        float den = 0.0f;
        if (lane < nsplit) {
            const float wgt = exp2f(ml0[0] - muse);
            wsp[lane] = wgt;
            den = ml0[1] * wgt;
        }
        for (int j = lane + 64; j < nsplit; j += 64) {
            const int64_t pr = (j * nrows + rowid) * H + h;
            const float wgt = exp2f(wml[2 * pr] - muse);
            wsp[j] = wgt;
            den += wml[2 * pr + 1] * wgt;
        }
        den = wave_sum_dpp(den) + (sink ? exp2f(z - muse) : 0.0f);
        if (lane == 0) {
            s_mu = mu;
            s_den = den;
        }
    }
    __syncthreads();
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f}, accp = {0.0f, 0.0f, 0.0f, 0.0f};
    if (grp) {
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const int jx = q + ng * u;
            const float wgt = jx < nsplit ? wsp[jx] : 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[c] = fmaf(v0[u][c], wgt, acc[c]);
                if (rot) accp[c] = fmaf(vp0[u][c], wgt, accp[c]);
            }
        }
        // the rest, eight splits at a time: all loads first, then the sums in order
        for (int j = q + ng * kPre; j < nsplit; j += ng * kPre) {
            f32x4 v[kPre], vp[kPre];
#pragma unroll
            for (int u = 0; u < kPre; ++u) {
                const int jx = j + ng * u < nsplit ? j + ng * u : j;
                v[u] = p0[jx * stride + e];
                vp[u] = p0[jx * stride + dp / 4];
            }
#pragma unroll
            for (int u = 0; u < kPre; ++u) {
                const int jx = j + ng * u;
                const float wgt = jx < nsplit ? wsp[jx] : 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc[c] = fmaf(v[u][c], wgt, acc[c]);
                    if (rot) accp[c] = fmaf(vp[u][c], wgt, accp[c]);
                }
            }
        }
    }
    if (q > 0 && grp) {
        part[q - 1][el][0] = acc;
        part[q - 1][el][1] = accp;
    }
    __syncthreads();
    if (q > 0) return;
    for (int g = 0; g < ng - 1; ++g) {
        acc += part[g][el][0];
        if (rot) accp += part[g][el][1];
    }
    const float den = s_den, mu = s_mu;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    if (a.lse && tid == 0 && qz == 0)
        a.lse[rowid * H + h] = den > 0.0f ? (mu + log2f(den)) * kLn2 : -INFINITY;
    f32x4 ov = acc * inv;
    if (rot) {
        const int pi = r < kDR / 2 ? r : r - kDR / 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float sn, cs;
            rope_sincos(a.rope.inv, pi + c, -(double)t, &sn, &cs);
            const float x = ov[c], y = accp[c] * inv;
            ov[c] = r < kDR / 2 ? x * cs - y * sn : y * sn + x * cs;
        }
    }
    const int64_t oi = (rowid * H + h) * kC + d;
    if (a.out_dtype == LCA_F32) {
        *(f32x4*)((float*)a.out + oi) = ov;
    } else {
        uint2 w;
        w.x = (uint32_t)f2bf(ov[0]) | ((uint32_t)f2bf(ov[1]) << 16);
        w.y = (uint32_t)f2bf(ov[2]) | ((uint32_t)f2bf(ov[3]) << 16);
        *(uint2*)((uint16_t*)a.out + oi) = w;
    }
}


// ---------------------------------------------------------------------------------------------
// Decode-sized launches (fewer than kDecRows query rows).  A launch of one or a few query rows
// has too little work to fill the chip with one workgroup per (row, split) over all 64 heads, and
// the partial outputs of many splits would cost more than the rows they cover (64 x 576 f32 per
// split).  Here a workgroup of four waves serves one (query row, slot split, group of 16 heads):
// the splits' partial outputs stay 16 x 576, and the four head groups of one (row, split) are
// launched on the same XCD (workgroups are dealt to the eight XCDs round-robin), so three of the
// four gathers of each row hit that XCD's L2.
//   The split's raw rows are fetched into registers up to NP tiles ahead (one HBM round trip
// before the first tile instead of one per tile); a tile is expanded into one of three LDS
// buffers (the layout of attn_mfma), so one barrier per tile separates the producers from the
// readers.  Scores: wave w computes S^T = K Q^T over dims [d0(w), +32 nks(w)) (160, 160, 128 and
// 128 dims), the four partial sums meet in LDS and every wave adds them in the same order, so
// all four hold identical scores and softmax states.  Values: wave w owns output dims
// [144 w, +144), O^T += V^T P^T with P as a bf16 hi + lo pair (as attn_mfma).
constexpr int kDecRows = 128;      // query rows below which a launch takes the decode kernel
constexpr int kDecMaxTiles = 8;    // tiles per split at most: the tile loop is unrolled in full
constexpr int kDecMaxLen = kDecMaxTiles * kKT;
constexpr int kDecWGs = 256;       // workgroups a multi-row decode launch (attn_mfma) aims for: one per CU
// workgroups an attn_dec launch aims for: three per four CUs measured best on the 1M decode step
// (its HCA layers then take 44 six-tile splits x 4 head groups instead of 52 five-tile ones: 101.0
// against 101.6 us per step; a target of 160: 104.3 us, 320: 130 us)
constexpr int kDecTargetWGs = 192;

template <int FMT>
struct DecRegs {  // one tile's raw rows for this thread
    static constexpr int kN = FMT == LCA_FP8 ? 1 : 2;  // nope chunks of 16 bytes per row
    u32x4 v[4][kN];                                    // nope chunk(s) c of rows hw + 8 u (u < 4)
    u32x4 rp;                                          // RoPE chunk c % 8 of row hw + 8 (c / 8)
    float sc[4];                                       // fp8: scale group c / 8 of rows hw + 8 u
    uint32_t ok;                                       // bit u: row hw + 8 u is a valid slot
};

// Issue the loads of tile [s0, s0 + 32) (nothing is waited for here).  Slot -> row as slot_row;
// for CSA the entry ids come from LDS.  hw = thread / 32 (eight half-waves), c = thread % 32:
// 16-byte nope chunk c of rows hw + 8 u (fp8: codes 16c .. 16c+15; bf16: dims 8c .. 8c+7 and
// 256 + 8c ..), RoPE chunk c % 8 of row hw + 8 (c / 8), scale group c / 8.  Every call issues the
// same loads with no branch: a slot that is past the end or invalid reads compressed row 0 (its
// data is dropped in dec_store), so the compiler can count the loads in flight across tiles and
// each tile waits only for its own rows.  Offsets are 32-bit (the caller checks that every plane
// of one sequence spans less than 4 GiB).
template <int FMT, bool DENSE>
__device__ __forceinline__ void dec_load(DecRegs<FMT>& R, int ncs, int w_row, int s_end, int vis, int win_cap,
                                         const KvPtrs& P, const int32_t* ent, int s_begin, int s0, int hw,
                                         int c) {
    constexpr uint32_t kRow = FMT == LCA_FP8 ? kDN : 2 * kDN;
    R.ok = 0;
    uint32_t rrow = 0;
    bool rw = false;
    if (s0 + kKT <= min(ncs, s_end)) {
        // (wave-uniform) every slot of the tile is a compressed slot: no window rows, no wrap, no
        // per-row choice of plane.  Dense: the tile's rows are consecutive entries, addressed from one
        // scalar base per tile plus loop-invariant lane offsets.  Selected: 32-bit row offsets of the
        // entry ids.  The same loads as the general path below, so the waits count alike.
        const uint32_t lane_off = (uint32_t)hw * kRow + 16u * c;
        const GMEM uint8_t* nb = P.nope[0];
        const GMEM uint8_t* sb = (const GMEM uint8_t*)P.scale[0];
        const GMEM uint8_t* rb = (const GMEM uint8_t*)P.rope[0];
        if constexpr (DENSE) {
            nb += (uint64_t)(uint32_t)s0 * kRow;
            if constexpr (FMT == LCA_FP8) sb += (uint64_t)(uint32_t)s0 * 16u;
            rb += (uint64_t)(uint32_t)s0 * 128u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t noff, soff, row;
            if constexpr (DENSE) {
                row = (uint32_t)(hw + 8 * u);  // (relative to s0)
                noff = lane_off + (uint32_t)(8 * u) * kRow;
            } else {
                const int e = ent[s0 + hw + 8 * u - s_begin];
                const bool ok = (uint32_t)e < (uint32_t)vis;
                R.ok |= (uint32_t)ok << u;
                row = ok ? (uint32_t)e : 0u;
                noff = row * kRow + 16u * c;
            }
            soff = row * 16u + 4u * (c >> 3);
            if (u == (c >> 3)) rrow = row;
            R.v[u][0] = *(const GMEM u32x4*)(nb + noff);
            if constexpr (FMT == LCA_FP8) R.sc[u] = *(const GMEM float*)(sb + soff);
            else R.v[u][1] = *(const GMEM u32x4*)(nb + (noff + 512u));
        }
        if constexpr (DENSE) R.ok = 0xfu;
        R.rp = *(const GMEM u32x4*)(rb + (rrow * 128u + 16u * (c & 7)));
        return;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int slot = s0 + hw + 8 * u;
        const bool wnd = slot >= ncs;
        int r = w_row + (slot - ncs);
        if (r >= win_cap) r -= win_cap;
        // (entry ids are read only for slots of this split: the index is clamped for the rest)
        const int e = DENSE ? slot : ent[min(slot - s_begin, kDecMaxLen - 1)];
        const bool ok = slot < s_end && (wnd || (uint32_t)e < (uint32_t)vis);
        const uint32_t row = !ok ? 0u : (uint32_t)(wnd ? r : e);
        const bool w = ok && wnd;
        R.ok |= (uint32_t)ok << u;
        if (u == (c >> 3)) {
            rrow = row;
            rw = w;
        }
        const GMEM uint8_t* nope = w ? P.nope[1] : P.nope[0];
        R.v[u][0] = *(const GMEM u32x4*)(nope + (row * kRow + 16u * c));
        if constexpr (FMT == LCA_FP8) {
            const GMEM float* scale = w ? P.scale[1] : P.scale[0];
            R.sc[u] = *(const GMEM float*)((const GMEM uint8_t*)scale + (row * 16u + 4u * (c >> 3)));
        } else {
            R.v[u][1] = *(const GMEM u32x4*)(nope + (row * kRow + 16u * c + 512u));
        }
    }
    const GMEM uint16_t* rope = rw ? P.rope[1] : P.rope[0];
    R.rp = *(const GMEM u32x4*)((const GMEM uint8_t*)rope + (rrow * 128u + 16u * (c & 7)));
}

// Expand one tile into an LDS buffer (fp8 codes times their power-of-two scale, exact in bf16);
// rows of invalid slots become zeros; flags[r] = slot r valid.
template <int FMT>
__device__ __forceinline__ void dec_store(DecRegs<FMT>& R, uint16_t* Kt, uint8_t* flags, int hw, int c) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = hw + 8 * u;
        if constexpr (FMT == LCA_FP8) {
            u32x4 lo, hi;
            lo[0] = fp8x2_bf16<false>(R.v[u][0][0], R.sc[u]);
            lo[1] = fp8x2_bf16<true>(R.v[u][0][0], R.sc[u]);
            lo[2] = fp8x2_bf16<false>(R.v[u][0][1], R.sc[u]);
            lo[3] = fp8x2_bf16<true>(R.v[u][0][1], R.sc[u]);
            hi[0] = fp8x2_bf16<false>(R.v[u][0][2], R.sc[u]);
            hi[1] = fp8x2_bf16<true>(R.v[u][0][2], R.sc[u]);
            hi[2] = fp8x2_bf16<false>(R.v[u][0][3], R.sc[u]);
            hi[3] = fp8x2_bf16<true>(R.v[u][0][3], R.sc[u]);
            put8(Kt, r, 2 * c, lo);
            put8(Kt, r, 2 * c + 1, hi);
        } else {
            put8(Kt, r, c, R.v[u][0]);
            put8(Kt, r, c + 32, R.v[u][1]);
        }
        if (c == 0) flags[r] = (R.ok >> u) & 1u;
    }
    put8(Kt, hw + 8 * (c >> 3), kDN / 8 + (c & 7), R.rp);
    // Rows of invalid slots (a range's last tile, CSA padding: rare, wave-uniform test) are
    // overwritten with zeros, so that codes read from row 0 -- NaN ones included -- never reach the
    // products.  (Clearing the registers before the conversion instead was computed ahead of the
    // test for every tile.)
    if (__builtin_amdgcn_ballot_w64(R.ok != 0xfu)) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if ((R.ok >> u) & 1u) continue;
            const int r = hw + 8 * u;
            if constexpr (FMT == LCA_FP8) {
                put8(Kt, r, 2 * c, z);
                put8(Kt, r, 2 * c + 1, z);
            } else {
                put8(Kt, r, c, z);
                put8(Kt, r, c + 32, z);
            }
        }
        if (!((R.ok >> (c >> 3)) & 1u)) put8(Kt, hw + 8 * (c >> 3), kDN / 8 + (c & 7), z);
    }
}

// Tile row trow (if in [0, 32)) is the query row's own window row: after dec_store, the threads that
// wrote it (half-wave hw = trow mod 8) overwrite it with rowt (bf16, decoded), the row the launch
// computes and stores itself (the ring does not hold it yet when the tile's loads are issued).
template <int FMT>
__device__ __forceinline__ void dec_fix_row(uint16_t* Kt, int hw, int c, const uint16_t* rowt, int trow) {
    if ((unsigned)trow >= (unsigned)kKT || hw != (trow & 7)) return;
    const u32x4* src = (const u32x4*)rowt;  // 8 bf16 per chunk
    if constexpr (FMT == LCA_FP8) {
        put8(Kt, trow, 2 * c, src[2 * c]);
        put8(Kt, trow, 2 * c + 1, src[2 * c + 1]);
    } else {
        put8(Kt, trow, c, src[c]);
        put8(Kt, trow, c + 32, src[c + 32]);
    }
    if ((c >> 3) == (trow >> 3)) put8(Kt, trow, kDN / 8 + (c & 7), src[kDN / 8 + (c & 7)]);
}

// Grid (x, T, B): query row i = blockIdx.y of sequence b = blockIdx.z, so the row's position
// comes from the first batch of argument loads.  Along x (a multiple of 8 workgroups, so x mod 8
// is the XCD): x = 8 j + xcd, head group j mod ng, split (j / ng) * 8 + xcd.
// MT: tiles per split of the launch (its longest split): the tile loop is unrolled for exactly MT
// tiles and prefetches NPE = min(NP, MT) ahead, so no load is issued for a tile past the split's
// end (the launch picks MT from the plan).
template <int FMT, bool DENSE, int NP, int MT>
__global__ void __launch_bounds__(256) attn_dec(AttnArgs a, int64_t split_len, int nsplit) {
    constexpr int NPE = NP < MT ? NP : MT;
    __shared__ __attribute__((aligned(16))) uint16_t Kt[3][kTileElems];
    __shared__ __attribute__((aligned(16))) f32x4 Sx[2][4][2][64];  // partial scores, two tiles
    __shared__ uint32_t vflag[3][kKT / 4];
    __shared__ int32_t ent[DENSE ? 1 : kDecMaxLen];

    // Every argument the prologue needs is read here, before the first branch: the scalar loads
    // then go out together instead of as a chain of dependent round trips.
    const int b = blockIdx.z, ri = blockIdx.y;
    const int64_t rowid = (int64_t)b * gridDim.y + ri;
    const int H = a.H;
    {
        const int64_t qp = a.q_pos.v[b], wb = a.w_base.v[b], cc = a.comp.cap, wc = a.win.cap;
        const int msh = a.m_shift, mm = a.m, kk = a.k, nw = a.n_win;
        const void *pq = a.q, *pi = a.idx, *pn0 = a.comp.nope, *pn1 = a.win.nope, *pr0 = a.comp.rope,
                   *pr1 = a.win.rope, *ps0 = a.comp.scale, *ps1 = a.win.scale, *pax = a.app_x, *pag = a.app_gamma;
        const float aeps = a.app_eps;
        const int64_t ast = a.app_stride;
        asm volatile("" ::"s"(qp), "s"(wb), "s"(cc), "s"(wc), "s"(msh), "s"(mm), "s"(kk), "s"(nw), "s"(H), "s"(pq),
                     "s"(pi), "s"(pn0), "s"(pn1), "s"(pr0), "s"(pr1), "s"(ps0), "s"(ps1), "s"(pax), "s"(pag),
                     "s"(aeps), "s"(ast));
    }
    const uint32_t ng = ((uint32_t)H + 15) >> 4;  // head groups (the last may be partial)
    const uint32_t L = blockIdx.x, jj = L >> 3;
    const int hg = (int)(jj % ng);
    const int split = (int)((jj / ng) * 8u + (L & 7u));
    if (split >= nsplit) return;
    int64_t t;
    const SlotMap sm = slot_map(a, b, ri, &t);
    // slot bookkeeping in 32 bits (slot counts and ring rows are below 2^31)
    const int s_begin = split * (int)split_len;
    const int s_end = (int)min(sm.nslots, (int64_t)s_begin + split_len);
    const int ntile = s_end > s_begin ? (s_end - s_begin + kKT - 1) / kKT : 0;
    const int ncs = (int)sm.ncs, w_row = (int)sm.w_row;
    const int vis = (int)sm.vis, win_cap = (int)a.win.cap;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, g4 = lane >> 4;  // MFMA lane coordinates
    const int hw = tid >> 5, c = tid & 31;     // gather coordinates
    const int h0 = 16 * hg;
    const bool hv = h0 + n < H;  // this lane's head exists (a partial last group: zero queries, no stores)

    // Q^T fragments for this wave's score dims: B[k = dim d0 + 32 ks + 8 g4 + e][n = head h0 + n]
    const int d0 = wv < 2 ? 160 * wv : 320 + 128 * (wv - 2);
    const int nks = wv < 2 ? 5 : 4;
    bf16x8 qf[5];
    {
        const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + (rowid * a.H + (hv ? h0 + n : 0)) * kC + d0);
#pragma unroll
        for (int ks = 0; ks < 5; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, ks < nks && hv ? qp[4 * ks + g4] : u32x4{0u, 0u, 0u, 0u});
    }
    if constexpr (!DENSE) {  // this split's entry ids
        const int lim = min(ncs, s_end);
        const int nent = lim > s_begin ? lim - s_begin : 0;
        const GMEM int32_t* irow = sptr<int32_t>(a.idx) + rowid * a.k + s_begin;
        for (int i = tid; i < nent; i += 256) ent[i] = irow[i];
        __syncthreads();
    }

    constexpr int64_t kRowBytes = FMT == LCA_FP8 ? kDN : 2 * kDN;
    KvPtrs P;
    P.nope[0] = sptr<uint8_t>(a.comp.nope) + (int64_t)b * a.comp.cap * kRowBytes;
    P.nope[1] = sptr<uint8_t>(a.win.nope) + (int64_t)b * a.win.cap * kRowBytes;
    P.rope[0] = sptr<uint16_t>(a.comp.rope) + (int64_t)b * a.comp.cap * kDR;
    P.rope[1] = sptr<uint16_t>(a.win.rope) + (int64_t)b * a.win.cap * kDR;
    P.scale[0] = FMT == LCA_FP8 ? sptr<float>(a.comp.scale) + (int64_t)b * a.comp.cap * 4 : nullptr;
    P.scale[1] = FMT == LCA_FP8 ? sptr<float>(a.win.scale) + (int64_t)b * a.win.cap * 4 : nullptr;

    // Fused window store (T = 1): the split holding the last slot -- the query row's own window
    // slot -- computes that row from the raw row (the compressor's m = 1 store) into rowt, and head
    // group 0 also writes it to the ring.  Its loads go out first, with the tiles'.
    __shared__ __attribute__((aligned(16))) uint16_t rowt[kC];
    __shared__ float rys[64 * 9];
    const bool app = a.app_x != nullptr && s_begin < s_end && s_end == (int)sm.nslots && sm.nslots > sm.ncs;
    RowOut<9> arow;
    // The 32-bit words holding this lane's channels lane + 64 j (the high half for odd lanes), taken
    // apart only when the row is prepared, after the tile loads are issued: any use here would make
    // the wave wait for these loads before the tiles' went out.
    uint32_t xr[9];
    float ag[9];
    double ainv = 0.0;  // RoPE frequency of this lane's pair (channel 512 + lane, d_rope = 64)
    if (app && wv == 0) {
        const uint32_t* xp = (const uint32_t*)((const uint16_t*)a.app_x + (int64_t)b * a.app_stride * kC);
#pragma unroll
        for (int j = 0; j < 9; ++j) xr[j] = xp[(lane + 64 * j) >> 1];
        if (a.app_gamma)
#pragma unroll
            for (int j = 0; j < 9; ++j) ag[j] = a.app_gamma[lane + 64 * j];
        ainv = a.rope.inv[lane & 31];
    }
    const int tl = app ? (int)sm.nslots - 1 - s_begin : -(1 << 30);  // tile row of slot t in tile 0

    // (loads of tiles past the end read row 0 and are dropped: the same loads on every path)
    DecRegs<FMT> R[NPE];
#pragma unroll
    for (int j = 0; j < NPE; ++j) {
        dec_load<FMT, DENSE>(R[j], ncs, w_row, s_end, vis, win_cap, P, ent, s_begin, s_begin + j * kKT, hw, c);
        // (tile by tile, in the order the loop consumes them: the loop's waits count on it)
        asm volatile("" ::: "memory");
    }
    constexpr uint32_t kTileBytes = 2 * kTileElems;
    uint32_t bq = 0, bn = kTileBytes, bo = 2 * kTileBytes;  // byte offsets: tiles t, t + 1, t - 1
    int fq = 0, fn = 1;
    if (app) {  // (the ring store waits for the epilogue: a global store here would make this barrier
                // wait for every tile load in flight)
        if (wv == 0) {
            const uint32_t sh = (lane & 1) ? 0u : 16u, mask = (lane & 1) ? 0xffff0000u : 0xffffffffu;
#pragma unroll
            for (int j = 0; j < 9; ++j) {  // bf16 -> f32 (in asm: the compiler would move it up to the loads)
                float f;
                asm volatile("v_lshlrev_b32 %0, %1, %2\n\tv_and_b32 %0, %3, %0" : "=&v"(f) : "v"(sh), "v"(xr[j]), "v"(mask));
                arow.y[j] = f;
            }
            row_prepare<FMT, 9>(arow, ag, a.app_gamma, a.app_eps, kC, kDN, kDR, a.rope_theta != 0.0, ainv, (double)t,
                                rys, rowt);
        }
        __syncthreads();
    }
    dec_store<FMT>(R[0], &Kt[0][0], (uint8_t*)vflag[0], hw, c);
    if (app) dec_fix_row<FMT>(&Kt[0][0], hw, c, rowt, tl);
    if (NPE < MT)
        dec_load<FMT, DENSE>(R[0], ncs, w_row, s_end, vis, win_cap, P, ent, s_begin, s_begin + NPE * kKT, hw, c);
#pragma unroll
    for (int ks = 0; ks < 5; ++ks) asm volatile("" ::"v"(qf[ks]));
    __syncthreads();

    f32x4 o[9];
#pragma unroll
    for (int nb = 0; nb < 9; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = -INFINITY, lpart = 0.0f;
    const float qk_scale = a.sm_scale * kLog2e;
    const int koff = n * kKS + d0 + 8 * g4;
    const int dbase = 144 * wv;
    const uint32_t vbase = lds_addr(&Kt[0][0]) + 2 * ((4 * g4 + (n >> 2)) * kKS + dbase + 4 * (n & 3));

    // The tile loop is unrolled in full (MT tiles): with no back edge the compiler counts the loads
    // in flight exactly, and tile t + 1 waits only for its own rows.
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        {
            if (t >= ntile) break;
            // partial scores of tile t over this wave's dims
            f32x4 s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
            {
                const uint16_t* kr = (const uint16_t*)((const char*)&Kt[0][0] + bq) + koff;
#pragma unroll
                for (int ks = 0; ks < 5; ++ks) {
                    if (ks < nks) {
                        const bf16x8 k0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr + 32 * ks));
                        const bf16x8 k1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr + 16 * kKS + 32 * ks));
                        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s[0], 0, 0, 0);
                        s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s[1], 0, 0, 0);
                    }
                }
            }
            Sx[t & 1][wv][0][lane] = s[0];
            Sx[t & 1][wv][1][lane] = s[1];
            // tile t + 1 into the buffer tile t - 2 used; its registers take tile t + 1 + NP (after
            // the last tile: a harmless store of dropped rows into the free buffer)
            if (t + 1 < MT) {
                DecRegs<FMT>& Rn = R[(t + 1) % NPE];
                dec_store<FMT>(Rn, (uint16_t*)((char*)&Kt[0][0] + bn), (uint8_t*)vflag[fn], hw, c);
                if (app) dec_fix_row<FMT>((uint16_t*)((char*)&Kt[0][0] + bn), hw, c, rowt, tl - (t + 1) * kKT);
                if (t + 1 + NPE < MT)
                    dec_load<FMT, DENSE>(Rn, ncs, w_row, s_end, vis, win_cap, P, ent, s_begin,
                                         s_begin + (t + 1 + NPE) * kKT, hw, c);
            }
            __syncthreads();
            // the four partial sums in a fixed order: identical scores in every wave
            f32x4 sc0 = Sx[t & 1][0][0][lane], sc1 = Sx[t & 1][0][1][lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                sc0 += Sx[t & 1][w][0][lane];
                sc1 += Sx[t & 1][w][1][lane];
            }
            {
                const uint32_t f0 = vflag[fq][g4], f1 = vflag[fq][4 + g4];
                if (__builtin_amdgcn_ballot_w64((f0 & f1) != 0x01010101u)) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (!((f0 >> (8 * i)) & 1u)) sc0[i] = -INFINITY;
                        if (!((f1 >> (8 * i)) & 1u)) sc1[i] = -INFINITY;
                    }
                }
            }
            const float smax = fmaxf(fmaxf(fmaxf(sc0[0], sc0[1]), fmaxf(sc0[2], sc0[3])),
                                     fmaxf(fmaxf(sc1[0], sc1[1]), fmaxf(sc1[2], sc1[3])));
            const float tmax = max4g(smax) * qk_scale;
            const bool grow = __builtin_amdgcn_ballot_w64(tmax > mrun + 8.0f) != 0;  // lazy rescale, as attn_mfma
            const float mnew = grow ? fmaxf(mrun, tmax) : mrun;
            const float corr = mnew == mrun ? 1.0f : exp2f(mrun - mnew);
            mrun = mnew;
            const float mneg = mrun == -INFINITY ? 0.0f : -mrun;
            float p[2][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[0][i] = __builtin_amdgcn_exp2f(fmaf(sc0[i], qk_scale, mneg));
                p[1][i] = __builtin_amdgcn_exp2f(fmaf(sc1[i], qk_scale, mneg));
            }
            lpart = lpart * corr +
                    (((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3])));
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float x0 = p[kb][2 * q], x1 = p[kb][2 * q + 1];
                    const uint32_t hb = pk_bf16(x0, x1);
                    ph[2 * kb + q] = hb;
                    pl[2 * kb + q] = pk_bf16(x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u));
                }
            const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
            if (grow) {
                asm volatile("");
#pragma unroll
                for (int nb = 0; nb < 9; ++nb) o[nb] *= corr;
            }
            {
                const uint32_t vr = vbase + bq;
#pragma unroll
                for (int nb = 0; nb < 9; ++nb) {
                    const s16x4 w0 = lds_tr16(vr + 32 * nb);
                    const s16x4 w1 = lds_tr16(vr + 32 * kKS + 32 * nb);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pa, o[nb], 0, 0, 0);
                    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[nb], 0, 0, 0);
                }
            }
            const uint32_t bt = bo;
            bo = bq;
            bq = bn;
            bn = bt;
            fq = fn;
            fn = fn == 2 ? 0 : fn + 1;
        }
    }
    const float lrun = sum4g(lpart);
    if (app && hg == 0 && wv == 0) {  // the query row's window row into the ring
        int trw = w_row + ((int)sm.nslots - 1 - ncs);  // ring row of position t
        if (trw >= win_cap) trw -= win_cap;
        row_commit<FMT, 9>(arow, kC, kDN, kDR, a.win.nope, a.win.rope, a.win.scale, (int64_t)b * win_cap + trw);
    }

    // epilogue: head h = h0 + n, dims dbase + 16 nb + 4 g4 + i
    const int h = h0 + n;
    const int64_t nrows = (int64_t)a.B * a.T;
    if (!hv) return;
    if (nsplit > 1) {
        float* wo = (float*)a.ws;
        float* wml = wo + (int64_t)nsplit * nrows * a.H * kC;
        const int64_t pr = ((int64_t)split * nrows + rowid) * a.H + h;
        float* dst = wo + pr * kC + dbase + 4 * g4;
        // non-temporal: the merge launch reads them once; written through now, they are not left
        // dirty in L2 for the end of the launch to write back
#pragma unroll
        for (int nb = 0; nb < 9; ++nb) __builtin_nontemporal_store(o[nb], (f32x4*)(dst + 16 * nb));
        if (g4 == 0 && wv == 0) {
            __builtin_nontemporal_store(mrun, wml + 2 * pr);
            __builtin_nontemporal_store(lrun, wml + 2 * pr + 1);
        }
        return;
    }
    float mu = mrun, den = lrun;
    if (a.sink) {
        const float z = a.sink[h] * kLog2e;
        mu = fmaxf(mrun, z);
        den = (mrun == -INFINITY ? 0.0f : lrun * exp2f(mrun - mu)) + exp2f(z - mu);
    }
    const float f = den > 0.0f && mrun != -INFINITY ? exp2f(mrun - mu) / den : 0.0f;
#pragma unroll
    for (int nb = 0; nb < 9; ++nb) o[nb] *= f;
    // output RoPE by -t: wave 3 holds dims 432 ..; 512 + j and 544 + j (j = 16 q2 + 4 g4 + i) are
    // blocks 5 + q2 and 7 + q2
    if (a.rope_theta != 0.0 && wv == 3) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sn, cs;
                rope_sincos(a.rope.inv, 16 * q2 + 4 * g4 + i, -(double)t, &sn, &cs);
                const float x0 = o[5 + q2][i], x1 = o[7 + q2][i];
                o[5 + q2][i] = x0 * cs - x1 * sn;
                o[7 + q2][i] = x0 * sn + x1 * cs;
            }
    }
    const int64_t orow = (rowid * a.H + h) * kC + dbase + 4 * g4;
    if (a.out_dtype == LCA_F32) {
        float* dst = (float*)a.out + orow;
#pragma unroll
        for (int nb = 0; nb < 9; ++nb) *(f32x4*)(dst + 16 * nb) = o[nb];
    } else {
        uint16_t* dst = (uint16_t*)a.out + orow;
#pragma unroll
        for (int nb = 0; nb < 9; ++nb) {
            uint2 w;
            w.x = (uint32_t)f2bf(o[nb][0]) | ((uint32_t)f2bf(o[nb][1]) << 16);
            w.y = (uint32_t)f2bf(o[nb][2]) | ((uint32_t)f2bf(o[nb][3]) << 16);
            *(uint2*)(dst + 16 * nb) = w;
        }
    }
    if (a.lse && g4 == 0 && wv == 0)
        a.lse[rowid * a.H + h] = den > 0.0f ? (mu + log2f(den)) * kLn2 : -INFINITY;
}

// f32 caches: one wave per (row, head); lane owns dims lane + 64 u.
__global__ void __launch_bounds__(64) attn_f32(AttnArgs a) {
    const int64_t rowid = blockIdx.x;
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    int b, ri;
    row_coords(a, rowid, &b, &ri);
    int64_t t;
    const SlotMap sm = slot_map(a, b, ri, &t);
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

// Split policy.  Short launches (rows x head groups <= kDecMaxUnits) take attn_dec: the slot list
// is cut into ns_t = kDecTargetWGs / (rows x head groups) splits of whole tiles (32 .. kDecMaxLen
// slots), so that the launch comes near kDecTargetWGs workgroups.  Other launches of fewer than kDecRows
// rows take attn_mfma (64 heads per workgroup, which amortises each gathered tile over four times
// the work) with up to ceil(256 / rows) splits of at least 128 slots; longer launches one split
// per row.  Either way the split count never exceeds a bound that does not fall as max_keys grows
// (dec: max(ns_t, ceil(max_keys / kDecMaxLen)); split: ceil(256 / rows)), which the workspace size
// for "at most max_keys" rows uses.
constexpr int kDecMaxUnits = 64;
struct AttnPlan {
    bool dec;
    int nsplit;
    int64_t len;  // slots per split
};
static int64_t head_groups(int32_t H) { return ((int64_t)H + 15) / 16; }  // (the last may be partial)
static bool dec_eligible(int64_t rows, int32_t H, int32_t c) {
    return c == kC && H >= 1 && rows * head_groups(H) <= kDecMaxUnits;
}
static bool split_eligible(int64_t rows, int32_t c) { return c == kC && rows < kDecRows; }
static int64_t dec_target(int64_t rows, int32_t H) {
    const int64_t per = rows * head_groups(H);  // workgroups per split index
    return per >= kDecTargetWGs ? 1 : kDecTargetWGs / per;
}
static int64_t split_target(int64_t rows) { return (kDecWGs + rows - 1) / rows; }
static AttnPlan attn_plan(int64_t rows, int32_t H, int32_t c, int64_t max_keys) {
    AttnPlan p = {false, 1, (max_keys + kKT - 1) / kKT * kKT};
    if (dec_eligible(rows, H, c)) {
        const int64_t nt = dec_target(rows, H);
        int64_t len = (max_keys + nt - 1) / nt;
        len = (len + kKT - 1) / kKT * kKT;
        if (len < kKT) len = kKT;
        if (len > kDecMaxLen) len = kDecMaxLen;
        int64_t ns = (max_keys + len - 1) / len;
        if (ns < 1) ns = 1;
        if (ns <= 1024) {  // (the merge keeps the split weights in LDS)
            p.dec = true;
            p.nsplit = (int)ns;
            p.len = len;
        }
        return p;
    }
    if (split_eligible(rows, c) && max_keys > 128) {
        int64_t want = split_target(rows);
        const int64_t most = (max_keys + 127) / 128;
        if (want > most) want = most;
        if (want > 1024) want = 1024;
        int64_t len = (max_keys + want - 1) / want;
        len = (len + kKT - 1) / kKT * kKT;
        p.nsplit = (int)((max_keys + len - 1) / len);
        p.len = len;
    }
    return p;
}

size_t attn_ws_need(int64_t rows, int32_t H, int32_t c, int64_t max_keys) {
    const AttnPlan p = attn_plan(rows, H, c, max_keys);
    if (p.nsplit <= 1) return 0;
    return (size_t)p.nsplit * rows * H * (c + 2) * sizeof(float);
}

size_t attn_ws_bytes(int64_t rows, int32_t H, int32_t c, int64_t max_keys) {
    int64_t ns = 1;
    if (dec_eligible(rows, H, c)) {
        ns = dec_target(rows, H);
        const int64_t hi = (max_keys + kDecMaxLen - 1) / kDecMaxLen;
        if (hi > ns) ns = hi;
    } else if (split_eligible(rows, c)) {
        ns = split_target(rows);
    }
    if (ns > 1024) ns = 1024;
    if (ns <= 1) return 0;
    return (size_t)ns * rows * H * (c + 2) * sizeof(float);
}

// Expansion of fp8 rows to bf16: 8 rows per 256-thread block; thread (row r = tid / 32, lane c)
// expands nope codes 16c .. 16c+15 (two 16-byte bf16 stores), lanes c < 8 copy RoPE chunk c.
__global__ void __launch_bounds__(256) kv_expand(ExpandArgs a) {
    const int b = blockIdx.y;
    const int r = threadIdx.x >> 5, c = threadIdx.x & 31;
    const int64_t i = (int64_t)blockIdx.x * 8 + r;
    if (i >= a.count.v[b]) return;
    const int64_t p = a.first.v[b] + i;
    const int64_t sr = (int64_t)b * a.src.cap + p % a.src.cap;
    const int64_t dr = (int64_t)b * a.dst.cap + p % a.dst.cap;
    const u32x4 codes = ((const u32x4*)((const uint8_t*)a.src.nope + sr * kDN))[c];
    const float sc = ((const float*)a.src.scale)[sr * 4 + (c >> 3)];
    u32x4 lo, hi;
    lo[0] = fp8x2_bf16<false>(codes[0], sc);
    lo[1] = fp8x2_bf16<true>(codes[0], sc);
    lo[2] = fp8x2_bf16<false>(codes[1], sc);
    lo[3] = fp8x2_bf16<true>(codes[1], sc);
    hi[0] = fp8x2_bf16<false>(codes[2], sc);
    hi[1] = fp8x2_bf16<true>(codes[2], sc);
    hi[2] = fp8x2_bf16<false>(codes[3], sc);
    hi[3] = fp8x2_bf16<true>(codes[3], sc);
    u32x4* dn = (u32x4*)((uint16_t*)a.dst.nope + dr * kDN);
    dn[2 * c] = lo;
    dn[2 * c + 1] = hi;
    if (c < 8) ((u32x4*)((uint16_t*)a.dst.rope + dr * kDR))[c] = ((const u32x4*)((const uint16_t*)a.src.rope + sr * kDR))[c];
}

hipError_t launch_kv_expand(const ExpandArgs& a, hipStream_t st) {
    if (a.max_count <= 0) return hipSuccess;
    if (trace_on()) trace("  kv_expand: grid (%lld, %d) x 256, fp8 rows -> bf16", (long long)((a.max_count + 7) / 8), a.B);
    hipLaunchKernelGGL(kv_expand, dim3((unsigned)((a.max_count + 7) / 8), (unsigned)a.B), dim3(256), 0, st, a);
    return hipGetLastError();
}

// attn_dec for fp8 rows, unrolled for the launch's tile count mt
template <int FMT, bool DENSE, int NP>
static void launch_dec(int mt, dim3 grid, hipStream_t st, const AttnArgs& a, int64_t len, int ns) {
    static_assert(kDecMaxTiles == 8, "one instantiation per tile count");
    switch (mt) {
        case 1: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 1>), grid, dim3(256), 0, st, a, len, ns); break;
        case 2: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 2>), grid, dim3(256), 0, st, a, len, ns); break;
        case 3: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 3>), grid, dim3(256), 0, st, a, len, ns); break;
        case 4: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 4>), grid, dim3(256), 0, st, a, len, ns); break;
        case 5: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 5>), grid, dim3(256), 0, st, a, len, ns); break;
        case 6: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 6>), grid, dim3(256), 0, st, a, len, ns); break;
        case 7: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 7>), grid, dim3(256), 0, st, a, len, ns); break;
        default: hipLaunchKernelGGL((attn_dec<FMT, DENSE, NP, 8>), grid, dim3(256), 0, st, a, len, ns); break;
    }
}

// (the decode kernel is taken and its row offsets fit 32 bits)
static bool dec_launch(const AttnArgs& a, const AttnPlan& p) {
    const int64_t rb = a.comp.fmt == LCA_FP8 ? kDN : 2 * kDN;
    const bool off32 = a.comp.cap * rb < ((int64_t)1 << 32) && a.win.cap * rb < ((int64_t)1 << 32);
    return p.dec && off32;
}

bool attn_fuses_store(const AttnArgs& a) {
    if (a.comp.fmt == LCA_F32 || a.T != 1 || a.n_win < 1) return false;
    const int c = a.comp.d_nope + a.comp.d_rope;
    return dec_launch(a, attn_plan((int64_t)a.B * a.T, a.H, c, a.max_keys));
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.T;
    if (rows <= 0) return hipSuccess;
    const int c = a.comp.d_nope + a.comp.d_rope;
    if (a.comp.fmt == LCA_F32) {
        if (trace_on()) trace("  attn_f32: grid (%lld, %d) x 64", (long long)rows, a.H);
        hipLaunchKernelGGL(attn_f32, dim3((unsigned)rows, (unsigned)a.H), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    const AttnPlan p = attn_plan(rows, a.H, c, a.max_keys);
    const int ns = p.nsplit;
    const bool dense = a.idx == nullptr;
    // attn_dec addresses one sequence's rows with 32-bit offsets; larger planes take attn_mfma
    // (same splits, same workspace layout)
    if (dec_launch(a, p)) {
        dim3 grid((unsigned)((ns + 7) / 8 * 8 * head_groups(a.H)), (unsigned)a.T, (unsigned)a.B);
        if (trace_on())
            trace("  attn_dec<%s, %s>: grid (%u, %u, %u) x 256, %d split(s) of %lld slots (%lld tiles)%s", a.comp.fmt == LCA_FP8 ? "fp8" : "bf16",
                  dense ? "dense" : "selected", grid.x, grid.y, grid.z, ns, (long long)p.len,
                  (long long)((p.len + kKT - 1) / kKT), a.app_x ? ", window store fused" : "");
        const int mt = (int)((p.len + kKT - 1) / kKT);  // (1 .. kDecMaxTiles)
        if (a.comp.fmt == LCA_FP8) {
            if (dense) launch_dec<LCA_FP8, true, 4>(mt, grid, st, a, p.len, ns);
            else launch_dec<LCA_FP8, false, 4>(mt, grid, st, a, p.len, ns);
        } else {  // (bf16 rows: one tile count)
            if (dense) hipLaunchKernelGGL((attn_dec<LCA_BF16, true, 3, kDecMaxTiles>), grid, dim3(256), 0, st, a, p.len, ns);
            else hipLaunchKernelGGL((attn_dec<LCA_BF16, false, 3, kDecMaxTiles>), grid, dim3(256), 0, st, a, p.len, ns);
        }
    } else {
        dim3 grid((unsigned)rows, (unsigned)ns);
        if (trace_on())
            trace("  attn_mfma<%s, %s>: grid (%u, %u) x 512, %d split(s) of %lld slots", a.comp.fmt == LCA_FP8 ? "fp8" : "bf16",
                  dense ? "dense" : "selected", grid.x, grid.y, ns, (long long)p.len);
        if (a.comp.fmt == LCA_FP8) {
            if (dense) hipLaunchKernelGGL((attn_mfma<LCA_FP8, true>), grid, dim3(512), 0, st, a, p.len, ns);
            else hipLaunchKernelGGL((attn_mfma<LCA_FP8, false>), grid, dim3(512), 0, st, a, p.len, ns);
        } else {
            if (dense) hipLaunchKernelGGL((attn_mfma<LCA_BF16, true>), grid, dim3(512), 0, st, a, p.len, ns);
            else hipLaunchKernelGGL((attn_mfma<LCA_BF16, false>), grid, dim3(512), 0, st, a, p.len, ns);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns <= 1) return e;
    const int groups = comb_groups(ns);
    if (trace_on()) trace("  attn_combine: %d split(s), %d group(s)", ns, groups);
    if (groups == 1) {
        hipLaunchKernelGGL(attn_combine, dim3((unsigned)a.T, (unsigned)a.H, (unsigned)a.B),
                           dim3(kCombQuarters * kCombPer), 0, st, a, ns, 1);
    } else {
        const int ct = groups * kCombPer;
        hipLaunchKernelGGL(attn_combine, dim3((unsigned)a.T, (unsigned)(a.H * kCombQuarters), (unsigned)a.B),
                           dim3(ct < 64 ? 64 : ct), 0, st, a, ns, 0);
    }
    return hipGetLastError();
}

}  // namespace lca
