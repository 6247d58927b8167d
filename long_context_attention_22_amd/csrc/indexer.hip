// indexer.hip -- the lightning indexer ("DeepSeek-V4 中文翻译" section 2.3.1;
// BF16 index scores, section 5.2.1):
//   S[t][s] = sum_h w[t][h] * ReLU(q_I[t][h] . k_I[s])  for s < vis(t).
//
// bf16 path (H_I = 16, d_I = 128): a bf16 MFMA contraction.  The 16 heads of
// one query token are the M = 16 rows of v_mfma_f32_16x16x32_bf16, 16 keys
// are its N columns and d_I = 128 is four K = 32 steps.  Each wave keeps the
// A fragments of TOK tokens in registers and streams 64-key chunks of the key
// cache straight from HBM into B fragments (each lane loads 16 contiguous
// bytes of one key row, so a chunk is one contiguous 16 KB read).  The
// epilogue applies ReLU and the head weights in the accumulator layout, sums
// the 16 heads of four 16-key blocks at once with a reduce-scatter over the
// lane rows (two v_permlane16_swap, one v_permlane32_swap) and writes 64 consecutive scores
// per token with one coalesced store.  Key chunks beyond the last token's
// visible count are skipped (causal tile skip).
//
// MXFP4 path (section 5.2.1: the QK path in FP4): the keys are stored MXFP4
// (64 bytes of E2M1 codes and 4 E8M0 scale bytes per key) and every query
// head is quantised to MXFP4 in the prologue.  One
// v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 A and B covers 16 heads x 16 keys
// x d_I = 128: lane l supplies head (A) or key (B) l & 15, elements
// [32 (l >> 4), +32) as 16 bytes of packed codes, and that block's scale byte.
// Same grid, epilogue and causal skip as the bf16 path.
//
// f32 path: one thread per (token, key), f32 FMA (used for fp32 workloads).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace lca {

constexpr int kIdxH = 16, kIdxD = 128;

template <typename TS>
__device__ __forceinline__ void store_score(TS* p, float v);
template <>
__device__ __forceinline__ void store_score<float>(float* p, float v) {
    *p = v == 0.0f ? 0.0f : v;
}
template <>
__device__ __forceinline__ void store_score<uint16_t>(uint16_t* p, float v) {
    *p = f2bf(v == 0.0f ? 0.0f : v);
}

// High byte of the top-k's monotone key of a stored bf16 score h (the bits store_score writes, -0
// stored as +0): positive scores map to 0x80.. and up, negative ones below.
__device__ __forceinline__ uint32_t key_high_of_bits(uint32_t h) {
    const uint32_t key = (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
    return key >> 8;
}

// A score's store and, with the fused top-k pass on, its count in the LDS histogram hist (bf16 scores).
template <typename TS>
__device__ __forceinline__ void store_count(TS* p, float v, uint32_t* hist, bool count) {
    if constexpr (std::is_same<TS, uint16_t>::value) {
        const uint32_t h = f2bf(v == 0.0f ? 0.0f : v);
        *p = (uint16_t)h;
        if (count) atomicAdd(&hist[key_high_of_bits(h)], 1u);
    } else {
        store_score<TS>(p, v);
    }
}

// The fused top-k pass's LDS histograms (one per token of the workgroup) into the top-k's workspace:
// row (b, i) at th_h1 + (b T + i) th_row, plus (key_lo / kTopkChunk) kTopkHistWords in 16-bit counts
// when the top-k takes its chunked (split) schedule, else 32-bit counts.  Only nonzero bins cost a
// device atomic.
template <int TOK>
__device__ __forceinline__ void flush_hist(const uint32_t* hist, uint32_t* th_h1, int64_t th_row, int th_chunked,
                                           int64_t row0, int ntok, int64_t key_lo) {
    __syncthreads();
    const int bin = threadIdx.x;
    const int64_t off = th_chunked ? (key_lo >> kTopkChunkLog2) * kTopkHistWords + (bin >> 1) : bin;
    const int sh = th_chunked ? 16 * (bin & 1) : 0;
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        const uint32_t c = hist[tk * 256 + bin];
        if (tk < ntok && c) atomicAdd(th_h1 + (row0 + tk) * th_row + off, c << sh);
    }
}

// (visible count (t + 1) / m: a shift when m is a power of two)
__device__ __forceinline__ int64_t vis_of(int64_t t1, int m) {
    return (m & (m - 1)) == 0 ? t1 >> __builtin_ctz((unsigned)m) : t1 / m;
}

// the visible counts of TOK consecutive tokens, min(vis, k_cap), 0 past the last token; uniform,
// so kept in scalar registers for the key loop
template <int TOK>
__device__ __forceinline__ void token_vis(int64_t (&vis)[TOK], int64_t pos0, int ntok, int m, int64_t k_cap) {
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        const int64_t v = tk < ntok ? min(vis_of(pos0 + tk + 1, m), k_cap) : 0;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
        vis[tk] = (int64_t)(((uint64_t)hi << 32) | lo);
    }
}

// HIST: the fused top-k pass is on (bf16 scores; a.th_h1 set).  (Two waves per SIMD: the register budget
// the 8-token form has to fit, 256 per lane.)
template <int TOK, typename TS, bool HIST>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) indexer_mfma(IndexerArgs a,
                                                                                           int64_t keys_per_wg) {
    const int b = blockIdx.z;
    const int i0 = blockIdx.y * TOK;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // the arguments in one batch of scalar loads, before the first branch
    const int T = a.T, m = a.m;
    const int64_t p0 = a.q_pos.v[b], k_cap = a.k_cap, s_stride = a.s_stride;
    const void *pq = a.q, *pk = a.k, *psc = a.scores;
    const float* pw = a.w;
    uint32_t* th_h1 = a.th_h1;
    const int64_t th_row = a.th_row;
    const int th_chunked = a.th_chunked;
    asm volatile("" ::"s"(T), "s"(m), "s"(p0), "s"(k_cap), "s"(s_stride), "s"(pq), "s"(pk), "s"(psc), "s"(pw),
                 "s"(th_h1), "s"(th_row), "s"(th_chunked));
    const int ntok = min(TOK, T - i0);
    const int64_t pos0 = p0 + i0;
    const int64_t vis_last = min(vis_of(pos0 + ntok, m), k_cap);
    const int64_t key_lo = (int64_t)blockIdx.x * keys_per_wg;
    const int64_t key_hi = min(key_lo + keys_per_wg, vis_last);
    if (key_lo >= key_hi) return;
    // fused top-k pass: high-byte histograms of this workgroup's stored scores, one per token
    static_assert(!HIST || std::is_same<TS, uint16_t>::value, "the fused top-k pass needs bf16 scores");
    __shared__ uint32_t th_hist[HIST ? TOK * 256 : 1];
    constexpr bool hist = HIST;
    if (hist) {
#pragma unroll
        for (int tk = 0; tk < TOK; ++tk) th_hist[tk * 256 + threadIdx.x] = 0u;
        __syncthreads();
    }

    const int hrow = lane & 15, kgrp = lane >> 4;
    bf16x8 qa[TOK][4];
    float wt[TOK][4];
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        const int64_t qi = ((int64_t)b * a.T + i0 + tk) * kIdxH;
        const u32x4* qp = (const u32x4*)((const uint16_t*)a.q + (qi + hrow) * kIdxD);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 v = tk < ntok ? qp[4 * ks + kgrp] : u32x4{0u, 0u, 0u, 0u};
            qa[tk][ks] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wt[tk][r] = tk < ntok ? (a.w ? a.w[qi + 4 * kgrp + r] : 1.0f) : 0.0f;
    }

    const uint16_t* kbase = (const uint16_t*)a.k + (int64_t)b * a.k_cap * kIdxD;
    TS* sbase = (TS*)a.scores + ((int64_t)b * a.T + i0) * a.s_stride;

    int64_t vis_tk[TOK];  // visible keys of each token (loop invariant)
    token_vis<TOK>(vis_tk, pos0, ntok, m, k_cap);

    for (int64_t c0 = key_lo + 64 * wv; c0 < key_hi; c0 += 256) {
        // B fragments of four 16-key blocks: block bl, lane -> key c0 + 16 bl + (lane & 15).  With
        // several tokens the loads are branch-free: keys past the range re-read its last key.
        bf16x8 kf[4][4];
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
            const int64_t key = TOK > 1 ? min(c0 + 16 * bl + hrow, key_hi - 1) : c0 + 16 * bl + hrow;
            const u32x4* kp = (const u32x4*)(kbase + key * kIdxD);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4 v = (TOK > 1 || key < key_hi) ? kp[4 * ks + kgrp] : u32x4{0u, 0u, 0u, 0u};
                kf[bl][ks] = __builtin_bit_cast(bf16x8, v);
            }
        }
        const int64_t mykey = c0 + lane;  // the score this lane stores
        float mine_all[TOK];
#pragma unroll
        for (int tk = 0; tk < TOK; ++tk) {
            float part[4];
#pragma unroll
            for (int bl = 0; bl < 4; ++bl) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[tk][ks], kf[bl][ks], acc, 0, 0, 0);
                // lane holds heads 4*kgrp + r of key 16 bl + hrow
                float v = wt[tk][0] * fmaxf(acc[0], 0.0f);
                v = fmaf(wt[tk][1], fmaxf(acc[1], 0.0f), v);
                v = fmaf(wt[tk][2], fmaxf(acc[2], 0.0f), v);
                part[bl] = fmaf(wt[tk][3], fmaxf(acc[3], 0.0f), v);
            }
            // the four head quartets of each key: lane l gets key 16 (l >> 4) + (l & 15) = l
            const float mine = sum4g_scatter(part[0], part[1], part[2], part[3]);
            if (TOK == 1) {
                if (mykey < vis_tk[tk]) store_count<TS>(sbase + (int64_t)tk * a.s_stride + mykey, mine, th_hist, hist);
            }
            mine_all[tk] = mine;
        }
        // Several tokens: every key of the workgroup's range is stored for every token, after the
        // whole chunk (one masked region instead of one per token); a token's columns in
        // [vis(t), key_hi) hold scores of keys it cannot see, which the contract leaves unspecified
        // (and which the histograms do not count).
        if constexpr (TOK > 1) {
            if (mykey < key_hi) {
#pragma unroll
                for (int tk = 0; tk < TOK; ++tk)
                    if (tk < ntok)
                        store_count<TS>(sbase + (int64_t)tk * a.s_stride + mykey, mine_all[tk], th_hist + tk * 256,
                                        hist && mykey < vis_tk[tk]);
            }
        }
    }
    if (hist) flush_hist<TOK>(th_hist, th_h1, th_row, th_chunked, (int64_t)b * T + i0, ntok, key_lo);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// (through a parameter: a bit cast applied directly to a vector element subscript was compiled as a
// cast of element 0)
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }

// (at most 128 VGPRs: four waves per SIMD hide the key loads better than wider token pipelining)
// (the fused top-k pass's per-token histograms need more registers than the four-wave budget holds)
template <int TOK, typename TS, bool HIST>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HIST && TOK > 1 ? 2 : 4, 8)))
indexer_fp4(IndexerArgs a, int64_t keys_per_wg) {
    const int b = blockIdx.z;
    const int i0 = blockIdx.y * TOK;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int T = a.T, m = a.m;
    const int64_t p0 = a.q_pos.v[b], k_cap = a.k_cap, s_stride = a.s_stride;
    const void *pq = a.q, *pk = a.k, *pks = a.k_scale, *psc = a.scores;
    const float* pw = a.w;
    uint32_t* th_h1 = a.th_h1;
    const int64_t th_row = a.th_row;
    const int th_chunked = a.th_chunked;
    asm volatile("" ::"s"(T), "s"(m), "s"(p0), "s"(k_cap), "s"(s_stride), "s"(pq), "s"(pk), "s"(pks), "s"(psc),
                 "s"(pw), "s"(th_h1), "s"(th_row), "s"(th_chunked));
    const int ntok = min(TOK, T - i0);
    const int64_t pos0 = p0 + i0;
    const int64_t vis_last = min(vis_of(pos0 + ntok, m), k_cap);
    const int64_t key_lo = (int64_t)blockIdx.x * keys_per_wg;
    const int64_t key_hi = min(key_lo + keys_per_wg, vis_last);
    if (key_lo >= key_hi) return;
    // fused top-k pass (as in indexer_mfma)
    static_assert(!HIST || std::is_same<TS, uint16_t>::value, "the fused top-k pass needs bf16 scores");
    __shared__ uint32_t th_hist[HIST ? TOK * 256 : 1];
    constexpr bool hist = HIST;
    if (hist) {
#pragma unroll
        for (int tk = 0; tk < TOK; ++tk) th_hist[tk * 256 + threadIdx.x] = 0u;
        __syncthreads();
    }

    const int hrow = lane & 15, kgrp = lane >> 4;
    // this lane's head and 32-element block of each token's q (bf16), and the head weights.  All
    // loads are branch-free (rows past the last token re-read it and get weight 0; keys past the
    // range re-read its last key and are never stored), so the waits count them exactly.
    u32x4 qraw[TOK][4];
    float wt[TOK][4];
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        const int64_t qi = ((int64_t)b * T + i0 + min(tk, ntok - 1)) * kIdxH;
        const u32x4* qp = (const u32x4*)((const uint16_t*)pq + (qi + hrow) * kIdxD + 32 * kgrp);
#pragma unroll
        for (int r = 0; r < 4; ++r) qraw[tk][r] = qp[r];
        // (with no weights the load reads q's own memory, which is larger, and is discarded)
        const float* wsrc = pw ? pw : (const float*)pq;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float wv_ = wsrc[qi + 4 * kgrp + r];
            wt[tk][r] = tk < ntok ? (pw ? wv_ : 1.0f) : 0.0f;
        }
    }

    const uint8_t* kbase = (const uint8_t*)pk + (int64_t)b * k_cap * (kIdxD / 2);
    const uint32_t* ksbase = (const uint32_t*)pks + (int64_t)b * k_cap;  // 4 scale bytes per key
    TS* sbase = (TS*)psc + ((int64_t)b * T + i0) * s_stride;

    // the first key tile goes out before q is quantised, so the two latencies overlap
    int64_t c0 = key_lo + 64 * wv;
    u32x4 kc[4];
    uint32_t ks[4];
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
        const int64_t key = min(c0 + 16 * bl + hrow, key_hi - 1);
        kc[bl] = *(const u32x4*)(kbase + key * (kIdxD / 2) + 16 * kgrp);
        ks[bl] = ksbase[key];
    }
    asm volatile("" ::: "memory");

    // MXFP4 quantisation of q: block exponent from the largest magnitude (bf16 bit patterns of
    // finite values order like their magnitudes), then the E2M1 code of each element
    i32x8 qa[TOK];
    int qsc[TOK];
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        uint32_t am = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = qraw[tk][r][i];
                am = max(am, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
            }
        const int ex = mx_block_exp(__uint_as_float(am << 16));
        const float xs = ldexpf(1.0f, ex);
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // word r: elements 8r .. 8r + 7, element 8r + n in bits 4n
            // v_cvt_scalef32_pk_fp4_bf16: two bf16 divided by 2^ex, rounded to the nearest E2M1 code
            // (ties to even, saturating, sign kept) into byte i; checked equal to e2m1_code on every
            // finite bf16 value for exponents -127 .. 127
            const u32x4 v = qraw[tk][r];
            uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, as_bf16x2(v[0]), xs, 0);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, as_bf16x2(v[1]), xs, 1);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, as_bf16x2(v[2]), xs, 2);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, as_bf16x2(v[3]), xs, 3);
            qa[tk][r] = (int)word;
            qa[tk][r + 4] = 0;
        }
        qsc[tk] = ex + 127;
    }

    int64_t vis_tk[TOK];  // visible keys of each token (loop invariant)
    token_vis<TOK>(vis_tk, pos0, ntok, m, k_cap);

    for (;;) {
        const int64_t mykey = c0 + lane;  // the score this lane stores
        float mine_all[TOK];
#pragma unroll
        for (int tk = 0; tk < TOK; ++tk) {
            float part[4];
#pragma unroll
            for (int bl = 0; bl < 4; ++bl) {
                const i32x8 kb = {(int)kc[bl][0], (int)kc[bl][1], (int)kc[bl][2], (int)kc[bl][3], 0, 0, 0, 0};
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[tk], kb, acc, 4, 4, 0, qsc[tk], 0,
                                                                       (int)(ks[bl] >> (8 * kgrp)));
                // lane holds heads 4*kgrp + r of key 16 bl + hrow
                float v = wt[tk][0] * fmaxf(acc[0], 0.0f);
                v = fmaf(wt[tk][1], fmaxf(acc[1], 0.0f), v);
                v = fmaf(wt[tk][2], fmaxf(acc[2], 0.0f), v);
                part[bl] = fmaf(wt[tk][3], fmaxf(acc[3], 0.0f), v);
            }
            const float mine = sum4g_scatter(part[0], part[1], part[2], part[3]);  // key c0 + lane
            if (TOK == 1) {
                if (mykey < vis_tk[tk]) store_count<TS>(sbase + (int64_t)tk * s_stride + mykey, mine, th_hist, hist);
            }
            mine_all[tk] = mine;
        }
        // several tokens: stored after the chunk, every key of the range (as the bf16 kernel)
        if constexpr (TOK > 1) {
            if (mykey < key_hi) {
#pragma unroll
                for (int tk = 0; tk < TOK; ++tk)
                    if (tk < ntok)
                        store_count<TS>(sbase + (int64_t)tk * s_stride + mykey, mine_all[tk], th_hist + tk * 256,
                                        hist && mykey < vis_tk[tk]);
            }
        }
        c0 += 256;
        if (c0 >= key_hi) break;
        for (int bl = 0; bl < 4; ++bl) {  // (unrolled by the compiler)
            const int64_t key = min(c0 + 16 * bl + hrow, key_hi - 1);
            kc[bl] = *(const u32x4*)(kbase + key * (kIdxD / 2) + 16 * kgrp);
            ks[bl] = ksbase[key];
        }
    }
    if (hist) flush_hist<TOK>(th_hist, th_h1, th_row, th_chunked, (int64_t)b * T + i0, ntok, key_lo);
}

template <typename TIn, typename TS>
__global__ void __launch_bounds__(256) indexer_f32(IndexerArgs a) {
    const int b = blockIdx.z, i = blockIdx.y;
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = a.q_pos.v[b] + i;
    const int64_t vis = min((t + 1) / a.m, a.k_cap);
    if (s >= vis) return;
    const float* q = (const float*)a.q + ((int64_t)b * a.T + i) * a.H_I * a.d_I;
    const float* k = (const float*)a.k + ((int64_t)b * a.k_cap + s) * a.d_I;
    const float* w = a.w ? a.w + ((int64_t)b * a.T + i) * a.H_I : nullptr;
    float acc = 0.0f;
    for (int h = 0; h < a.H_I; ++h) {
        float dot = 0.0f;
        for (int d = 0; d < a.d_I; ++d) dot = fmaf(q[h * a.d_I + d], k[d], dot);
        acc = fmaf(w ? w[h] : 1.0f, fmaxf(dot, 0.0f), acc);
    }
    store_score<TS>((TS*)a.scores + ((int64_t)b * a.T + i) * a.s_stride + s, acc);
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st) {
    if (a.max_vis <= 0 || a.T <= 0) return hipSuccess;
    const bool bf_scores = a.score_dtype == LCA_BF16;
    if (a.in_dtype == LCA_F32) {
        dim3 grid((unsigned)((a.max_vis + 255) / 256), (unsigned)a.T, (unsigned)a.B);
        if (bf_scores) hipLaunchKernelGGL((indexer_f32<float, uint16_t>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((indexer_f32<float, float>), grid, dim3(256), 0, st, a);
        return hipGetLastError();
    }
    const bool fp4 = a.in_dtype == LCA_MXFP4;
    const int tok = a.T >= 64 ? 8 : 1;
    const int64_t groups = ((int64_t)a.T + tok - 1) / tok;
    // enough workgroups to cover the chip: split the key range in 256-key multiples
    int64_t want_split = (2048 + (int64_t)a.B * groups - 1) / ((int64_t)a.B * groups);
    int64_t kpw = (a.max_vis + want_split - 1) / want_split;
    kpw = ((kpw + 255) / 256) * 256;
    // MXFP4 keys are 68 bytes: a single-token launch gives each workgroup twice the keys
    if (fp4 && tok == 1) kpw *= 2;
    if (kpw < 256) kpw = 256;
    if (a.th_h1 && a.th_chunked) {
        // a workgroup's keys must lie in one chunk of the top-k: a power of two, rounded down (rounded
        // up, a row of 32,769 .. 32,768 + 767 keys took 33 workgroups of 1,024 keys instead of 43 of
        // 768, and the fused launch ran 15 % behind the plain one)
        int64_t p = 256;
        while (2 * p <= kpw && 2 * p <= kTopkChunk) p <<= 1;
        kpw = p;
    }
    const int64_t nsplit = (a.max_vis + kpw - 1) / kpw;
    dim3 grid((unsigned)nsplit, (unsigned)groups, (unsigned)a.B);
    const bool hist = a.th_h1 != nullptr && bf_scores;
#define LCA_IDX_LAUNCH(K, TOKN, TS, H) hipLaunchKernelGGL((K<TOKN, TS, H>), grid, dim3(256), 0, st, a, kpw)
#define LCA_IDX_PICK(K, TOKN)                                                         \
    do {                                                                              \
        if (!bf_scores) LCA_IDX_LAUNCH(K, TOKN, float, false);                        \
        else if (hist) LCA_IDX_LAUNCH(K, TOKN, uint16_t, true);                       \
        else LCA_IDX_LAUNCH(K, TOKN, uint16_t, false);                                \
    } while (0)
    if (fp4) {
        if (tok == 8) LCA_IDX_PICK(indexer_fp4, 8);
        else LCA_IDX_PICK(indexer_fp4, 1);
    } else {
        if (tok == 8) LCA_IDX_PICK(indexer_mfma, 8);
        else LCA_IDX_PICK(indexer_mfma, 1);
    }
#undef LCA_IDX_PICK
#undef LCA_IDX_LAUNCH
    return hipGetLastError();
}

}  // namespace lca
