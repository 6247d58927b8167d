// topk.hip -- the top-k selector ("DeepSeek-V4 中文翻译" section 2.3.1; BF16
// index scores, section 5.2.1): per query row keep K = min(k, vis) entries
// with the largest scores, ties to the lower index, emitted in ascending
// index order and padded with -1.
//
// Scores become monotone unsigned keys (bf16: 16 bits, f32: 32 bits; -0 is
// folded onto +0).  An MSB-first radix select with 8-bit digits finds the
// K-th largest key tau and how many keys equal to tau are taken (the
// lowest-indexed ones); a final pass walks the row in index order and
// compacts the winners with a block-wide exclusive scan, which yields the
// ascending output and the lower-index tie rule directly.  Histograms live
// in LDS with 16 copies (one per lane mod 16) so that lanes sharing a bin
// rarely hit the same LDS word; rows are read with 16-byte loads, four in
// flight per thread.
//
// Two schedules:
//   row   -- one 1024-thread workgroup per row (many rows: prefill).
//   split -- bf16 rows that are few and long (decode): each row is cut into
//            16384-key chunks, one workgroup per chunk, in three launches
//            (high-byte histograms, low-byte histograms of the chosen high
//            byte, emit).  Every workgroup re-derives the digits and its
//            output offset from the per-chunk histograms in the workspace,
//            so no launch needs a grid-wide barrier or zeroed memory.
#include "device.h"
#include "kernels.h"

namespace lca {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kChunk = 16384;          // keys per workgroup in the split schedule
constexpr int kSplitThreads = 512;

__device__ __forceinline__ uint32_t mono_key(uint16_t h) {
    if (h == 0x8000u) h = 0;
    return (h & 0x8000u) ? (uint32_t)(~h & 0xffffu) : (uint32_t)(h | 0x8000u);
}
__device__ __forceinline__ uint32_t mono_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename TS>
struct Vec;
template <>
struct Vec<uint16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ uint32_t key(const u32x4& v, int u) {
        return mono_key((uint16_t)((v[u >> 1] >> (16 * (u & 1))) & 0xffffu));
    }
};
template <>
struct Vec<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ uint32_t key(const u32x4& v, int u) {
        return mono_key(__uint_as_float(v[u]));
    }
};

// f(index, key) for every element of row[lo, hi); NT threads, order unspecified.
template <typename TS, int NT, typename F>
__device__ __forceinline__ void for_each_key(const TS* row, int64_t lo, int64_t hi, F f) {
    constexpr int V = Vec<TS>::N;
    const int tid = threadIdx.x;
    const uintptr_t addr = (uintptr_t)(row + lo);
    int64_t head = (int64_t)(((16u - (addr & 15u)) & 15u) / sizeof(TS));
    if (head > hi - lo) head = hi - lo;
    for (int64_t e = lo + tid; e < lo + head; e += NT) f(e, mono_key(row[e]));
    const int64_t b0 = lo + head;
    const int64_t nv = (hi - b0) / V;
    const u32x4* vp = (const u32x4*)(row + b0);
    for (int64_t v = tid; v < nv; v += 4 * NT) {
        u32x4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (v + j * NT < nv) x[j] = vp[v + j * NT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (v + j * NT < nv) {
#pragma unroll
                for (int u = 0; u < V; ++u) f(b0 + (v + j * NT) * V + u, Vec<TS>::key(x[j], u));
            }
        }
    }
    for (int64_t e = b0 + nv * V + tid; e < hi; e += NT) f(e, mono_key(row[e]));
}

// inclusive prefix sum over the workgroup; also returns the total
template <int NW>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
    }
    if (lane == 63) wsum[wv] = v;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        uint32_t x = wsum[w];
        off += w < wv ? x : 0u;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

// Find the digit d with (count of digits > d) < rem <= (count of digits >= d).
// Run by one wave over hsum[256]; writes *digit and *rem_out (rem minus keys above d).
__device__ __forceinline__ void pick_digit(const uint32_t* hsum, uint32_t rem, uint32_t* digit,
                                           uint32_t* rem_out) {
    const int lane = threadIdx.x & 63;
    const uint32_t h0 = hsum[4 * lane], h1 = hsum[4 * lane + 1], h2 = hsum[4 * lane + 2],
                   h3 = hsum[4 * lane + 3];
    const uint32_t loc = h0 + h1 + h2 + h3;
    uint32_t suf = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t nb = __shfl_down(suf, o, kWave);
        if (lane + o < 64) suf += nb;
    }
    const uint32_t above = suf - loc;
    if (above < rem && suf >= rem) {
        uint32_t acc = above;
        const uint32_t hs[4] = {h0, h1, h2, h3};
        for (int d = 3; d >= 0; --d) {
            if (acc + hs[d] >= rem) {
                *digit = 4 * lane + d;
                *rem_out = rem - acc;
                break;
            }
            acc += hs[d];
        }
    }
}

// ---------------------------------------------------------------------------
// row schedule
// ---------------------------------------------------------------------------
constexpr int kCand = 10240;  // keys sharing the chosen high byte that the two-pass tail takes
constexpr int kDef = 4096;   // keys above it (at most K)

// Two-pass end of a 16-bit row (the high byte d1 chosen, rem keys to take from its bucket): one
// pass lists, in index order, the keys above bucket d1 (all selected) and the bucket's keys with
// their low bytes in LDS; the low byte and the tie rule are resolved on that list, and the two
// ascending lists are merged into the output by binary search.  Same result as the low-byte
// histogram pass followed by the emission pass.
template <typename TS>
__device__ __forceinline__ void row_tail16(const TS* row, int64_t n, int32_t* out, uint32_t d1, uint32_t rem,
                                        uint32_t K, uint32_t* hist, uint32_t* hsum, uint32_t* wsum,
                                        uint32_t* sel_digit, uint32_t* sel_rem) {
    __shared__ uint32_t cand[kCand];  // (index << 8) | low byte, ascending index
    __shared__ int32_t defl[kDef];    // indices above bucket d1, ascending
    __shared__ int32_t chosen[kDef];  // the bucket's selected indices, ascending
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t def_base = 0, cand_base = 0;
    for (int64_t base = 0; base < n; base += 8 * kTopkThreads) {
        const int64_t e0 = base + 8 * (int64_t)tid;
        uint32_t keys[8];
        uint32_t nd = 0, nc = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool valid = e0 + u < n;
            keys[u] = valid ? mono_key(row[e0 + u]) : 0u;
            nd += (valid && (keys[u] >> 8) > d1) ? 1u : 0u;
            nc += (valid && (keys[u] >> 8) == d1) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t packed = nd | (nc << 16);
        const uint32_t excl = block_incl_scan<kTopkWaves>(packed, wsum, &tot) - packed;
        uint32_t dp = def_base + (excl & 0xffffu), cp = cand_base + (excl >> 16);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (e0 + u >= n) break;
            const uint32_t hb = keys[u] >> 8;
            if (hb > d1) defl[dp++] = (int32_t)(e0 + u);
            else if (hb == d1) cand[cp++] = ((uint32_t)(e0 + u) << 8) | (keys[u] & 255u);
        }
        def_base += tot & 0xffffu;
        cand_base += tot >> 16;
    }
    const uint32_t D = def_base, C = cand_base;  // D = K - rem, C = the bucket's size
    // low byte: histogram of the bucket
    for (int j = tid; j < 256 * 16; j += kTopkThreads) hist[j] = 0;
    __syncthreads();
    for (uint32_t j = tid; j < C; j += kTopkThreads) atomicAdd(&hist[(cand[j] & 255u) * 16 + (lane & 15)], 1u);
    __syncthreads();
    if (tid < 256) {
        uint32_t s = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) s += hist[tid * 16 + ((c + tid) & 15)];
        hsum[tid] = s;
    }
    __syncthreads();
    if (tid < 64) pick_digit(hsum, rem, sel_digit, sel_rem);
    __syncthreads();
    const uint32_t d2 = *sel_digit, rem2 = *sel_rem;
    // the bucket's selected keys: low byte above d2, and the first rem2 (in index order) equal to it
    const uint32_t per = (C + kTopkThreads - 1) / kTopkThreads;
    const uint32_t c0 = min(C, tid * per), c1 = min(C, c0 + per);
    uint32_t neq = 0;
    for (uint32_t j = c0; j < c1; ++j) neq += (cand[j] & 255u) == d2 ? 1u : 0u;
    uint32_t tot;
    uint32_t eq_before = block_incl_scan<kTopkWaves>(neq, wsum, &tot) - neq;
    uint32_t nsel = 0;
    for (uint32_t j = c0; j < c1; ++j) {
        const uint32_t lo = cand[j] & 255u;
        if (lo > d2) ++nsel;
        else if (lo == d2 && eq_before++ < rem2) ++nsel;
    }
    uint32_t sel_pos = block_incl_scan<kTopkWaves>(nsel, wsum, &tot) - nsel;
    eq_before = block_incl_scan<kTopkWaves>(neq, wsum, &tot) - neq;  // (restart this thread's count)
    for (uint32_t j = c0; j < c1; ++j) {
        const uint32_t lo = cand[j] & 255u;
        const bool take = lo > d2 || (lo == d2 && eq_before++ < rem2);
        if (take) chosen[sel_pos++] = (int32_t)(cand[j] >> 8);
    }
    __syncthreads();
    // merge: each entry's place is its rank in its own list plus the entries of the other list below it
    for (uint32_t j = tid; j < D; j += kTopkThreads) {
        const int32_t v = defl[j];
        uint32_t lo = 0, hi = rem;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (chosen[mid] < v) lo = mid + 1;
            else hi = mid;
        }
        out[j + lo] = v;
    }
    for (uint32_t j = tid; j < rem; j += kTopkThreads) {
        const int32_t v = chosen[j];
        uint32_t lo = 0, hi = D;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (defl[mid] < v) lo = mid + 1;
            else hi = mid;
        }
        out[j + lo] = v;
    }
    (void)K;
}

template <typename TS, int BITS>
__global__ void __launch_bounds__(kTopkThreads) topk_row(TopkArgs a) {
    const int b = blockIdx.y, i = blockIdx.x;
    const int64_t t = a.q_pos.v[b] + i;
    const int64_t n = min((t + 1) / a.m, a.s_stride);
    const TS* row = (const TS*)a.scores + ((int64_t)b * a.T + i) * a.s_stride;
    int32_t* out = a.idx + ((int64_t)b * a.T + i) * a.k;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t K = min((int64_t)a.k, n);

    for (int64_t j = K + tid; j < a.k; j += kTopkThreads) out[j] = -1;
    if (n <= a.k) {
        for (int64_t j = tid; j < n; j += kTopkThreads) out[j] = (int32_t)j;
        return;
    }

    __shared__ uint32_t hist[256 * 16];
    __shared__ uint32_t hsum[256];
    __shared__ uint32_t wsum[kTopkWaves];
    __shared__ uint32_t sel_digit, sel_rem;

    uint32_t prefix = 0;
    uint32_t rem = (uint32_t)K;
#pragma unroll 1
    for (int shift = BITS - 8; shift >= 0; shift -= 8) {
        for (int j = tid; j < 256 * 16; j += kTopkThreads) hist[j] = 0;
        __syncthreads();
        const uint32_t hmask = (shift + 8 >= 32) ? 0u : (0xffffffffu << (shift + 8));
        const uint32_t want = prefix & hmask;
        const int sub = lane & 15;
        for_each_key<TS, kTopkThreads>(row, 0, n, [&](int64_t, uint32_t key) {
            if ((key & hmask) == want) atomicAdd(&hist[((key >> shift) & 255u) * 16 + sub], 1u);
        });
        __syncthreads();
        if (tid < 256) {
            uint32_t s = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) s += hist[tid * 16 + ((c + tid) & 15)];
            hsum[tid] = s;
        }
        __syncthreads();
        if (tid < 64) pick_digit(hsum, rem, &sel_digit, &sel_rem);
        __syncthreads();
        prefix |= sel_digit << shift;
        rem = sel_rem;
        if constexpr (BITS == 16) {
            // few keys share the chosen high byte: one more pass over the row instead of two
            if (shift == 8 && hsum[sel_digit] <= kCand && K <= kDef && n < (int64_t)1 << 24) {
                row_tail16<TS>(row, n, out, prefix >> 8, rem, (uint32_t)K, hist, hsum, wsum, &sel_digit, &sel_rem);
                return;
            }
        }
        __syncthreads();
    }
    const uint32_t tau = prefix;

    uint32_t gt_base = 0, eq_base = 0;
    for (int64_t base = 0; base < n; base += 8 * kTopkThreads) {
        const int64_t e0 = base + 8 * (int64_t)tid;
        uint32_t keys[8];
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool valid = e0 + u < n;
            keys[u] = valid ? mono_key(row[e0 + u]) : 0u;
            ngt += (valid && keys[u] > tau) ? 1u : 0u;
            neq += (valid && keys[u] == tau) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t packed = ngt | (neq << 16);
        const uint32_t excl = block_incl_scan<kTopkWaves>(packed, wsum, &tot) - packed;
        uint32_t gt_before = gt_base + (excl & 0xffffu);
        uint32_t eq_before = eq_base + (excl >> 16);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (e0 + u >= n) break;
            const uint32_t pos = gt_before + min(eq_before, rem);
            if (keys[u] > tau) {
                out[pos] = (int32_t)(e0 + u);
                ++gt_before;
            } else if (keys[u] == tau) {
                if (eq_before < rem) out[pos] = (int32_t)(e0 + u);
                ++eq_before;
            }
        }
        gt_base += tot & 0xffffu;
        eq_base += tot >> 16;
        if (gt_base + min(eq_base, rem) >= (uint32_t)K && eq_base >= rem) break;  // all found
    }
}

// ---------------------------------------------------------------------------
// split schedule (bf16 scores)
// ---------------------------------------------------------------------------
// Grid (G, T, B): chunk g = blockIdx.x of row i = blockIdx.y of sequence b = blockIdx.z.  Each
// launch is short and bound by latency, so every kernel reads its arguments, its 32 keys per
// thread and every histogram column it needs in one round of loads before any of them is used.
constexpr int kPer = kChunk / kSplitThreads;  // 32 keys per thread
struct SplitRow {
    const uint16_t* row;
    int32_t* out;
    int64_t n, K, stride;
    uint32_t* h1;   // [G][256] high-byte histograms of this row
    uint32_t* h2;   // [G][256] low-byte histograms (keys with the chosen high byte)
};

__device__ __forceinline__ SplitRow split_row(const TopkArgs& a, int G) {
    // arguments first, all in one batch of scalar loads (see the launch comment above)
    const int b = blockIdx.z;
    const int64_t qp = a.q_pos.v[b], stride = a.s_stride;
    const int m = a.m, k = a.k;
    const void* sc = a.scores;
    int32_t* idx = a.idx;
    void* ws = a.ws;
    asm volatile("" ::"s"(qp), "s"(stride), "s"(m), "s"(k), "s"(sc), "s"(idx), "s"(ws));
    SplitRow r;
    const int64_t rowid = (int64_t)b * gridDim.y + blockIdx.y;
    const int64_t t1 = qp + blockIdx.y + 1;
    const int64_t vis = (m & (m - 1)) == 0 ? t1 >> __builtin_ctz((unsigned)m) : t1 / m;  // (t + 1) / m
    r.n = min(vis, stride);
    r.K = min((int64_t)k, r.n);
    r.stride = stride;
    r.row = (const uint16_t*)sc + rowid * stride;
    r.out = idx + rowid * k;
    r.h1 = (uint32_t*)ws + rowid * (int64_t)G * 512;
    r.h2 = r.h1 + (int64_t)G * 256;
    return r;
}

// This thread's 32 consecutive scores of chunk [lo, hi) as bf16 pairs (element lo + 32 tid + 2q in
// the low half of raw[q]).  Elements at or past hi are never counted: a thread whose 32 keys lie
// inside the row's s_stride reads them as two 16-byte pairs whatever their validity, the others
// element by element.
__device__ __forceinline__ void load_keys(const SplitRow& r, int64_t lo, int64_t hi, uint32_t* raw) {
    const int64_t e0 = lo + (int64_t)kPer * threadIdx.x;
    const bool vec = (((uintptr_t)(r.row + lo)) & 15u) == 0 && e0 + kPer <= r.stride;
    if (vec) {
#pragma unroll
        for (int q = 0; q < kPer / 8; ++q) {
            const u32x4 x = ((const u32x4*)(r.row + e0))[q];
#pragma unroll
            for (int w = 0; w < 4; ++w) raw[4 * q + w] = x[w];
        }
    } else {
#pragma unroll
        for (int q = 0; q < kPer / 2; ++q) {
            const uint32_t l = e0 + 2 * q < hi ? r.row[e0 + 2 * q] : 0u;
            const uint32_t h = e0 + 2 * q + 1 < hi ? r.row[e0 + 2 * q + 1] : 0u;
            raw[q] = l | (h << 16);
        }
    }
}

__device__ __forceinline__ uint32_t raw_key(const uint32_t* raw, int u) {
    return mono_key((uint16_t)(raw[u >> 1] >> (16 * (u & 1))));
}

// histogram (16 LDS copies, one per lane mod 16) of bin_of(key) over this thread's valid keys,
// reduced into hs[256]
template <typename F>
__device__ __forceinline__ void keys_hist(const uint32_t* raw, int64_t e0, int64_t hi, uint32_t* hist, uint32_t* hs,
                                          F bin_of) {
    const int tid = threadIdx.x, sub = tid & 15;
    for (int j = tid; j < 256 * 16; j += kSplitThreads) hist[j] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        if (e0 + u < hi) {
            const int bin = bin_of(raw_key(raw, u));
            if (bin >= 0) atomicAdd(&hist[bin * 16 + sub], 1u);
        }
    }
    __syncthreads();
    if (tid < 256) {
        uint32_t s = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) s += hist[tid * 16 + ((c + tid) & 15)];
        hs[tid] = s;
    }
    __syncthreads();
}

// Column sums of bin `bin` over the G chunk histograms h[g][256] of NH histograms (h2 = h1 + 256 G):
// the totals and the sums over the chunks before g_me.  All loads of a batch of 24 chunks go out
// before any sum (one round for G <= 24).
template <int NH>
__device__ __forceinline__ void col_sums(const uint32_t* h1, int G, int g_me, int bin, uint32_t* tot, uint32_t* pre) {
    constexpr int kB = 24;
#pragma unroll
    for (int k = 0; k < NH; ++k) tot[k] = pre[k] = 0;
    for (int g0 = 0; g0 < G; g0 += kB) {
        uint32_t v[NH][kB];
#pragma unroll
        for (int k = 0; k < NH; ++k)
#pragma unroll
            for (int u = 0; u < kB; ++u) v[k][u] = h1[(int64_t)k * G * 256 + (g0 + u < G ? g0 + u : 0) * 256 + bin];
#pragma unroll
        for (int k = 0; k < NH; ++k)
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint32_t x = g0 + u < G ? v[k][u] : 0u;
                tot[k] += x;
                pre[k] += g0 + u < g_me ? x : 0u;
            }
    }
}

__global__ void __launch_bounds__(kSplitThreads) topk_split_h1(TopkArgs a, int G) {
    const SplitRow r = split_row(a, G);
    const int g = blockIdx.x;
    const int64_t lo = (int64_t)g * kChunk, hi = min(lo + kChunk, r.n);
    __shared__ uint32_t hist[256 * 16];
    __shared__ uint32_t hs[256];
    if (r.n <= r.K) return;  // trivial row: the emit launch handles it
    uint32_t raw[kPer / 2];
    load_keys(r, lo, hi, raw);
    keys_hist(raw, lo + (int64_t)kPer * threadIdx.x, hi, hist, hs, [](uint32_t key) { return (int)(key >> 8); });
    if (threadIdx.x < 256) r.h1[g * 256 + threadIdx.x] = hs[threadIdx.x];
}

__global__ void __launch_bounds__(kSplitThreads) topk_split_h2(TopkArgs a, int G) {
    const SplitRow r = split_row(a, G);
    const int g = blockIdx.x, tid = threadIdx.x;
    const int64_t lo = (int64_t)g * kChunk, hi = min(lo + kChunk, r.n);
    __shared__ uint32_t hist[256 * 16];
    __shared__ uint32_t hs[256];
    __shared__ uint32_t d1, rem1;
    if (r.n <= r.K) return;
    uint32_t raw[kPer / 2];
    load_keys(r, lo, hi, raw);
    uint32_t t1[1] = {0}, p1[1] = {0};
    if (tid < 256) col_sums<1>(r.h1, G, 0, tid, t1, p1);
    if (tid < 256) hs[tid] = t1[0];
    __syncthreads();
    if (tid < 64) pick_digit(hs, (uint32_t)r.K, &d1, &rem1);
    __syncthreads();
    const uint32_t hb = d1;
    keys_hist(raw, lo + (int64_t)kPer * tid, hi, hist, hs,
              [hb](uint32_t key) { return (key >> 8) == hb ? (int)(key & 255u) : -1; });
    if (tid < 256) r.h2[g * 256 + tid] = hs[tid];
}

// Fused schedule (a.th_cnt): this workgroup has read the row's histograms for the last time; the
// last of the row's G workgroups to get here clears both (and the arrival counter), so the next
// call's indexer adds into zeros and the workspace is left as it came.  Every workgroup of the row
// comes here exactly once.
__device__ __forceinline__ void th_arrive(const TopkArgs& a, const SplitRow& r, int G, uint32_t* last) {
    if (!a.th_cnt) return;
    const int64_t rowid = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
    __syncthreads();  // (every histogram value this workgroup loaded has been used)
    if (threadIdx.x == 0) *last = atomicAdd(&a.th_cnt[rowid], 1u) == (uint32_t)G - 1u;
    __syncthreads();
    if (*last) {
        for (int j = threadIdx.x; j < G * 512; j += kSplitThreads) r.h1[j] = 0u;  // h1, then h2
        if (threadIdx.x == 0) a.th_cnt[rowid] = 0u;
    }
}

__global__ void __launch_bounds__(kSplitThreads) topk_split_emit(TopkArgs a, int G) {
    const SplitRow r = split_row(a, G);
    const int g = blockIdx.x, tid = threadIdx.x;
    const int64_t lo = (int64_t)g * kChunk, hi = min(lo + kChunk, r.n);
    const int kk = a.k;
    __shared__ uint32_t th_last;
    if (r.n <= r.K) {  // fewer candidates than k: all of them, in order
        th_arrive(a, r, G, &th_last);
        for (int64_t j = lo + tid; j < lo + kChunk && j < kk; j += kSplitThreads)
            r.out[j] = j < r.n ? (int32_t)j : -1;
        if (g == G - 1)
            for (int64_t j = (int64_t)G * kChunk + tid; j < kk; j += kSplitThreads) r.out[j] = j < r.n ? (int32_t)j : -1;
        return;
    }
    // one round: this thread's keys and (thread = bin) both histograms' columns
    uint32_t raw[kPer / 2];
    load_keys(r, lo, hi, raw);
    uint32_t tt[2] = {0, 0}, pp[2] = {0, 0};
    if (tid < 256) col_sums<2>(r.h1, G, g, tid, tt, pp);
    const uint32_t t1 = tt[0], p1 = pp[0], t2 = tt[1], p2 = pp[1];
    __shared__ uint32_t tot1[256], tot2[256];
    __shared__ uint32_t d1, rem1, d2, rem2;
    __shared__ uint32_t wsum[kSplitThreads / 64];
    __shared__ uint32_t base_gt, base_eq;
    if (tid < 256) {
        tot1[tid] = t1;
        tot2[tid] = t2;
    }
    __syncthreads();
    th_arrive(a, r, G, &th_last);
    if (tid < 64) pick_digit(tot1, (uint32_t)r.K, &d1, &rem1);
    __syncthreads();
    if (tid < 64) pick_digit(tot2, rem1, &d2, &rem2);
    __syncthreads();
    const uint32_t tau = (d1 << 8) | d2, rem = rem2;
    if (g == 0)
        for (int64_t j = r.K + tid; j < kk; j += kSplitThreads) r.out[j] = -1;
    // keys above tau and equal to tau in the chunks before this one: thread = bin
    {
        uint32_t gt = 0, eq = 0;
        if (tid < 256) {
            gt = ((uint32_t)tid > d1 ? p1 : 0u) + ((uint32_t)tid > d2 ? p2 : 0u);
            eq = (uint32_t)tid == d2 ? p2 : 0u;
        }
        uint32_t s1, s2;
        block_incl_scan<kSplitThreads / 64>(gt, wsum, &s1);
        block_incl_scan<kSplitThreads / 64>(eq, wsum, &s2);
        if (tid == 0) {
            base_gt = s1;
            base_eq = s2;
        }
        __syncthreads();
    }
    const int64_t e0 = lo + (int64_t)kPer * tid;
    uint32_t keys[kPer];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const bool valid = e0 + u < hi;
        keys[u] = valid ? mono_key((uint16_t)(raw[u >> 1] >> (16 * (u & 1)))) : 0u;
        ngt += (valid && keys[u] > tau) ? 1u : 0u;
        neq += (valid && keys[u] == tau) ? 1u : 0u;
    }
    uint32_t t;
    const uint32_t packed = ngt | (neq << 16);  // at most 16384 each
    const uint32_t excl = block_incl_scan<kSplitThreads / 64>(packed, wsum, &t) - packed;
    uint32_t gt_before = base_gt + (excl & 0xffffu);
    uint32_t eq_before = base_eq + (excl >> 16);
    if (ngt + neq == 0) return;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        if (e0 + u >= hi) break;
        const uint32_t pos = gt_before + min(eq_before, rem);
        if (keys[u] > tau) {
            r.out[pos] = (int32_t)(e0 + u);
            ++gt_before;
        } else if (keys[u] == tau) {
            if (eq_before < rem) r.out[pos] = (int32_t)(e0 + u);
            ++eq_before;
        }
    }
}

// split schedule for few long bf16 rows
static bool use_split(const TopkArgs& a, int64_t max_n) {
    const int64_t rows = (int64_t)a.B * a.T;
    return a.score_dtype == LCA_BF16 && rows < 128 && max_n > kChunk;
}

static int split_chunks(int64_t max_n) { return (int)((max_n + kChunk - 1) / kChunk); }

size_t topk_ws_bytes(int32_t B, int32_t T, int64_t s_stride, int32_t score_dtype) {
    TopkArgs a;
    a.B = B;
    a.T = T;
    a.score_dtype = score_dtype;
    if (!use_split(a, s_stride)) return 0;
    return (size_t)B * T * split_chunks(s_stride) * 512 * sizeof(uint32_t);
}

int topk_split_chunks(int32_t rows, int64_t max_n, int64_t s_stride, int32_t score_dtype) {
    TopkArgs a;
    a.B = rows;
    a.T = 1;
    a.score_dtype = score_dtype;
    return use_split(a, max_n) ? split_chunks(s_stride) : 0;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (use_split(a, a.max_n)) {
        const int G = split_chunks(a.s_stride);
        dim3 grid((unsigned)G, (unsigned)a.T, (unsigned)a.B);
        if (!a.th_cnt) hipLaunchKernelGGL(topk_split_h1, grid, dim3(kSplitThreads), 0, st, a, G);
        hipLaunchKernelGGL(topk_split_h2, grid, dim3(kSplitThreads), 0, st, a, G);
        hipLaunchKernelGGL(topk_split_emit, grid, dim3(kSplitThreads), 0, st, a, G);
        return hipGetLastError();
    }
    dim3 grid((unsigned)a.T, (unsigned)a.B);
    if (a.score_dtype == LCA_BF16)
        hipLaunchKernelGGL((topk_row<uint16_t, 16>), grid, dim3(kTopkThreads), 0, st, a);
    else
        hipLaunchKernelGGL((topk_row<float, 32>), grid, dim3(kTopkThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lca
