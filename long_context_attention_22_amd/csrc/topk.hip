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
// rarely hit the same LDS word; the split schedule's second-digit histogram,
// which counts only the threshold bucket's keys, keeps four.
//
// Two schedules:
//   row   -- one 1024-thread workgroup per row (many rows: prefill); rows are
//            read with 16-byte loads, four in flight per thread.
//   split -- bf16 rows that are few and long (decode): each row is cut into
//            kTopkChunk-key chunks, one workgroup per chunk, in three launches
//            (high-byte histograms, low-byte histograms of the chosen high
//            byte, emit).  Every workgroup re-derives the digits and its
//            output offset from the per-chunk histograms in the workspace,
//            so no launch needs a grid-wide barrier or zeroed memory.  Short
//            chunks spread the per-key work of these latency-bound launches
//            over many CUs; the price is more histogram columns to sum.
#include "device.h"
#include "kernels.h"

namespace lca {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kChunk = kTopkChunk;     // keys per workgroup in the split schedule
constexpr int kSplitMin = 16384;       // rows longer than this may take it
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

// Comparisons of mono_key(h) with a key tau done on the raw bf16 bits h: the key grows with h on the
// non-negative half and falls with h on the negative half (-0 counts as +0), so the raw values whose
// key is above tau form one interval, and those whose key equals tau are one value (two for tau =
// +0: +0 and -0).  Raw values sit zero-extended in 32 bits; kNoKey, what a lane past the row holds,
// passes neither test.
constexpr uint32_t kNoKey = 0x10000u;
struct KeyCut {
    uint32_t gt_lo, gt_span;   // key(h) > tau  <=>  h - gt_lo < gt_span (unsigned)
    uint32_t eq_mask, eq_raw;  // key(h) == tau <=>  (h & eq_mask) == eq_raw
    __device__ __forceinline__ bool gt(uint32_t h) const { return h - gt_lo < gt_span; }
    __device__ __forceinline__ bool eq(uint32_t h) const { return (h & eq_mask) == eq_raw; }
};
// tau in [-1, 0xffff]; -1 stands below every key
__device__ __forceinline__ KeyCut key_cut(int tau) {
    KeyCut c;
    if (tau < 0) {
        c = KeyCut{0u, 0x10000u, 0x1ffffu, 0x20000u};
    } else if (tau >= 0x8000) {  // a non-negative value with raw bits rt
        const uint32_t rt = (uint32_t)tau & 0x7fffu;
        c = KeyCut{rt + 1u, 0x7fffu - rt, rt == 0u ? 0x17fffu : 0x1ffffu, rt};
    } else {  // a negative value with raw bits rt (0x8000, -0, is no key: the interval then takes it in)
        const uint32_t rt = ~(uint32_t)tau & 0xffffu;
        c = KeyCut{0u, rt == 0x8000u ? 0x8001u : rt, 0x1ffffu, rt == 0x8000u ? 0x20000u : rt};
    }
    return c;
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

// f(index, key) for every element of row[lo, hi); NT threads, order unspecified.  Each thread has
// kVecs 16-byte loads in flight per round.
constexpr int kVecs = 8;
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
    for (int64_t v = tid; v < nv; v += kVecs * NT) {
        u32x4 x[kVecs];
#pragma unroll
        for (int j = 0; j < kVecs; ++j)
            if (v + j * NT < nv) x[j] = vp[v + j * NT];
#pragma unroll
        for (int j = 0; j < kVecs; ++j) {
            if (v + j * NT < nv) {
#pragma unroll
                for (int u = 0; u < V; ++u) f(b0 + (v + j * NT) * V + u, Vec<TS>::key(x[j], u));
            }
        }
    }
    for (int64_t e = b0 + nv * V + tid; e < hi; e += NT) f(e, mono_key(row[e]));
}

// lanes of the wave where p holds
__device__ __forceinline__ uint32_t lane_count(bool p) {
    return (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(p));
}
// lanes below this one in the mask
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// inclusive prefix sum over the workgroup; also returns the total
template <int NW>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    v = wave_incl_scan(v);
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
    // keys in digits above this lane's four: the total less the inclusive prefix
    const uint32_t incl = wave_incl_scan(loc);
    const uint32_t above = wave_lane63(incl) - incl, suf = above + loc;
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
        if (j + lo < K) out[j + lo] = v;  // (always: D + rem = K; a guard on the global store)
    }
    for (uint32_t j = tid; j < rem; j += kTopkThreads) {
        const int32_t v = chosen[j];
        uint32_t lo = 0, hi = D;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (defl[mid] < v) lo = mid + 1;
            else hi = mid;
        }
        if (j + lo < K) out[j + lo] = v;  // (always: D + rem = K; a guard on the global store)
    }
}

// Emission of a row (threshold key tau, rem keys equal to it to take, K in all): the row in index
// order, kRowIter keys a round; wave w holds keys base + kRowWave w + 64 u + lane (u < kRowBlk), so
// each u is 64 consecutive keys across the wave and counts and ranks come from lane masks.  The next
// round's keys are loaded before this round's are ranked (the pass is otherwise one memory round trip
// per round); the waves' counts meet in LDS, double-buffered by round, one barrier a round.
constexpr int kRowBlk = 16;
constexpr int kRowWave = 64 * kRowBlk;
constexpr int kRowIter = kRowWave * kTopkWaves;
// (branch-free, so that the compiler can count the loads in flight and wait for one round's loads
// only: a round inside the first `lim` keys of the row -- n or the row's stride -- loads its keys
// at constant offsets from one address, the last ones re-read key lim - 1 past it; keys past n are
// masked where they are used)
template <typename TS>
__device__ __forceinline__ void row_load(const TS* row, int64_t lim, int64_t base, uint32_t (&raw)[kRowBlk]) {
    const int64_t e = base + (int64_t)(threadIdx.x >> 6) * kRowWave + (threadIdx.x & 63);
    if (base + kRowIter <= lim) {  // (uniform)
        const TS* p = row + e;
#pragma unroll
        for (int u = 0; u < kRowBlk; ++u) {
            if constexpr (sizeof(TS) == 2) raw[u] = (uint32_t)p[64 * u];
            else raw[u] = __float_as_uint(p[64 * u]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kRowBlk; ++u) {
            const int64_t j = min(e + 64 * u, lim - 1);
            if constexpr (sizeof(TS) == 2) raw[u] = (uint32_t)row[j];
            else raw[u] = __float_as_uint(row[j]);
        }
    }
}
// the tests against tau on raw score bits: interval tests for bf16, monotone keys for f32
template <typename TS>
struct RowCut;
template <>
struct RowCut<uint16_t> {
    KeyCut c;
    __device__ explicit RowCut(uint32_t tau) : c(key_cut((int)tau)) {}
    __device__ __forceinline__ bool gt(uint32_t r) const { return c.gt(r); }
    __device__ __forceinline__ bool eq(uint32_t r) const { return c.eq(r); }
};
template <>
struct RowCut<float> {
    uint32_t tau;
    __device__ explicit RowCut(uint32_t t) : tau(t) {}
    __device__ __forceinline__ bool gt(uint32_t r) const { return mono_key(__uint_as_float(r)) > tau; }
    __device__ __forceinline__ bool eq(uint32_t r) const { return mono_key(__uint_as_float(r)) == tau; }
};

// one round of row_emit: ranks and stores the keys in cur (round base), with the next round's loads
// into nxt issued first; returns true once every kept key is out.  TAIL: the round reaches the row's
// end (keys at or past n are masked; other rounds test nothing but the keys).
template <typename TS, bool TAIL>
__device__ __forceinline__ bool row_round(const TS* row, int64_t n, int64_t stride, int32_t* out, const RowCut<TS>& cut,
                                          uint32_t rem, uint32_t K, int64_t base, int wv, int64_t lane0,
                                          uint32_t (&cur)[kRowBlk], uint32_t (&nxt)[kRowBlk], u32x4 (&wc)[2 * kTopkWaves / 4],
                                          uint32_t& gt_base, uint32_t& eq_base) {
    if (!TAIL) row_load<TS>(row, stride, base + kRowIter, nxt);  // (a round before the last: the next exists)
    const int64_t e = base + lane0;
    const int lim = TAIL ? (int)min(max(n - e, (int64_t)0), (int64_t)kRowWave) : kRowWave;  // keys of this lane's column
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < kRowBlk; ++u) {
        const bool v = !TAIL || 64 * u < lim;
        ngt += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v && cut.gt(cur[u])));
        neq += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v && cut.eq(cur[u])));
    }
    uint32_t* wcw = (uint32_t*)wc;  // the waves' counts: (above, equal) of wave w at 2w, 2w + 1
    if ((threadIdx.x & 63) == 0) {
        wcw[2 * wv] = ngt;
        wcw[2 * wv + 1] = neq;
    }
    __syncthreads();
    uint32_t gr = gt_base, qr = eq_base, tg = 0, tq = 0;
#pragma unroll
    for (int j = 0; j < 2 * kTopkWaves / 4; ++j) {  // (16-byte broadcast reads)
        const u32x4 x = wc[j];
        gr += (2 * j < wv ? x[0] : 0u) + (2 * j + 1 < wv ? x[2] : 0u);
        qr += (2 * j < wv ? x[1] : 0u) + (2 * j + 1 < wv ? x[3] : 0u);
        tg += x[0] + x[2];
        tq += x[1] + x[3];
    }
    gr = __builtin_amdgcn_readfirstlane(gr);
    qr = __builtin_amdgcn_readfirstlane(qr);
    if (ngt + neq != 0) {
#pragma unroll
        for (int u = 0; u < kRowBlk; ++u) asm volatile("" : "+v"(cur[u]));  // (the tests again, not kept)
#pragma unroll
        for (int u = 0; u < kRowBlk; ++u) {
            const bool v = !TAIL || 64 * u < lim;
            const bool gk = v && cut.gt(cur[u]), qk = v && cut.eq(cur[u]);
            const uint64_t gm = __builtin_amdgcn_ballot_w64(gk), qm = __builtin_amdgcn_ballot_w64(qk);
            if ((gm | qm) == 0) continue;
            const uint32_t gb = gr + lanes_below(gm), qb = qr + lanes_below(qm);
            const uint32_t pos = gb + min(qb, rem);  // < K for every kept key
            if ((gk | (qk & (qb < rem))) & (pos < K)) out[pos] = (int32_t)(e + 64 * u);
            gr += (uint32_t)__builtin_popcountll(gm);
            qr += (uint32_t)__builtin_popcountll(qm);
        }
    }
    gt_base += tg;
    eq_base += tq;
    return TAIL || (gt_base + min(eq_base, rem) >= K && eq_base >= rem);  // (uniform)
}

template <typename TS>
__device__ __forceinline__ void row_emit(const TS* row, int64_t n, int64_t stride, int32_t* out, uint32_t tau,
                                         uint32_t rem, uint32_t K) {
    __shared__ u32x4 wc[2][2 * kTopkWaves / 4];
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t lane0 = (int64_t)wv * kRowWave + (threadIdx.x & 63);
    const RowCut<TS> cut(tau);
    uint32_t ra[kRowBlk], rb[kRowBlk];
    row_load<TS>(row, stride, 0, ra);
    uint32_t gt_base = 0, eq_base = 0;
    // two rounds per trip, the register sets alternating (no copies between rounds), the LDS counts
    // of consecutive rounds in different buffers
    for (int64_t base = 0;; base += 2 * kRowIter) {
        if (base + kRowIter < n) {
            if (row_round<TS, false>(row, n, stride, out, cut, rem, K, base, wv, lane0, ra, rb, wc[0], gt_base, eq_base))
                break;
        } else {
            row_round<TS, true>(row, n, stride, out, cut, rem, K, base, wv, lane0, ra, rb, wc[0], gt_base, eq_base);
            break;
        }
        const int64_t b2 = base + kRowIter;
        if (b2 + kRowIter < n) {
            if (row_round<TS, false>(row, n, stride, out, cut, rem, K, b2, wv, lane0, rb, ra, wc[1], gt_base, eq_base))
                break;
        } else {
            row_round<TS, true>(row, n, stride, out, cut, rem, K, b2, wv, lane0, rb, ra, wc[1], gt_base, eq_base);
            break;
        }
    }
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
    // The first pass made by the indexer (a.row_h1, bf16 rows): this row's high-byte histogram, read
    // and zeroed for the next call (also for the rows that need no selection).
    const bool pre = BITS == 16 && a.row_h1 != nullptr;
    uint32_t h1 = 0;
    if (pre && tid < 256) {
        uint32_t* hp = a.row_h1 + ((int64_t)b * a.T + i) * 256 + tid;
        h1 = *hp;
        *hp = 0u;
    }

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
        if (pre && shift == BITS - 8) {
            if (tid < 256) hsum[tid] = h1;
        } else {
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
    row_emit<TS>(row, n, a.s_stride, out, tau, rem, (uint32_t)K);
}

// ---------------------------------------------------------------------------
// split schedule (bf16 scores)
// ---------------------------------------------------------------------------
// Grid (G, T, B): chunk g = blockIdx.x of row i = blockIdx.y of sequence b = blockIdx.z.  Each
// launch is short and bound by latency, so every kernel reads its arguments, its keys per
// thread and every histogram column it needs in one round of loads before any of them is used.
//   Workspace of R = B T rows: the rows' high-byte histograms h1 [R][G][kTopkHistWords], then their
// low-byte histograms h2 [R][G][kTopkHistWords] (keys with the chosen high byte; both in 16-bit
// counts, two bins per word), then per row and chunk g the word quadruple (keys above the chosen
// high byte in the chunks before g, that byte, the keys still to take from its bucket, 0) that the
// second launch leaves for the third.  Only h1 may need zeros:
// where the indexer adds it up (TopkArgs::split_fused) the third launch clears it again, each
// workgroup its own chunk, since by then the second launch -- its last reader -- has ended.
constexpr int kPer = kChunk / kSplitThreads;  // keys per thread
struct SplitRow {
    const uint16_t* row;
    int32_t* out;
    int64_t n, K, stride;
    uint32_t* h1;    // [G][kTopkHistWords] high-byte histograms of this row
    uint32_t* h2;    // [G][kTopkHistWords] low-byte histograms (keys with the chosen high byte)
    uint32_t* meta;  // [G][4] (above d1 before chunk g, d1, rem1, 0)
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
    const int64_t rows = (int64_t)gridDim.y * gridDim.z;
    r.h1 = (uint32_t*)ws + rowid * (int64_t)G * kTopkHistWords;
    r.h2 = (uint32_t*)ws + (rows + rowid) * (int64_t)G * kTopkHistWords;
    r.meta = (uint32_t*)ws + 2 * rows * (int64_t)G * kTopkHistWords + rowid * (int64_t)G * 4;
    return r;
}

// This thread's kPer consecutive scores of chunk [lo, hi) as bf16 pairs (element lo + kPer tid + 2q
// in the low half of raw[q]).  Elements at or past hi are never counted: a thread whose keys lie
// inside the row's s_stride reads them as 16-byte vectors whatever their validity, the others
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

// The second and third launches hold a chunk wave by wave: wave w has keys lo + kWaveKeys w + 64 u +
// lane for u < kBlk, so each u is 64 consecutive keys across the wave, and counts and ranks in index
// order come from lane masks (ballot, mbcnt) instead of per-thread loops.
constexpr int kWaveKeys = kChunk / (kSplitThreads / 64);
constexpr int kBlk = kWaveKeys / 64;  // = kPer
__device__ __forceinline__ int64_t lane_first(int64_t lo) {
    return lo + (int64_t)(threadIdx.x >> 6) * kWaveKeys + (threadIdx.x & 63);
}
// The loads take any key inside the row's s_stride, so that their addresses need no position; keys
// at or past hi (visible count, chunk end) become kNoKey afterwards.
__device__ __forceinline__ void load_lane_keys(const SplitRow& r, int64_t lo, uint32_t* h) {
    const int64_t e = lane_first(lo);
#pragma unroll
    for (int u = 0; u < kBlk; ++u) h[u] = e + 64 * u < r.stride ? (uint32_t)r.row[e + 64 * u] : kNoKey;
}
__device__ __forceinline__ void mask_lane_keys(int64_t lo, int64_t hi, uint32_t* h) {
    const int64_t e = lane_first(lo);
#pragma unroll
    for (int u = 0; u < kBlk; ++u) h[u] = e + 64 * u < hi ? h[u] : kNoKey;
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

// Column sums over the G chunk histograms h[g][kTopkHistWords] (16-bit counts, two bins per word):
// for bins 2t and 2t + 1 of thread t < 128, the totals over every chunk and the sums over the chunks
// before g_me.  The 512 threads share the loads: thread (t = tid mod 128, c = tid / 128) takes the
// chunks g = c mod 4, all of a batch of kB at once (one round for up to 4 kB chunks); the four parts
// meet in LDS (red, 16 x 128 words).  Every thread of the workgroup must call it.
__device__ __forceinline__ void col_sums(const uint32_t* h, int G, int g_me, uint32_t* red, uint32_t* tot,
                                         uint32_t* pre) {
    constexpr int kB = 18;
    const int tid = threadIdx.x, t = tid & 127, cg = tid >> 7;  // (cg is uniform over a wave)
    uint32_t tl = 0, th = 0, pl = 0, ph = 0;
    for (int g0 = cg; g0 < G; g0 += 4 * kB) {
        uint32_t v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = g0 + 4 * u < G ? h[(g0 + 4 * u) * kTopkHistWords + t] : 0u;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const uint32_t lo = v[u] & 0xffffu, hi = v[u] >> 16;
            tl += lo;
            th += hi;
            pl += g0 + 4 * u < g_me ? lo : 0u;
            ph += g0 + 4 * u < g_me ? hi : 0u;
        }
    }
    red[(4 * cg + 0) * 128 + t] = tl;
    red[(4 * cg + 1) * 128 + t] = th;
    red[(4 * cg + 2) * 128 + t] = pl;
    red[(4 * cg + 3) * 128 + t] = ph;
    __syncthreads();
    if (tid < 128) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            tot[j] = red[j * 128 + t] + red[(4 + j) * 128 + t] + red[(8 + j) * 128 + t] + red[(12 + j) * 128 + t];
            pre[j] = red[(2 + j) * 128 + t] + red[(6 + j) * 128 + t] + red[(10 + j) * 128 + t] +
                     red[(14 + j) * 128 + t];
        }
    }
}

// the reduced LDS histogram hs[256] as one chunk's packed column (16-bit counts)
__device__ __forceinline__ void store_packed(const uint32_t* hs, uint32_t* col) {
    const int t = threadIdx.x;
    if (t < kTopkHistWords) col[t] = hs[2 * t] | (hs[2 * t + 1] << 16);
}

// After col_sums: lane l of wave 0 takes bins 4l .. 4l + 3 (words 2l, 2l + 1 of the packed columns) --
// their totals over every chunk and their sums over the chunks before g_me -- from col_sums' LDS parts.
__device__ __forceinline__ void col_quad(const uint32_t* red, int l, uint32_t* tot, uint32_t* pre) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int w = 2 * l + (j >> 1), hf = j & 1;
        tot[j] = red[hf * 128 + w] + red[(4 + hf) * 128 + w] + red[(8 + hf) * 128 + w] + red[(12 + hf) * 128 + w];
        pre[j] = red[(2 + hf) * 128 + w] + red[(6 + hf) * 128 + w] + red[(10 + hf) * 128 + w] +
                 red[(14 + hf) * 128 + w];
    }
}

// pick_digit on bins held in registers, four per lane of one wave (lane l: bins 4l .. 4l + 3); every lane
// of the wave gets the digit and the remainder.  0 < rem <= the bins' total, so one lane's bins hold it.
__device__ __forceinline__ void pick_digit_regs(const uint32_t* hq, uint32_t rem, uint32_t* digit,
                                                uint32_t* rem_out) {
    const int lane = threadIdx.x & 63;
    const uint32_t loc = hq[0] + hq[1] + hq[2] + hq[3];
    const uint32_t incl = wave_incl_scan(loc);
    const uint32_t above = wave_lane63(incl) - incl;
    const bool mine = above < rem && above + loc >= rem;
    uint32_t d = 0, ro = 0;
    if (mine) {
        uint32_t acc = above;
        for (int j = 3; j >= 0; --j) {
            if (acc + hq[j] >= rem) {
                d = 4 * lane + j;
                ro = rem - acc;
                break;
            }
            acc += hq[j];
        }
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(mine);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    *digit = (uint32_t)__builtin_amdgcn_readlane((int)d, src);
    *rem_out = (uint32_t)__builtin_amdgcn_readlane((int)ro, src);
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
    store_packed(hs, r.h1 + g * kTopkHistWords);
}

// Second digit: every chunk finds the high byte d1 from the column totals of h1 and counts the low
// bytes of its keys in bucket d1; it also leaves, for the third launch, the number of keys above
// d1 in the chunks before it.  Wave 0 finishes the column sums and picks d1 in registers; only
// bucket d1's keys are counted, so the low-byte histogram keeps four LDS copies (lane mod 4),
// cleared before the column sums' barrier.
__global__ void __launch_bounds__(kSplitThreads) topk_split_h2(TopkArgs a, int G) {
    const SplitRow r = split_row(a, G);
    const int g = blockIdx.x, tid = threadIdx.x;
    const int64_t lo = (int64_t)g * kChunk;
    __shared__ uint32_t red[16 * 128];  // the column sums' LDS
    __shared__ uint32_t hl[4 * 256];    // low-byte counts: bin b, copy c at 4 b + c
    __shared__ uint32_t d1, rem1, above1;
    for (int j = tid; j < 4 * 256; j += kSplitThreads) hl[j] = 0;
    uint32_t h[kBlk];
    load_lane_keys(r, lo, h);
    uint32_t t1[2] = {0u, 0u}, p1[2] = {0u, 0u};
    col_sums(r.h1, G, g, red, t1, p1);
    if (r.n <= r.K) return;  // (uniform) every candidate is kept: the emit launch lists them
    mask_lane_keys(lo, min(lo + kChunk, r.n), h);
    if (tid < 64) {
        uint32_t tq[4], pq[4], d, rm;
        col_quad(red, tid, tq, pq);
        pick_digit_regs(tq, (uint32_t)r.K, &d, &rm);
        uint32_t pa = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) pa += (uint32_t)(4 * tid + j) > d ? pq[j] : 0u;
        const uint32_t ab = wave_lane63(wave_incl_scan(pa));
        if (tid == 0) {
            d1 = d;
            rem1 = rm;
            above1 = ab;
        }
    }
    __syncthreads();
    const uint32_t hb = d1;
    // low bytes of the keys in bucket hb: keys above (hb, 0) - 1 and not above (hb, 255); the bucket
    // holds keys of one sign, so the low byte is the raw one, inverted for negatives
    const KeyCut in_lo = key_cut((int)(hb << 8) - 1), in_hi = key_cut((int)((hb << 8) | 255u));
    const uint32_t flip = hb >= 0x80u ? 0u : 255u;
    const int sub = tid & 3;
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
        const bool in = in_lo.gt(h[u]) && !in_hi.gt(h[u]);
        if (__builtin_amdgcn_ballot_w64(in) != 0 && in)
            atomicAdd(&hl[(((h[u] & 255u) ^ flip) << 2) + sub], 1u);
    }
    __syncthreads();
    if (tid == 0) *(u32x4*)(r.meta + 4 * g) = u32x4{above1, hb, rem1, 0u};
    if (tid < kTopkHistWords) {  // bins 2 tid and 2 tid + 1, packed
        const uint32_t* q = hl + 8 * tid;
        r.h2[g * kTopkHistWords + tid] = (q[0] + q[1] + q[2] + q[3]) | ((q[4] + q[5] + q[6] + q[7]) << 16);
    }
}

// Emission: the threshold key tau = (d1, d2) and the number rem of keys equal to it to keep; keys
// above tau are kept, keys equal to it in index order until rem are taken.  Where the indexer made
// h1, the workgroup clears its chunk of it for the next call.
__global__ void __launch_bounds__(kSplitThreads) topk_split_emit(TopkArgs a, int G) {
    const SplitRow r = split_row(a, G);
    const int g = blockIdx.x, tid = threadIdx.x;
    const int64_t lo = (int64_t)g * kChunk;
    const int kk = a.k;
    if (a.split_fused && tid < kTopkHistWords) r.h1[g * kTopkHistWords + tid] = 0u;
    // one round: this lane's keys, the second launch's figures and h2's columns
    uint32_t h[kBlk];
    load_lane_keys(r, lo, h);
    const u32x4 mt = *(const u32x4*)(r.meta + 4 * g);
    __shared__ uint32_t red[16 * 128];
    uint32_t t2[2] = {0u, 0u}, p2[2] = {0u, 0u};
    col_sums(r.h2, G, g, red, t2, p2);
    if (r.n <= r.K) {  // (uniform) fewer candidates than k: all of them, in order
        for (int64_t j = lo + tid; j < lo + kChunk && j < kk; j += kSplitThreads)
            r.out[j] = j < r.n ? (int32_t)j : -1;
        if (g == G - 1)
            for (int64_t j = (int64_t)G * kChunk + tid; j < kk; j += kSplitThreads) r.out[j] = j < r.n ? (int32_t)j : -1;
        return;
    }
    const int64_t hi = min(lo + kChunk, r.n);
    mask_lane_keys(lo, hi, h);
    // wave 0: the low byte d2 of tau from h2's column totals, and the keys above tau and equal to it in
    // the chunks before this one
    __shared__ uint32_t d2, rem2, bgt, beq;
    const uint32_t above1 = mt[0], d1 = mt[1], rem1 = mt[2];
    if (tid < 64) {
        uint32_t tq[4], pq[4], d, rm;
        col_quad(red, tid, tq, pq);
        pick_digit_regs(tq, rem1, &d, &rm);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gt += (uint32_t)(4 * tid + j) > d ? pq[j] : 0u;
            eq += (uint32_t)(4 * tid + j) == d ? pq[j] : 0u;
        }
        const uint32_t sg = wave_lane63(wave_incl_scan(gt)), se = wave_lane63(wave_incl_scan(eq));
        if (tid == 0) {
            d2 = d;
            rem2 = rm;
            bgt = sg;
            beq = se;
        }
    }
    __syncthreads();
    const uint32_t tau = (d1 << 8) | d2, rem = rem2;
    if (g == 0)
        for (int64_t j = r.K + tid; j < kk; j += kSplitThreads) r.out[j] = -1;
    // this wave's keys above tau and equal to it, then the waves before it
    const KeyCut cut = key_cut((int)tau);
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
        ngt += lane_count(cut.gt(h[u]));
        neq += lane_count(cut.eq(h[u]));
    }
    __shared__ uint32_t wgt[kSplitThreads / 64], weq[kSplitThreads / 64];
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if ((tid & 63) == 0) {
        wgt[wv] = ngt;
        weq[wv] = neq;
    }
    __syncthreads();
    uint32_t gt_run = above1 + bgt, eq_run = beq;
#pragma unroll
    for (int w = 0; w < kSplitThreads / 64; ++w) {
        gt_run += w < wv ? wgt[w] : 0u;
        eq_run += w < wv ? weq[w] : 0u;
    }
    gt_run = __builtin_amdgcn_readfirstlane(gt_run);  // (wave-uniform: kept in scalar registers)
    eq_run = __builtin_amdgcn_readfirstlane(eq_run);
    if (ngt + neq == 0) return;
    // the tests are made again below rather than kept: 64 lane masks would not fit the scalar registers
#pragma unroll
    for (int u = 0; u < kBlk; ++u) asm volatile("" : "+v"(h[u]));
    // in index order, 64 keys at a time: a key's list position is the keys above tau before it plus
    // the ties before it (at most rem); ties at or past rem are dropped
    const int64_t e = lane_first(lo);
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
        const bool gk = cut.gt(h[u]), qk = cut.eq(h[u]);
        const uint64_t gm = __builtin_amdgcn_ballot_w64(gk), qm = __builtin_amdgcn_ballot_w64(qk);
        if ((gm | qm) == 0) continue;
        const uint32_t gb = gt_run + lanes_below(gm), qb = eq_run + lanes_below(qm);
        const uint32_t pos = gb + min(qb, rem);  // < K for every kept key
        if ((gk | (qk & (qb < rem))) & (pos < (uint32_t)r.K)) r.out[pos] = (int32_t)(e + 64 * u);
        gt_run += (uint32_t)__builtin_popcountll(gm);
        eq_run += (uint32_t)__builtin_popcountll(qm);
    }
}

// split schedule for few long bf16 rows
static bool use_split(const TopkArgs& a, int64_t max_n) {
    const int64_t rows = (int64_t)a.B * a.T;
    return a.score_dtype == LCA_BF16 && rows < 128 && max_n > kSplitMin;
}

static int split_chunks(int64_t max_n) { return (int)((max_n + kChunk - 1) / kChunk); }

size_t topk_ws_bytes(int32_t B, int32_t T, int64_t s_stride, int32_t score_dtype) {
    TopkArgs a;
    a.B = B;
    a.T = T;
    a.score_dtype = score_dtype;
    if (!use_split(a, s_stride)) return 0;
    return (size_t)B * T * split_chunks(s_stride) * (2 * kTopkHistWords + 4) * sizeof(uint32_t);
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
        if (!a.split_fused) hipLaunchKernelGGL(topk_split_h1, grid, dim3(kSplitThreads), 0, st, a, G);
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
