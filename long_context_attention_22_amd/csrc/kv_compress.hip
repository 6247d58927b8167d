// kv_compress.hip -- the compressor of the DeepSeek-V4 hybrid attention
// ("DeepSeek-V4 中文翻译", sections 2.3.1 / 2.3.2 / 2.3.3): softmax-gated pooling
// with a per-position bias, RMSNorm, partial RoPE and the store (f32, bf16,
// fp8-e4m3fn with a power-of-two scale per 128 dims and bf16 RoPE dims, or
// MXFP4 for the indexer keys, section 5.2.1: E2M1 codes with one E8M0 scale
// per 32 dims).
//
// HBM-bound: every input element is read exactly once.  One workgroup per
// (entry, sequence).  bf16 inputs: each lane reads 16 bytes (8 channels) of a
// row, eight row slots side by side, each an online softmax over its share of
// the block's rows, merged through LDS (kv_pool_wide); other inputs: thread j
// owns channel j and walks the rows (kv_compress_kernel).  Then thread j owns
// channel j: the per-entry reductions (RMS, fp8 group max) and the RoPE pair
// exchange go through LDS.
#include "device.h"
#include "kernels.h"
#include "rowstore.h"
#include "trace.h"

namespace lca {

// online softmax over `cnt` rows (stride c) of one channel
template <typename T>
__device__ __forceinline__ void pool_rows(const T* zp, const T* cp, const float* bp, int cnt, int c,
                                          float& mx, float& den, float& num) {
    for (int i0 = 0; i0 < cnt; i0 += 8) {
        float lz[8], lc[8];
        const int n = min(8, cnt - i0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u < n) {
                const int64_t off = (int64_t)(i0 + u) * c;
                lz[u] = ldin(zp, off) + (bp ? bp[off] : 0.0f);
                lc[u] = ldin(cp, off);
            }
        }
        float cm = lz[0];
#pragma unroll
        for (int u = 1; u < 8; ++u)
            if (u < n) cm = fmaxf(cm, lz[u]);
        const float nm = fmaxf(mx, cm);
        const float corr = __expf(mx - nm);
        den *= corr;
        num *= corr;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u < n) {
                const float e = __expf(lz[u] - nm);
                den += e;
                num = fmaf(e, lc[u], num);
            }
        }
        mx = nm;
    }
}

// The rest of an entry once its pooled value y of channel j (thread j < c) is known: RMSNorm over all
// c dims, RoPE at position s m, the store.  red: 16 floats of LDS, ys: 1024.
template <int FMT>
__device__ __forceinline__ void finish_entry(const CompressArgs& a, float y, int b, int64_t s, float* red, float* ys) {
    const int m = a.m;
    const int d_nope = a.out.d_nope, d_rope = a.out.d_rope;
    const int c = d_nope + d_rope;
    const int j = threadIdx.x;
    const int lane = j & 63, wv = j >> 6;
    if (a.gamma) {  // RMSNorm over all c dims
        float ss = wave_sum(y * y);
        if (lane == 0) red[wv] = ss;
        __syncthreads();
        float tot = 0.0f;
        for (int w = 0; w < (int)((blockDim.x + 63) >> 6); ++w) tot += red[w];
        if (j < c) y = a.gamma[j] * y * (1.0f / sqrtf(tot / (float)c + a.eps));
        __syncthreads();
    }

    if (a.rope_theta != 0.0 && d_rope > 0) {
        ys[j] = y;
        __syncthreads();
        if (j >= d_nope && j < c) {
            const int half = d_rope >> 1;
            const int r = j - d_nope;
            const int i = r < half ? r : r - half;
            float sn, cs;
            rope_sincos(a.rope.inv, i, (double)(s * m), &sn, &cs);
            if (r < half) y = y * cs - ys[j + half] * sn;
            else y = ys[j - half] * sn + y * cs;
        }
    }

    const int64_t row = (int64_t)b * a.out.cap + (a.ring ? s % a.out.cap : s);
    if (FMT == LCA_FP8) {
        // power-of-two scale per 128 nope dims: smallest 2^k with amax <= 448 * 2^k
        float am = wave_max(j < d_nope ? fabsf(y) : 0.0f);
        if (lane == 0) red[wv] = am;
        __syncthreads();
        if (j < d_nope) {
            const int g = j >> 7;
            const float amax = fmaxf(red[2 * g], red[2 * g + 1]);
            int ex = 0;
            float scale = 1.0f;
            if (amax > 0.0f) {
                frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
                const int e = ex - 1;
                scale = (amax <= ldexpf(1.75f, e)) ? ldexpf(1.0f, e - 8) : ldexpf(1.0f, e - 7);
            }
            const float inv = 1.0f / scale;  // exact: power of two
            ((uint8_t*)a.out.nope)[row * d_nope + j] = (uint8_t)f32_to_fp8(y * inv);
            if ((j & 127) == 0) ((float*)a.out.scale)[row * (d_nope >> 7) + g] = scale;
        } else if (j < c) {
            ((uint16_t*)a.out.rope)[row * d_rope + (j - d_nope)] = f2bf(y);
        }
    } else if (FMT == LCA_MXFP4) {  // d_rope == 0, c % 32 == 0: a 32-channel block is half a wave
        mxfp4_store_lane(y, j < c, (uint8_t*)a.out.scale + row * (c >> 5), j >> 5,
                         (uint32_t*)a.out.nope + row * (c >> 3), j >> 3);
    } else if (FMT == LCA_BF16) {
        if (j < d_nope) ((uint16_t*)a.out.nope)[row * d_nope + j] = f2bf(y);
        else if (j < c) ((uint16_t*)a.out.rope)[row * d_rope + (j - d_nope)] = f2bf(y);
    } else {
        if (j < d_nope) ((float*)a.out.nope)[row * d_nope + j] = y;
        else if (j < c) ((float*)a.out.rope)[row * d_rope + (j - d_nope)] = y;
    }
}

// One workgroup per (entry, sequence), thread j = channel j: the pooling walks the block's rows one
// channel per thread (any input type and width).
template <typename T, int FMT>
__global__ void __launch_bounds__(1024) kv_compress_kernel(CompressArgs a) {
    const int b = blockIdx.y;
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t s = a.s_lo.v[b] + blockIdx.x;
    const int64_t s_hi = (p0 + a.n_rows) / m;
    if (s >= s_hi) return;  // uniform over the workgroup
    const int c = a.out.d_nope + a.out.d_rope;
    const int j = threadIdx.x;
    __shared__ float red[16];
    __shared__ float ys[1024];
    float y = 0.0f;
    if (j < c) {
        float mx = -INFINITY, den = 0.0f, num = 0.0f;
        const int64_t ra = (int64_t)b * a.in_stride + (s * m - p0);
        pool_rows<T>((const T*)a.z_a + ra * c + j, (const T*)a.c_a + ra * c + j,
                     a.bias_a ? a.bias_a + j : nullptr, m, c, mx, den, num);
        if (a.overlap && s >= 1) {
            const int64_t rb = ra - m;
            pool_rows<T>((const T*)a.z_b + rb * c + j, (const T*)a.c_b + rb * c + j,
                         a.bias_b ? a.bias_b + j : nullptr, m, c, mx, den, num);
        }
        y = num / den;
    }
    finish_entry<FMT>(a, y, b, s, red, ys);
}

// bf16 inputs, c a multiple of 8 (at most kPoolMaxC): the block's rows are read 16 bytes (8 channels) per
// lane.  Thread t = (row slot rs = t / (c / 8), chunk ch = t % (c / 8)) pools channels 8 ch .. 8 ch + 7
// over the rows rs, rs + kPoolSlots, ... of the entry's row list (the a-block's m rows, then the
// b-block's m rows when overlapping), kPoolRows rows' loads (C, Z and the bias rows) in flight at a time,
// as an online softmax per channel; the kPoolSlots partial states (max, sum, weighted sum) of a
// channel are merged through LDS in slot order, then thread j < c finishes channel j as above.  Each
// wave moves 1 KB per load instruction instead of 128 bytes, and a row is read by c / 8 lanes side by
// side.
constexpr int kPoolSlots = 8;
constexpr int kPoolRows = 4;    // rows whose loads a thread has in flight at once (registers: 16 each)
constexpr int kPoolMaxC = 576;  // (the merge's LDS: 3 x 8 x 576 floats, so two workgroups fit a CU)
constexpr int kPairRows = 2;    // kv_pool_pair: rows of each of its two entries in flight at once
constexpr int64_t kPoolPairMin = 512;  // (entry, sequence) pairs from which kv_pool_pair serves a call

// One row of a thread's 8 channels into their online-softmax states: zw, cw the row's Z and C values (bf16
// pairs), bs its 8 bias values.
__device__ __forceinline__ void pool_row(const u32x4& zw4, const u32x4& cw4, const f32x4* bs, float* mx, float* den,
                                         float* num) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t zw = zw4[i >> 1], cw = cw4[i >> 1];
        const float z = __uint_as_float((i & 1) ? (zw & 0xffff0000u) : (zw << 16)) + bs[i >> 2][i & 3];
        const float cv = __uint_as_float((i & 1) ? (cw & 0xffff0000u) : (cw << 16));
        // lazy rescaling: the reference moves only when a logit exceeds it by more than 16
        // (weights stay <= e^16), so most rows cost one exponential instead of two
        if (z > mx[i] + 16.0f) {
            const float corr = __expf(mx[i] - z);  // (reference -inf: 0)
            den[i] *= corr;
            num[i] *= corr;
            mx[i] = z;
        }
        const float e = __expf(z - mx[i]);
        den[i] += e;
        num[i] = fmaf(e, cv, num[i]);
    }
}

// Online softmax of this thread's rows k_lo + rs, k_lo + rs + kPoolSlots, ... (below k_hi) of entry s's row
// list, channels 8 ch .. 8 ch + 7, NR rows' loads in flight at a time.
template <int NR>
__device__ __forceinline__ void pool_wide_rows(const CompressArgs& a, int b, int64_t s, int k_lo, int k_hi, int rs,
                                               int ch, int c, float* mx, float* den, float* num) {
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t ra = (int64_t)b * a.in_stride + (s * m - p0);  // the a-block's first row
    for (int k0 = k_lo + rs; k0 < k_hi; k0 += NR * kPoolSlots) {
        u32x4 zc[NR][2];
        f32x4 bs[NR][2];
        bool ok[NR];
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            const int k = k0 + u * kPoolSlots;
            ok[u] = k < k_hi;
            // b-block row k - m (block s - 1); a slot past the range reads the a-block's first row (in
            // range, dropped below)
            const bool bb = ok[u] && k >= m;
            const int i = ok[u] ? (bb ? k - m : k) : 0;
            const int64_t row = ra + (bb ? i - m : i);
            const uint16_t* zp = (const uint16_t*)(bb ? a.z_b : a.z_a) + row * c + 8 * ch;
            const uint16_t* cp = (const uint16_t*)(bb ? a.c_b : a.c_a) + row * c + 8 * ch;
            const float* bp = bb ? a.bias_b : a.bias_a;
            // C and Z rows are read by this entry only: non-temporal, so they do not push the bias
            // rows (read by every entry) out of the caches
            zc[u][0] = __builtin_nontemporal_load((const u32x4*)zp);
            zc[u][1] = __builtin_nontemporal_load((const u32x4*)cp);
            if (bp) {
                bs[u][0] = *(const f32x4*)(bp + (int64_t)i * c + 8 * ch);
                bs[u][1] = *(const f32x4*)(bp + (int64_t)i * c + 8 * ch + 4);
            } else {
                bs[u][0] = bs[u][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
#pragma unroll
        for (int u = 0; u < NR; ++u)
            if (ok[u]) pool_row(zc[u][0], zc[u][1], bs[u], mx, den, num);
    }
}

// Two consecutive entries s, s + 1 of a call without overlap (each list is its own block's m rows), as
// pool_wide_rows for each, with each bias row loaded once for both: the rows of entry s + 1 are m rows
// further.  two = false (s + 1 past the call's entries): the second state repeats the first entry's rows
// and is dropped.
template <int NR>
__device__ __forceinline__ void pool_pair_rows(const CompressArgs& a, int b, int64_t s, bool two, int rs, int ch,
                                               int c, float* mx, float* den, float* num, float* mx2, float* den2,
                                               float* num2) {
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t ra = (int64_t)b * a.in_stride + (s * m - p0);  // entry s's first row
    const int64_t d2 = two ? (int64_t)m * c : 0;                 // entry s + 1's rows, in elements
    for (int k0 = rs; k0 < m; k0 += NR * kPoolSlots) {
        u32x4 zc[NR][4];
        f32x4 bs[NR][2];
        bool ok[NR];
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            const int k = k0 + u * kPoolSlots;
            ok[u] = k < m;
            const int i = ok[u] ? k : 0;  // a slot past the block reads its first row (dropped below)
            const uint16_t* zp = (const uint16_t*)a.z_a + (ra + i) * c + 8 * ch;
            const uint16_t* cp = (const uint16_t*)a.c_a + (ra + i) * c + 8 * ch;
            zc[u][0] = __builtin_nontemporal_load((const u32x4*)zp);
            zc[u][1] = __builtin_nontemporal_load((const u32x4*)cp);
            zc[u][2] = __builtin_nontemporal_load((const u32x4*)(zp + d2));
            zc[u][3] = __builtin_nontemporal_load((const u32x4*)(cp + d2));
            if (a.bias_a) {
                bs[u][0] = *(const f32x4*)(a.bias_a + (int64_t)i * c + 8 * ch);
                bs[u][1] = *(const f32x4*)(a.bias_a + (int64_t)i * c + 8 * ch + 4);
            } else {
                bs[u][0] = bs[u][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
#pragma unroll
        for (int u = 0; u < NR; ++u)
            if (ok[u]) {
                pool_row(zc[u][0], zc[u][1], bs[u], mx, den, num);
                pool_row(zc[u][2], zc[u][3], bs[u], mx2, den2, num2);
            }
    }
}

// The kPoolSlots row slots' states of each channel through LDS; thread t < c gets channel t's merged state
// (reference M, sum dn, weighted sum nu; slots added in slot order).  Every thread must call it.
__device__ __forceinline__ void merge_slots(float (*st)[kPoolSlots][kPoolMaxC], int rs, int ch, int c,
                                            const float* mx, const float* den, const float* num, float& M,
                                            float& dn, float& nu) {
    const int t = threadIdx.x;
    if (rs < kPoolSlots) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            st[0][rs][8 * ch + i] = mx[i];
            st[1][rs][8 * ch + i] = den[i];
            st[2][rs][8 * ch + i] = num[i];
        }
    }
    __syncthreads();
    M = -INFINITY;
    dn = nu = 0.0f;
    if (t < c) {
#pragma unroll
        for (int r = 0; r < kPoolSlots; ++r) M = fmaxf(M, st[0][r][t]);
#pragma unroll
        for (int r = 0; r < kPoolSlots; ++r) {
            const float w = st[0][r][t] == -INFINITY ? 0.0f : __expf(st[0][r][t] - M);
            dn = fmaf(st[1][r][t], w, dn);
            nu = fmaf(st[2][r][t], w, nu);
        }
    }
}

// bf16 inputs, c a multiple of 8 (at most kPoolMaxC): the block's rows are read 16 bytes (8 channels) per
// lane.  Thread t = (row slot rs = t / (c / 8), chunk ch = t % (c / 8)) pools channels 8 ch .. 8 ch + 7
// over the rows rs, rs + kPoolSlots, ... of the entry's row list (the a-block's m rows, then the
// b-block's m rows when overlapping), NR rows' loads (C, Z and the bias rows) in flight at a time, as
// an online softmax per channel; the kPoolSlots partial states (max, sum, weighted sum) of a channel are
// merged through LDS in slot order, then thread j < c finishes channel j as above.  Each wave moves 1 KB
// per load instruction instead of 128 bytes, and a row is read by c / 8 lanes side by side.  NR is
// kPoolRows for long row lists and the rows a slot holds for short ones (a CSA entry's 8 rows are one per
// slot), so that no thread issues padding loads and two workgroups share a CU (the 4096-token chunk's CSA
// call, 1,024 entries: 25.7 -> 23.1 us).  An HCA entry's 128 rows are 16 per slot, four rounds of
// kPoolRows = 4 (115 VGPRs, one workgroup per CU); with the C / Z loads non-temporal a 65,536-row call
// took 38.9 us this way against 41.4 us at six rows in flight (three rounds, two of the 18 row loads
// padding) and 39.5 us at three -- such calls now go to kv_pool_pair below (35 us).
template <int FMT, int NR>
__global__ void __launch_bounds__(kPoolMaxC, NR <= 2 ? 5 : 1) kv_pool_wide(CompressArgs a) {
    const int b = blockIdx.y;
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t s = a.s_lo.v[b] + blockIdx.x;
    const int64_t s_hi = (p0 + a.n_rows) / m;
    if (s >= s_hi) return;  // uniform over the workgroup
    const int c = a.out.d_nope + a.out.d_rope;
    const int nch = c >> 3;
    const int t = threadIdx.x;
    const int rs = t / nch, ch = t - rs * nch;
    __shared__ float red[16];
    __shared__ float ys[1024];
    __shared__ float st[3][kPoolSlots][kPoolMaxC];  // reference, sum, weighted sum of (slot, channel)
    const int L = (a.overlap && s >= 1) ? 2 * m : m;  // rows of the entry's list
    float mx[8], den[8], num[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx[i] = -INFINITY;
        den[i] = 0.0f;
        num[i] = 0.0f;
    }
    pool_wide_rows<NR>(a, b, s, 0, L, rs, ch, c, mx, den, num);
    float M, dn, nu;
    merge_slots(st, rs, ch, c, mx, den, num, M, dn, nu);
    const float y = t < c ? nu / dn : 0.0f;
    finish_entry<FMT>(a, y, b, s, red, ys);
}

// Many entries of long blocks without overlap (a prefill's m = 128 blocks: kPoolPairMin or more (entry,
// sequence) pairs): one workgroup per two consecutive entries (grid (ceil(entries / 2), B)), each row slot
// of a thread pooling both through pool_pair_rows, so that the bias rows -- the same for every entry, twice
// the bytes of its C and Z rows in f32 -- are read once per two entries; then kv_pool_wide's merge and
// finish for the first entry and for the second.  A 65,536-row call: 256 workgroups, one per CU.
template <int FMT, int NR>
__global__ void __launch_bounds__(kPoolMaxC, 1) kv_pool_pair(CompressArgs a) {
    const int b = blockIdx.y;
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t s = a.s_lo.v[b] + 2 * (int64_t)blockIdx.x;
    const int64_t s_hi = (p0 + a.n_rows) / m;
    if (s >= s_hi) return;            // uniform over the workgroup
    const bool two = s + 1 < s_hi;    // (uniform too)
    const int c = a.out.d_nope + a.out.d_rope;
    const int nch = c >> 3;
    const int t = threadIdx.x;
    const int rs = t / nch, ch = t - rs * nch;
    __shared__ float red[16];
    __shared__ float ys[1024];
    __shared__ float st[3][kPoolSlots][kPoolMaxC];
    float mx[8], den[8], num[8], mx2[8], den2[8], num2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx[i] = mx2[i] = -INFINITY;
        den[i] = den2[i] = 0.0f;
        num[i] = num2[i] = 0.0f;
    }
    pool_pair_rows<NR>(a, b, s, two, rs, ch, c, mx, den, num, mx2, den2, num2);
    float M, dn, nu;
    merge_slots(st, rs, ch, c, mx, den, num, M, dn, nu);
    finish_entry<FMT>(a, t < c ? nu / dn : 0.0f, b, s, red, ys);
    if (!two) return;
    __syncthreads();  // every thread is past the first merge's reads of st and the first finish's of red, ys
    merge_slots(st, rs, ch, c, mx2, den2, num2, M, dn, nu);
    finish_entry<FMT>(a, t < c ? nu / dn : 0.0f, b, s + 1, red, ys);
}

// Few entries (a 4096-token chunk's m = 128 blocks: 32 workgroups of kv_pool_wide would leave most of the
// GPU idle): with a workspace the call cuts each entry's row list into a.parts ranges of a.part_len rows,
// one workgroup each (kv_pool_part, grid (entries x parts, B)), which stores the range's merged state of
// every channel -- reference, sum, weighted sum: ws[((b E + e) parts + p)][3][c], E = a.max_entries --
// and kv_pool_finish (grid (entries, B)) merges an entry's parts in part order and finishes it.  NR: a part's
// rows per row slot (part_len / kPoolSlots, rounded up) when that is 1 or 2, else kPoolRows.
template <int NR>
__global__ void __launch_bounds__(kPoolMaxC) kv_pool_part(CompressArgs a) {
    const int b = blockIdx.y;
    const int P = a.parts;
    const int e = (int)(blockIdx.x / (uint32_t)P), p = (int)(blockIdx.x - (uint32_t)e * (uint32_t)P);
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t s = a.s_lo.v[b] + e;
    const int64_t s_hi = (p0 + a.n_rows) / m;
    if (s >= s_hi) return;  // uniform over the workgroup
    const int c = a.out.d_nope + a.out.d_rope;
    const int nch = c >> 3;
    const int t = threadIdx.x;
    const int rs = t / nch, ch = t - rs * nch;
    __shared__ float st[3][kPoolSlots][kPoolMaxC];
    const int L = (a.overlap && s >= 1) ? 2 * m : m;
    const int k_lo = p * a.part_len, k_hi = min(L, k_lo + a.part_len);  // (an empty range stores -inf, 0, 0)
    float mx[8], den[8], num[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx[i] = -INFINITY;
        den[i] = 0.0f;
        num[i] = 0.0f;
    }
    pool_wide_rows<NR>(a, b, s, k_lo, k_hi, rs, ch, c, mx, den, num);
    float M, dn, nu;
    merge_slots(st, rs, ch, c, mx, den, num, M, dn, nu);
    if (t < c) {
        float* w = a.ws + (((int64_t)b * a.max_entries + e) * P + p) * 3 * c;
        w[t] = M;
        w[c + t] = dn;
        w[2 * c + t] = nu;
    }
}

template <int FMT>
__global__ void __launch_bounds__(kPoolMaxC) kv_pool_finish(CompressArgs a) {
    const int b = blockIdx.y, e = blockIdx.x;
    const int P = a.parts;
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t s = a.s_lo.v[b] + e;
    const int64_t s_hi = (p0 + a.n_rows) / m;
    if (s >= s_hi) return;  // uniform over the workgroup
    const int c = a.out.d_nope + a.out.d_rope;
    const int t = threadIdx.x;
    __shared__ float red[16];
    __shared__ float ys[1024];
    float y = 0.0f;
    if (t < c) {
        // every part's state in one round of loads (parts past P read part 0 and are dropped)
        const float* w = a.ws + ((int64_t)b * a.max_entries + e) * P * 3 * c + t;
        float mp[kCompressMaxParts], dp[kCompressMaxParts], np[kCompressMaxParts];
#pragma unroll
        for (int p = 0; p < kCompressMaxParts; ++p) {
            const float* wp = w + (p < P ? p : 0) * 3 * c;
            mp[p] = wp[0];
            dp[p] = wp[c];
            np[p] = wp[2 * c];
        }
        float M = -INFINITY;
#pragma unroll
        for (int p = 0; p < kCompressMaxParts; ++p) M = p < P ? fmaxf(M, mp[p]) : M;
        float dn = 0.0f, nu = 0.0f;
#pragma unroll
        for (int p = 0; p < kCompressMaxParts; ++p) {
            const float wt = p >= P || mp[p] == -INFINITY ? 0.0f : __expf(mp[p] - M);
            dn = fmaf(dp[p], wt, dn);
            nu = fmaf(np[p], wt, nu);
        }
        y = nu / dn;
    }
    finish_entry<FMT>(a, y, b, s, red, ys);
}

// m = 1 (the window / state-cache store, [R] 2.3.3 and 3.5.1): the softmax over one position is 1,
// so the entry is the row itself, then RMSNorm, RoPE and the store.  One wave per row, lane l
// owns channels l + 64 j (j < J): every reduction is a wave reduction.  This store is one small
// launch per layer and decode token, so its latency is what counts: every argument is read at
// the top, before the first branch (the scalar loads go out in one batch instead of a chain of
// round trips), and the row, gamma and the RoPE frequencies are loaded in one round.
template <typename T, int FMT, int J>
__global__ void __launch_bounds__(64) kv_store_rows(CompressArgs a) {
    const int b = blockIdx.y, lane = threadIdx.x;
    const int64_t p0 = a.first_pos.v[b], s = a.s_lo.v[b] + blockIdx.x, n_rows = a.n_rows;
    const int d_nope = a.out.d_nope, d_rope = a.out.d_rope, c = d_nope + d_rope;
    const int64_t in_stride = a.in_stride, cap = a.out.cap;
    const T* c_a = (const T*)a.c_a;
    const float* gamma = a.gamma;
    const float eps = a.eps;
    const bool rope = a.rope_theta != 0.0 && d_rope > 0;
    const int ring = a.ring;
    void* const onope = a.out.nope;
    void* const orope = a.out.rope;
    void* const oscale = a.out.scale;
    const int half = d_rope >> 1;
    // this lane's RoPE pair index (channel d_nope + lane, when lane < d_rope <= 64)
    const int ri = half > 0 ? (lane < half ? lane : lane - half) : 0;
    const double inv = a.rope.inv[ri < kMaxRopeHalf ? ri : 0];
    asm volatile("" ::"s"(p0), "s"(s), "s"(n_rows), "s"(d_nope), "s"(d_rope), "s"(in_stride), "s"(cap), "s"(c_a),
                 "s"(gamma), "s"(eps), "s"(ring), "s"(onope), "s"(orope), "s"(oscale));
    // (a workgroup past the last row reads row 0 of its sequence and stores nothing)
    const bool live = s < p0 + n_rows;
    const T* src = c_a + ((int64_t)b * in_stride + (live ? s - p0 : 0)) * c;
    RowOut<J> o;
    float g[J];
    row_load<T, J>(src, gamma, c, o.y, g);
    if (!live) return;
    __shared__ float ys[64 * J];
    const int64_t row = (int64_t)b * cap + (ring ? s % cap : s);
    row_prepare<FMT, J>(o, g, gamma, eps, c, d_nope, d_rope, rope, inv, (double)s, ys, nullptr);
    row_commit<FMT, J>(o, c, d_nope, d_rope, onope, orope, oscale, row);
}

template <typename T, int FMT>
static void launch_store_rows(const CompressArgs& a, int c, dim3 grid, hipStream_t st) {
    if (c <= 64) hipLaunchKernelGGL((kv_store_rows<T, FMT, 1>), grid, dim3(64), 0, st, a);
    else if (c <= 128) hipLaunchKernelGGL((kv_store_rows<T, FMT, 2>), grid, dim3(64), 0, st, a);
    else if (c <= 576) hipLaunchKernelGGL((kv_store_rows<T, FMT, 9>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((kv_store_rows<T, FMT, 16>), grid, dim3(64), 0, st, a);
}

template <int FMT>
static void launch_pool_wide(int per_slot, dim3 grid, dim3 block, hipStream_t st, const CompressArgs& a) {
    if (per_slot <= 1) hipLaunchKernelGGL((kv_pool_wide<FMT, 1>), grid, block, 0, st, a);
    else if (per_slot <= 2) hipLaunchKernelGGL((kv_pool_wide<FMT, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kv_pool_wide<FMT, kPoolRows>), grid, block, 0, st, a);
}

hipError_t launch_kv_compress(const CompressArgs& a, hipStream_t st) {
    if (a.max_entries <= 0) return hipSuccess;
    const int c = a.out.d_nope + a.out.d_rope;
    dim3 grid((unsigned)a.max_entries, (unsigned)a.B);
    dim3 block((unsigned)((c + 63) / 64 * 64));
    const bool bf = a.in_dtype == LCA_BF16;
    if (trace_on())
        trace("  compress: %s grid (%u, %u), %lld entr%s per sequence", a.m == 1 && !a.overlap && a.out.d_rope <= 64
              ? "kv_store_rows" : bf && c % 8 == 0 && c <= kPoolMaxC ? "kv_pool_wide" : "kv_compress_kernel", grid.x, grid.y,
              (long long)a.max_entries, a.max_entries == 1 ? "y" : "ies");
    if (a.m == 1 && !a.overlap && a.out.d_rope <= 64) {
        switch (a.out.fmt) {
            case LCA_F32:
                if (bf) launch_store_rows<uint16_t, LCA_F32>(a, c, grid, st);
                else launch_store_rows<float, LCA_F32>(a, c, grid, st);
                break;
            case LCA_BF16:
                if (bf) launch_store_rows<uint16_t, LCA_BF16>(a, c, grid, st);
                else launch_store_rows<float, LCA_BF16>(a, c, grid, st);
                break;
            case LCA_MXFP4:
                if (bf) launch_store_rows<uint16_t, LCA_MXFP4>(a, c, grid, st);
                else launch_store_rows<float, LCA_MXFP4>(a, c, grid, st);
                break;
            default:
                if (bf) launch_store_rows<uint16_t, LCA_FP8>(a, c, grid, st);
                else launch_store_rows<float, LCA_FP8>(a, c, grid, st);
                break;
        }
        return hipGetLastError();
    }
    if (bf && c % 8 == 0 && c <= kPoolMaxC) {
        const dim3 wblock((unsigned)(c / 8 * kPoolSlots));
        if (a.parts > 1) {  // few entries, with a workspace: the rows of an entry over a.parts workgroups
            if (trace_on()) trace("  compress: kv_pool_part grid (%lld, %u) + kv_pool_finish, %d parts of %d rows",
                                  (long long)a.max_entries * a.parts, grid.y, a.parts, a.part_len);
            const dim3 pgrid((unsigned)(a.max_entries * a.parts), grid.y);
            const int nr = (a.part_len + kPoolSlots - 1) / kPoolSlots;
            if (nr == 1) hipLaunchKernelGGL(kv_pool_part<1>, pgrid, wblock, 0, st, a);
            else if (nr == 2) hipLaunchKernelGGL(kv_pool_part<2>, pgrid, wblock, 0, st, a);
            else hipLaunchKernelGGL(kv_pool_part<kPoolRows>, pgrid, wblock, 0, st, a);
            switch (a.out.fmt) {
                case LCA_F32: hipLaunchKernelGGL((kv_pool_finish<LCA_F32>), grid, wblock, 0, st, a); break;
                case LCA_BF16: hipLaunchKernelGGL((kv_pool_finish<LCA_BF16>), grid, wblock, 0, st, a); break;
                case LCA_MXFP4: hipLaunchKernelGGL((kv_pool_finish<LCA_MXFP4>), grid, wblock, 0, st, a); break;
                default: hipLaunchKernelGGL((kv_pool_finish<LCA_FP8>), grid, wblock, 0, st, a); break;
            }
            return hipGetLastError();
        }
        const int per_slot = (a.m * (1 + a.overlap) + kPoolSlots - 1) / kPoolSlots;  // rows per slot, at most
        if (!a.overlap && per_slot > 2 && a.max_entries * a.B >= kPoolPairMin) {
            const dim3 pgrid((unsigned)((a.max_entries + 1) / 2), grid.y);
            if (trace_on()) trace("  compress: kv_pool_pair grid (%u, %u)", pgrid.x, pgrid.y);
            switch (a.out.fmt) {
                case LCA_F32: hipLaunchKernelGGL((kv_pool_pair<LCA_F32, kPairRows>), pgrid, wblock, 0, st, a); break;
                case LCA_BF16: hipLaunchKernelGGL((kv_pool_pair<LCA_BF16, kPairRows>), pgrid, wblock, 0, st, a); break;
                case LCA_MXFP4: hipLaunchKernelGGL((kv_pool_pair<LCA_MXFP4, kPairRows>), pgrid, wblock, 0, st, a); break;
                default: hipLaunchKernelGGL((kv_pool_pair<LCA_FP8, kPairRows>), pgrid, wblock, 0, st, a); break;
            }
            return hipGetLastError();
        }
        switch (a.out.fmt) {
            case LCA_F32: launch_pool_wide<LCA_F32>(per_slot, grid, wblock, st, a); break;
            case LCA_BF16: launch_pool_wide<LCA_BF16>(per_slot, grid, wblock, st, a); break;
            case LCA_MXFP4: launch_pool_wide<LCA_MXFP4>(per_slot, grid, wblock, st, a); break;
            default: launch_pool_wide<LCA_FP8>(per_slot, grid, wblock, st, a); break;
        }
        return hipGetLastError();
    }
    switch (a.out.fmt) {
        case LCA_F32:
            if (bf) hipLaunchKernelGGL((kv_compress_kernel<uint16_t, LCA_F32>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((kv_compress_kernel<float, LCA_F32>), grid, block, 0, st, a);
            break;
        case LCA_BF16:
            if (bf) hipLaunchKernelGGL((kv_compress_kernel<uint16_t, LCA_BF16>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((kv_compress_kernel<float, LCA_BF16>), grid, block, 0, st, a);
            break;
        case LCA_MXFP4:
            if (bf) hipLaunchKernelGGL((kv_compress_kernel<uint16_t, LCA_MXFP4>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((kv_compress_kernel<float, LCA_MXFP4>), grid, block, 0, st, a);
            break;
        default:
            if (bf) hipLaunchKernelGGL((kv_compress_kernel<uint16_t, LCA_FP8>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((kv_compress_kernel<float, LCA_FP8>), grid, block, 0, st, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace lca
