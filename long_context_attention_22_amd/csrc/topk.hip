// topk.hip -- the top-k selector ("DeepSeek-V4 中文翻译" section 2.3.1; BF16
// index scores, section 5.2.1): per query row keep K = min(k, vis) entries
// with the largest scores, ties to the lower index, emitted in ascending
// index order and padded with -1.
//
// One 1024-thread workgroup per row.  Scores become monotone unsigned keys
// (bf16: 16 bits, f32: 32 bits; -0 folded onto +0).  An MSB-first radix
// select with 8-bit digits finds the K-th largest key tau and how many keys
// equal to tau are taken (the lowest-indexed ones): one LDS histogram pass
// per digit, with 16 sub-histograms (one per lane mod 16) so that lanes that
// share a bin rarely hit the same LDS word.  A final pass walks the row in
// index order and compacts the winners with a block-wide exclusive scan
// (wave shuffles + LDS), which yields ascending output and the
// lower-index tie rule directly.
#include "device.h"
#include "kernels.h"

namespace lca {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t mono_key(uint16_t h) {
    if (h == 0x8000u) h = 0;
    return (h & 0x8000u) ? (uint32_t)(~h & 0xffffu) : (uint32_t)(h | 0x8000u);
}
__device__ __forceinline__ uint32_t mono_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inclusive prefix sum over the workgroup; returns the inclusive value and the total
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
    for (int w = 0; w < kTopkWaves; ++w) {
        uint32_t x = wsum[w];
        off += w < wv ? x : 0u;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

template <typename TS, int BITS>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(TopkArgs a) {
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

    uint32_t prefix = 0;          // digits fixed so far (in place)
    uint32_t rem = (uint32_t)K;   // how many of the keys matching the prefix are still to take
#pragma unroll 1
    for (int shift = BITS - 8; shift >= 0; shift -= 8) {
        for (int j = tid; j < 256 * 16; j += kTopkThreads) hist[j] = 0;
        __syncthreads();
        const uint32_t hmask = (shift + 8 >= 32) ? 0u : (0xffffffffu << (shift + 8));
        for (int64_t e = tid; e < n; e += kTopkThreads) {
            const uint32_t key = mono_key(row[e]);
            if ((key & hmask) == (prefix & hmask))
                atomicAdd(&hist[((key >> shift) & 255u) * 16 + (lane & 15)], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t s = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) s += hist[tid * 16 + c];
            hsum[tid] = s;
        }
        __syncthreads();
        if (tid < 64) {
            // lane owns digits 4*lane .. 4*lane+3; suffix sums from the top digit down
            uint32_t h0 = hsum[4 * tid], h1 = hsum[4 * tid + 1], h2 = hsum[4 * tid + 2],
                     h3 = hsum[4 * tid + 3];
            uint32_t loc = h0 + h1 + h2 + h3;
            uint32_t suf = loc;  // sum over lanes >= tid
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                uint32_t nb = __shfl_down(suf, o, kWave);
                if (tid + o < 64) suf += nb;
            }
            const uint32_t above = suf - loc;  // keys in higher lanes' digits
            if (above < rem && suf >= rem) {
                uint32_t acc = above;
                uint32_t hs[4] = {h0, h1, h2, h3};
                for (int d = 3; d >= 0; --d) {
                    if (acc + hs[d] >= rem) {
                        sel_digit = 4 * tid + d;
                        sel_rem = rem - acc;
                        break;
                    }
                    acc += hs[d];
                }
            }
        }
        __syncthreads();
        prefix |= sel_digit << shift;
        rem = sel_rem;
        __syncthreads();
    }
    const uint32_t tau = prefix;   // the K-th largest key
    // rem = number of keys equal to tau to take (lowest indices first)

    // emit: each thread takes 8 consecutive elements per round, in index order
    uint32_t gt_base = 0, eq_base = 0;
    for (int64_t base = 0; base < n; base += 8 * kTopkThreads) {
        const int64_t e0 = base + 8 * (int64_t)tid;
        uint32_t keys[8];
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            keys[u] = (e0 + u < n) ? mono_key(row[e0 + u]) : 0u;
            const bool valid = e0 + u < n;
            ngt += (valid && keys[u] > tau) ? 1u : 0u;
            neq += (valid && keys[u] == tau) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t incl = block_incl_scan(ngt | (neq << 16), wsum, &tot);
        const uint32_t excl = incl - (ngt | (neq << 16));
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

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    dim3 grid((unsigned)a.T, (unsigned)a.B);
    if (a.score_dtype == LCA_BF16)
        hipLaunchKernelGGL((topk_kernel<uint16_t, 16>), grid, dim3(kTopkThreads), 0, st, a);
    else
        hipLaunchKernelGGL((topk_kernel<float, 32>), grid, dim3(kTopkThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lca
