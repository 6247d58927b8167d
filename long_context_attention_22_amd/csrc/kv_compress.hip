// kv_compress.hip -- the compressor of the DeepSeek-V4 hybrid attention
// ("DeepSeek-V4 中文翻译", sections 2.3.1 / 2.3.2 / 2.3.3): softmax-gated pooling
// with a per-position bias, RMSNorm, partial RoPE and the store (f32, bf16,
// fp8-e4m3fn with a power-of-two scale per 128 dims and bf16 RoPE dims, or
// MXFP4 for the indexer keys, section 5.2.1: E2M1 codes with one E8M0 scale
// per 32 dims).
//
// HBM-bound: every input element is read exactly once.  One workgroup per
// (entry, sequence); thread j owns channel j, so each wave reads 64
// consecutive channels of a row (one 128-byte line for bf16).  Pooling is an
// online softmax over the block's rows, eight rows in flight at a time.  The
// per-entry reductions (RMS, fp8 group max) and the RoPE pair exchange go
// through LDS.
#include "device.h"
#include "kernels.h"
#include "rowstore.h"

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

template <typename T, int FMT>
__global__ void __launch_bounds__(1024) kv_compress_kernel(CompressArgs a) {
    const int b = blockIdx.y;
    const int m = a.m;
    const int64_t p0 = a.first_pos.v[b];
    const int64_t s = a.s_lo.v[b] + blockIdx.x;
    const int64_t s_hi = (p0 + a.n_rows) / m;
    if (s >= s_hi) return;  // uniform over the workgroup

    const int d_nope = a.out.d_nope, d_rope = a.out.d_rope;
    const int c = d_nope + d_rope;
    const int j = threadIdx.x;
    const int lane = j & 63, wv = j >> 6;
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

hipError_t launch_kv_compress(const CompressArgs& a, hipStream_t st) {
    if (a.max_entries <= 0) return hipSuccess;
    const int c = a.out.d_nope + a.out.d_rope;
    dim3 grid((unsigned)a.max_entries, (unsigned)a.B);
    dim3 block((unsigned)((c + 63) / 64 * 64));
    const bool bf = a.in_dtype == LCA_BF16;
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
