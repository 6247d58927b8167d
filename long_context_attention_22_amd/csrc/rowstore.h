// rowstore.h -- one raw row through the compressor's m = 1 store ("DeepSeek-V4 中文翻译" sections
// 2.3.3 and 3.5.1: the sliding-window / state-cache rows): the softmax over a single position is
// 1, so the entry is the row itself; then RMSNorm over all c dims, RoPE on the last d_rope dims at
// the row's position, and the store (f32, bf16, fp8-e4m3fn with a power-of-two scale per 128 nope
// dims and bf16 RoPE dims, or MXFP4).  One wave does a row; lane l owns channels l + 64 j (j < J),
// so every reduction is a wave reduction.  Used by the compressor's m = 1 kernel and by the decode
// attention, which stores its query row's window row itself.
#pragma once
#include "device.h"
#include "kernels.h"

namespace lca {

template <typename T>
__device__ __forceinline__ float ldin(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ldin<float>(const float* p, int64_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ float ldin<uint16_t>(const uint16_t* p, int64_t i) {
    return bf2f(p[i]);
}

// The row's c values and gamma (branch-free: channels past c load channel c - 1 and become 0).
template <typename T, int J>
__device__ __forceinline__ void row_load(const T* src, const float* gamma, int c, float (&y)[J], float (&g)[J]) {
    // (the first J values of RowOut<J> are its y: callers pass o.y)
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int ch = lane + 64 * j;
        const float v = ldin(src, ch < c ? ch : c - 1);
        y[j] = ch < c ? v : 0.0f;
    }
    if (gamma) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            const float v = gamma[ch < c ? ch : c - 1];
            g[j] = ch < c ? v : 0.0f;
        }
    }
}

// The row after RMSNorm and RoPE, with the fp8 group scales: what row_commit stores.
template <int J>
struct RowOut {
    float y[J];
    float isc[J / 2 + 1], scl[J / 2 + 1];  // fp8: 1 / scale and scale per 128 nope dims (exact)
};

// RMSNorm (gamma != NULL) and RoPE at position pos (rope; inv = this lane's pair frequency
// theta^(-2i/d_rope), i = lane mod d_rope/2; d_rope <= 64) through the LDS scratch ys[64 J] of this
// wave, and the fp8 group scales.  dec != NULL: the values as stored, decoded (an fp8 code times
// its scale, exact in bf16), also go to dec[ch] as bf16 (f32 / bf16 / fp8 formats).  Called by one
// whole wave; it synchronises only that wave (LDS accesses of one wave are ordered).  No global
// memory is written here, so a caller can keep its loads in flight across a barrier that follows.
template <int FMT, int J>
__device__ __forceinline__ void row_prepare(RowOut<J>& o, const float (&g)[J], const float* gamma, float eps, int c,
                                            int d_nope, int d_rope, bool rope, double inv, double pos, float* ys,
                                            uint16_t* dec) {
    const int lane = threadIdx.x & 63;
    if (gamma) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) ss = fmaf(o.y[j], o.y[j], ss);
        const float r = 1.0f / sqrtf(wave_sum_dpp(ss) / (float)c + eps);
#pragma unroll
        for (int j = 0; j < J; ++j) o.y[j] = g[j] * o.y[j] * r;
    }
    if (rope) {
        // lane l < d_rope rotates channel d_nope + l with its partner d_nope + (l +- d_rope / 2)
        const int half = d_rope >> 1;
#pragma unroll
        for (int j = 0; j < J; ++j) ys[lane + 64 * j] = o.y[j];
        __builtin_amdgcn_wave_barrier();
        float rot = 0.0f;
        if (lane < d_rope) {
            float sn, cs;
            rope_sincos(&inv, 0, pos, &sn, &cs);
            const float x = ys[d_nope + lane];
            rot = lane < half ? x * cs - ys[d_nope + lane + half] * sn : ys[d_nope + lane - half] * sn + x * cs;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < d_rope) ys[d_nope + lane] = rot;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (lane + 64 * j >= d_nope) o.y[j] = ys[lane + 64 * j];
    }
    if (FMT == LCA_FP8) {
        // power-of-two scale per 128 nope dims (d_nope % 128 == 0): channels 128 g .. are j = 2g, 2g+1
#pragma unroll
        for (int g2 = 0; 2 * g2 < J; ++g2) {
            float am = 0.0f;
            if (128 * g2 < d_nope) {
                am = fabsf(o.y[2 * g2]);
                if (2 * g2 + 1 < J) am = fmaxf(am, fabsf(o.y[2 * g2 + 1]));
            }
            const float amax = wave_max_dpp(am);
            int e8 = 0;  // scale = 2^e8: the smallest with amax <= 448 2^e8
            if (amax > 0.0f) {
                int ex = 0;
                frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
                const int e = ex - 1;
                e8 = (amax <= ldexpf(1.75f, e)) ? e - 8 : e - 7;
            }
            o.isc[g2] = ldexpf(1.0f, -e8);
            o.scl[g2] = ldexpf(1.0f, e8);
        }
    }
    if (dec) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            if (FMT == LCA_FP8 && ch < d_nope) dec[ch] = f2bf(fp8_to_f32(f32_to_fp8(o.y[j] * o.isc[j >> 1])) * o.scl[j >> 1]);
            else if (ch < c) dec[ch] = f2bf(o.y[j]);
        }
    }
}

// The store of a prepared row into row `row` of the planes (one whole wave).
template <int FMT, int J>
__device__ __forceinline__ void row_commit(const RowOut<J>& o, int c, int d_nope, int d_rope, void* onope,
                                           void* orope, void* oscale, int64_t row) {
    const int lane = threadIdx.x & 63;
    if (FMT == LCA_FP8) {
#pragma unroll
        for (int g2 = 0; 2 * g2 < J; ++g2)
            if (lane == 0 && 128 * g2 < d_nope) ((float*)oscale)[row * (d_nope >> 7) + g2] = o.scl[g2];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            if (ch < d_nope)
                ((uint8_t*)onope)[row * d_nope + ch] = (uint8_t)f32_to_fp8(o.y[j] * o.isc[j >> 1]);
            else if (ch < c)
                ((uint16_t*)orope)[row * d_rope + (ch - d_nope)] = f2bf(o.y[j]);
        }
    } else if (FMT == LCA_MXFP4) {  // d_rope == 0, c % 32 == 0
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            mxfp4_store_lane(o.y[j], ch < c, (uint8_t*)oscale + row * (c >> 5), ch >> 5,
                             (uint32_t*)onope + row * (c >> 3), ch >> 3);
        }
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            if (FMT == LCA_BF16) {
                if (ch < d_nope) ((uint16_t*)onope)[row * d_nope + ch] = f2bf(o.y[j]);
                else if (ch < c) ((uint16_t*)orope)[row * d_rope + (ch - d_nope)] = f2bf(o.y[j]);
            } else {
                if (ch < d_nope) ((float*)onope)[row * d_nope + ch] = o.y[j];
                else if (ch < c) ((float*)orope)[row * d_rope + (ch - d_nope)] = o.y[j];
            }
        }
    }
}

}  // namespace lca
