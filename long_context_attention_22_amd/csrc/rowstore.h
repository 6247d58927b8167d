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

// RMSNorm (gamma != NULL), RoPE at position pos (rope; inv = this lane's pair frequency
// theta^(-2i/d_rope), i = lane mod d_rope/2; d_rope <= 64) through the LDS scratch ys[64 J] of
// this wave, then the store into row `row` of the planes (store != 0).  dec != NULL: the stored
// values, decoded (an fp8 code times its scale, exact in bf16), also go to dec[ch] as bf16.
// Called by one whole wave; it synchronises only that wave (LDS accesses of one wave are ordered).
template <int FMT, int J>
__device__ __forceinline__ void row_store(float (&y)[J], const float (&g)[J], const float* gamma, float eps, int c,
                                          int d_nope, int d_rope, bool rope, double inv, double pos, void* onope,
                                          void* orope, void* oscale, int64_t row, float* ys, uint16_t* dec,
                                          bool store) {
    const int lane = threadIdx.x & 63;
    if (gamma) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) ss = fmaf(y[j], y[j], ss);
        const float r = 1.0f / sqrtf(wave_sum_dpp(ss) / (float)c + eps);
#pragma unroll
        for (int j = 0; j < J; ++j) y[j] = g[j] * y[j] * r;
    }
    if (rope) {
        // lane l < d_rope rotates channel d_nope + l with its partner d_nope + (l +- d_rope / 2)
        const int half = d_rope >> 1;
#pragma unroll
        for (int j = 0; j < J; ++j) ys[lane + 64 * j] = y[j];
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
            if (lane + 64 * j >= d_nope) y[j] = ys[lane + 64 * j];
    }
    if (FMT == LCA_FP8) {
        // power-of-two scale per 128 nope dims (d_nope % 128 == 0): channels 128 g .. are j = 2g, 2g+1
        float isc[J / 2 + 1], scl[J / 2 + 1];  // 1 / scale and scale, exact
#pragma unroll
        for (int g2 = 0; 2 * g2 < J; ++g2) {
            float am = 0.0f;
            if (128 * g2 < d_nope) {
                am = fabsf(y[2 * g2]);
                if (2 * g2 + 1 < J) am = fmaxf(am, fabsf(y[2 * g2 + 1]));
            }
            const float amax = wave_max_dpp(am);
            int e8 = 0;  // scale = 2^e8: the smallest with amax <= 448 2^e8
            if (amax > 0.0f) {
                int ex = 0;
                frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
                const int e = ex - 1;
                e8 = (amax <= ldexpf(1.75f, e)) ? e - 8 : e - 7;
            }
            isc[g2] = ldexpf(1.0f, -e8);
            scl[g2] = ldexpf(1.0f, e8);
            if (store && lane == 0 && 128 * g2 < d_nope) ((float*)oscale)[row * (d_nope >> 7) + g2] = scl[g2];
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            if (ch < d_nope) {
                const uint32_t code = f32_to_fp8(y[j] * isc[j >> 1]);
                if (store) ((uint8_t*)onope)[row * d_nope + ch] = (uint8_t)code;
                if (dec) dec[ch] = f2bf(fp8_to_f32(code) * scl[j >> 1]);
            } else if (ch < c) {
                const uint16_t h = f2bf(y[j]);
                if (store) ((uint16_t*)orope)[row * d_rope + (ch - d_nope)] = h;
                if (dec) dec[ch] = h;
            }
        }
    } else if (FMT == LCA_MXFP4) {  // d_rope == 0, c % 32 == 0
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            mxfp4_store_lane(y[j], store && ch < c, (uint8_t*)oscale + row * (c >> 5), ch >> 5,
                             (uint32_t*)onope + row * (c >> 3), ch >> 3);
        }
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ch = lane + 64 * j;
            if (FMT == LCA_BF16) {
                const uint16_t h = f2bf(y[j]);
                if (store && ch < d_nope) ((uint16_t*)onope)[row * d_nope + ch] = h;
                else if (store && ch < c) ((uint16_t*)orope)[row * d_rope + (ch - d_nope)] = h;
                if (dec && ch < c) dec[ch] = h;
            } else {
                if (store && ch < d_nope) ((float*)onope)[row * d_nope + ch] = y[j];
                else if (store && ch < c) ((float*)orope)[row * d_rope + (ch - d_nope)] = y[j];
            }
        }
    }
}

}  // namespace lca
