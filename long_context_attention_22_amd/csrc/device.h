// device.h -- gfx950 device helpers shared by the library's kernels:
// bf16 / OCP-e4m3fn / MXFP4 conversions, wave reductions, MFMA fragment types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// nearest-even fp32 -> bf16 (inputs are finite)
__device__ __forceinline__ uint16_t f2bf(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP e4m3fn -> fp32.  Normal codes: (1 + m/8) 2^(e-7); exponent 0: m 2^-9.
__device__ __forceinline__ float fp8_to_f32(uint32_t code) {
    uint32_t s = (code & 0x80u) << 24, e = (code >> 3) & 15u, mt = code & 7u;
    float sub = (float)mt * 0.001953125f;
    float nrm = __uint_as_float(((e + 120u) << 23) | (mt << 20));
    return __uint_as_float(__float_as_uint(e ? nrm : sub) | s);
}

// fp32 -> OCP e4m3fn, nearest with ties to the even code, saturating at 448.
// With e = max(floor(log2|x|), -6) the code is 8(e+6) + rint(|x| 2^(3-e)) for
// e > -6 and rint(|x| 2^9) below: code order follows value order, so a
// mantissa carry simply moves to the next binade.
__device__ __forceinline__ uint32_t f32_to_fp8(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t s = (u >> 24) & 0x80u;
    float a = __uint_as_float(u & 0x7fffffffu);
    int e = (int)((u >> 23) & 0xffu) - 127;
    uint32_t code;
    if (e <= -6) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        float q = __builtin_rintf(__uint_as_float(__float_as_uint(a) - ((uint32_t)(e - 3) << 23)));
        code = (uint32_t)(8 * (e + 6)) + (uint32_t)q;
    }
    code = code > 126u ? 126u : code;
    return code | s;
}

// OCP MXFP4 (Microscaling Formats v1.0): blocks of 32 elements share an E8M0 scale 2^e and each
// element is an FP4 E2M1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit; values
// 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The block exponent puts the largest magnitude in [4, 8):
// e = floor(log2 amax) - 2, clamped to the E8M0 range [-127, 127]; an all-zero block gets e = 0.
__device__ __forceinline__ int mx_block_exp(float amax) {
    if (!(amax > 0.0f)) return 0;
    int ex = 0;
    frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
    const int e = ex - 3;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// E2M1 code of x (already divided by the block scale): the nearest value, an exact tie going to
// the even code, magnitudes beyond 6 saturating; the sign bit is copied from x.  Each term adds
// one code step at the midpoint between neighbouring values (strict where the upper neighbour
// has an odd code, inclusive where it is even).
__device__ __forceinline__ uint32_t e2m1_code(float x) {
    const float a = fabsf(x);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(x) >> 28) & 8u);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// reduction over the 16 lanes that share l / 16 (one MFMA column group)
__device__ __forceinline__ float max16(float v) {
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// RoPE rotation for pair i at position pos: inv[i] = theta^(-2i/d_rope) is computed on the
// host in fp64; the angle pos * inv[i] is formed and reduced by the nearest multiple k of pi/2 in
// fp64 (positions reach 2^20 and beyond), and sin / cos of the remainder |x| <= pi/4 come from
// their Taylor series in fp32 (terms to x^9 / x^10: truncation below 2e-10, far under one f32
// ulp), placed in the quadrant k mod 4.  A few dozen instructions instead of a library sincos,
// whose general argument reduction would be dead code here.
__device__ __forceinline__ void rope_sincos(const double* inv, int i, double pos, float* sn, float* cs) {
    const double ang = pos * inv[i];
    const double k = rint(ang * 0.63661977236758134308);  // 2 / pi
    const float x = (float)(ang - k * 1.57079632679489661923);
    const float x2 = x * x;
    const float sp = x * fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f), 1.0f / 120.0f),
                                       -1.0f / 6.0f), 1.0f);
    const float cp = fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f), -1.0f / 720.0f),
                                        1.0f / 24.0f), -0.5f), 1.0f);
    const int q = (int)((int64_t)k & 3);
    const float s0 = (q & 1) ? cp : sp, c0 = (q & 1) ? sp : cp;
    *sn = (q & 2) ? -s0 : s0;
    *cs = ((q + 1) & 2) ? -c0 : c0;
}

// 16-lane (one MFMA column group) reductions with DPP row rotations: every lane of the
// row ends with the result, no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0x128>(v));  // row_ror:8
    v = fmaxf(v, dpp<0x124>(v));  // row_ror:4
    v = fmaxf(v, dpp<0x4e>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0xb1>(v));   // quad_perm [1,0,3,2]
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0x128>(v);
    v += dpp<0x124>(v);
    v += dpp<0x4e>(v);
    v += dpp<0xb1>(v);
    return v;
}

// Cross-row exchanges of gfx950 (v_permlane16_swap / v_permlane32_swap), no LDS traffic.
__device__ __forceinline__ float xlane32(float v, bool mx) {  // combine with lane ^ 32
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
    return mx ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xlane16(float v, bool mx) {  // combine with lane ^ 16
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
    return mx ? fmaxf(a, b) : a + b;
}
// Reduce-scatter over the four 16-lane rows: lane l ends with the sum over the rows of v[l >> 4]
// at its column l & 15 (each v[b] holds one partial per lane).  Two permlane16 swaps pair rows
// (0, 1) and (2, 3) of two values at a time, one permlane32 swap pairs the halves.
__device__ __forceinline__ float sum4g_scatter(float v0, float v1, float v2, float v3) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
    const float s01 = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // rows: v0 (0+1), v1 (0+1), v0 (2+3), v1 (2+3)
    const float s23 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// over the four 16-lane groups: every lane gets the same value, summed in the same order
__device__ __forceinline__ float max4g(float v) { return xlane32(xlane16(v, true), true); }
__device__ __forceinline__ float sum4g(float v) { return xlane32(xlane16(v, false), false); }
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS traffic): shifts by 1, 2,
// 4 and 8 lanes scan each 16-lane row, then gfx9's row broadcasts carry lane 15 of rows 0 and 2 into
// rows 1 and 3 and lane 31 into rows 2 and 3.  Lanes whose source lies outside the row, or whose row
// the row mask leaves out, add the old value 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}
__device__ __forceinline__ uint32_t wave_lane63(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// bitwise OR over the eight lanes of each aligned group of 8 (quad swaps, then the half-row mirror)
__device__ __forceinline__ uint32_t or8(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);  // row_half_mirror
    return v;
}
// One MXFP4 block per 32 lanes (lanes 0-31 and 32-63 of the wave hold elements 0..31 of two
// blocks, one value each; lanes past the row hold 0).  Every lane of the wave must call this.
// Lane 0 / 32 stores the block's E8M0 byte at scales[blk]; lanes 8i store the 32-bit word of
// codes of elements 8i..8i+7 (element 8i + n in bits 4n) at codes[word].
__device__ __forceinline__ void mxfp4_store_lane(float y, bool live, uint8_t* scales, int64_t blk, uint32_t* codes,
                                                 int64_t word) {
    const int lane = threadIdx.x & 63;
    const float amax = xlane16(row_max16(fabsf(y)), true);  // over this lane's 32-lane half
    const int e = mx_block_exp(amax);
    const uint32_t w = or8(e2m1_code(ldexpf(y, -e)) << (4 * (lane & 7)));
    if (live && (lane & 7) == 0) codes[word] = w;
    if (live && (lane & 31) == 0) scales[blk] = (uint8_t)(e + 127);
}

// whole-wave reductions without LDS: DPP within each 16-lane row, then the row swaps
__device__ __forceinline__ float wave_max_dpp(float v) { return max4g(row_max16(v)); }
__device__ __forceinline__ float wave_sum_dpp(float v) { return sum4g(row_sum16(v)); }

}  // namespace lca
