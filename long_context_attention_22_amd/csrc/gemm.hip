// gemm.hip -- the linear maps around the attention ("DeepSeek-V4 中文翻译" section 2.3.1: the
// compressor inputs, the queries and the grouped output projection are projections of per-token
// vectors): Y[b][m][n] = sum_k X[b][m][k] W[b][n][k], X and W bf16 with K contiguous (W holds one
// output per row, as a weight matrix), f32 accumulation, Y f32 or bf16.
//
// Many rows: MFMA tiles.  A 256-thread workgroup computes a 128 x 128 tile of Y, each wave a
// 64 x 64 quarter as 4 x 4 blocks of v_mfma_f32_16x16x32_bf16 (both operands K-contiguous: lane l
// reads 8 consecutive k of row l mod 16 with one ds_read_b128).  K advances 64 at a time through
// two LDS buffers whose rows are padded to 72 elements (144 bytes: the sixteen rows one block read
// touches start 36 banks apart, so they fall in distinct banks); the next slice's global loads are
// issued before the current slice's MFMAs, one barrier per slice.
// Few rows (decode, M <= 4): the map is bound by reading W once.  Each wave produces 4 outputs for
// every row of X: lane l reads 16 bytes of each of its 4 weight rows per 512-element step, four
// steps in flight, and the 64 partial sums of an output meet in one wave reduction.
#include "device.h"
#include "kernels.h"

namespace lca {

constexpr int kGT = 128, kGK = 64, kGS = 72;  // tile rows / columns, K slice, LDS row stride
constexpr int kGemvRows = 4;                  // M at most this: the streaming kernel

template <typename TY>
__device__ __forceinline__ void put_y(TY* p, float v);
template <>
__device__ __forceinline__ void put_y<float>(float* p, float v) {
    *p = v;
}
template <>
__device__ __forceinline__ void put_y<uint16_t>(uint16_t* p, float v) {
    *p = f2bf(v);
}

template <typename TY>
__global__ void __launch_bounds__(256) gemm_mfma(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kGT * kGS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kGT * kGS];
    const int b = blockIdx.z;
    const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;
    const int M = a.M, N = a.N, K = a.K;
    const uint16_t* X = (const uint16_t*)a.x + (int64_t)b * a.sx;
    const uint16_t* W = (const uint16_t*)a.w + (int64_t)b * a.sw;

    // This thread's four 16-byte chunks of each operand's slice: chunk q = tid + 256 i is row q / 8,
    // elements 8 (q mod 8) .. of the slice.  Rows past M / N re-read the last row (their results are
    // not stored); chunks past K (K is a multiple of 8) read the last chunk and are zeroed.
    const uint16_t* xp[4];
    const uint16_t* wp[4];
    int kk[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i, r = q >> 3;
        kk[i] = 8 * (q & 7);
        lo[i] = r * kGS + kk[i];
        xp[i] = X + (int64_t)min(m0 + r, M - 1) * a.ldx;
        wp[i] = W + (int64_t)min(n0 + r, N - 1) * a.ldw;
    }
    u32x4 rx[4], rw[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + kk[i];
            const int kc = min(k, K - 8);
            const u32x4 vx = *(const u32x4*)(xp[i] + kc), vw = *(const u32x4*)(wp[i] + kc);
            rx[i] = k < K ? vx : u32x4{0u, 0u, 0u, 0u};
            rw[i] = k < K ? vw : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)&As[buf][lo[i]] = rx[i];
            *(u32x4*)&Bs[buf][lo[i]] = rw[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = (K + kGK - 1) / kGK;
    load(0);
    store(0);
    __syncthreads();
    const int fr = (lane & 15) * kGS + 8 * (lane >> 4);  // this lane's fragment offset in a block
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * kGK);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 af[4], bw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)&As[buf][(wm + 16 * i) * kGS + fr + 32 * s];
#pragma unroll
            for (int j = 0; j < 4; ++j) bw[j] = *(const bf16x8*)&Bs[buf][(wn + 16 * j) * kGS + fr + 32 * s];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }

    // lane holds rows 4 (lane / 16) + r of each block, column lane mod 16
    TY* Y = (TY*)a.y + (int64_t)b * a.sy;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                if (m < M && n < N) put_y<TY>(Y + (int64_t)m * a.ldy + n, acc[i][j][r]);
            }
        }
}

template <int MR, typename TY>
__global__ void __launch_bounds__(256) gemv_stream(GemmArgs a) {
    const int b = blockIdx.z, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int M = a.M, N = a.N, K = a.K;
    const int n0 = blockIdx.x * 16 + 4 * wv;  // this wave's 4 outputs (rows of W)
    const uint16_t* X = (const uint16_t*)a.x + (int64_t)b * a.sx;
    const uint16_t* W = (const uint16_t*)a.w + (int64_t)b * a.sw;
    const uint16_t* wr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[r] = W + (int64_t)min(n0 + r, N - 1) * a.ldw;
    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][r] = 0.0f;
    // four 512-element steps per round, loads first (branch-free: chunks past K read the last chunk
    // and count zero)
    for (int kb = 0; kb < K; kb += 2048) {
        u32x4 wv_[4][4], xv[4][MR];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = kb + 512 * u + 8 * lane;
            ok[u] = k < K;
            const int kc = min(k, K - 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv_[u][r] = *(const u32x4*)(wr[r] + kc);
#pragma unroll
            for (int m = 0; m < MR; ++m) xv[u][m] = *(const u32x4*)(X + (int64_t)min(m, M - 1) * a.ldx + kc);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (!ok[u]) continue;
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float xf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xf[2 * e] = __uint_as_float(xv[u][m][e] << 16);
                    xf[2 * e + 1] = __uint_as_float(xv[u][m][e] & 0xffff0000u);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[m][r] = fmaf(xf[2 * e], __uint_as_float(wv_[u][r][e] << 16), acc[m][r]);
                        acc[m][r] = fmaf(xf[2 * e + 1], __uint_as_float(wv_[u][r][e] & 0xffff0000u), acc[m][r]);
                    }
            }
        }
    }
    TY* Y = (TY*)a.y + (int64_t)b * a.sy;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = wave_sum_dpp(acc[m][r]);
            if (lane == 0 && m < M && n0 + r < N) put_y<TY>(Y + (int64_t)m * a.ldy + n0 + r, s);
        }
}

template <typename TY>
static void launch_gemm_t(const GemmArgs& a, hipStream_t st) {
    if (a.M <= kGemvRows) {
        dim3 grid((unsigned)((a.N + 15) / 16), 1, (unsigned)a.batch);
        if (a.M == 1) hipLaunchKernelGGL((gemv_stream<1, TY>), grid, dim3(256), 0, st, a);
        else if (a.M == 2) hipLaunchKernelGGL((gemv_stream<2, TY>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((gemv_stream<4, TY>), grid, dim3(256), 0, st, a);
        return;
    }
    dim3 grid((unsigned)((a.N + kGT - 1) / kGT), (unsigned)((a.M + kGT - 1) / kGT), (unsigned)a.batch);
    hipLaunchKernelGGL((gemm_mfma<TY>), grid, dim3(256), 0, st, a);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
    if (a.y_dtype == LCA_F32) launch_gemm_t<float>(a, st);
    else launch_gemm_t<uint16_t>(a, st);
    return hipGetLastError();
}

}  // namespace lca
