// gemm.hip -- the linear maps around the attention ("DeepSeek-V4 中文翻译" section 2.3.1: the
// compressor inputs, the queries and the grouped output projection are projections of per-token
// vectors): Y[b][m][n] = sum_k X[b][m][k] W[b][n][k], X and W bf16 with K contiguous (W holds one
// output per row, as a weight matrix), f32 accumulation, Y f32 or bf16.
//
// Many rows: MFMA tiles (gemm_big's 256 x 256 tiles for maps that have enough of them, below).  A
// 256-thread workgroup computes a 128 x 128 tile of Y, each wave a
// 64 x 64 quarter as 4 x 4 blocks of v_mfma_f32_16x16x32_bf16 (both operands K-contiguous: lane l
// reads 8 consecutive k of row l mod 16 with one ds_read_b128).  K advances 64 at a time through
// two LDS buffers whose rows are padded to 80 elements (160 bytes; measured against 64, 72, 88 and
// 96: the fewest bank conflicts); the global loads run two slices ahead (two register sets), one
// barrier per slice.
// Few rows (decode, M <= 4): the map is bound by reading W once.  Lane l reads 16 bytes of each of a
// wave's 4 weight rows per 512-element step of K, four steps in flight, and an output's 64 lane sums
// meet in a wave reduction.  With few outputs the four waves of a workgroup split K over the same 4
// outputs (their sums meet in LDS, added in a fixed order); with many, each wave has 4 of its own.
#include "device.h"
#include "kernels.h"
#include "trace.h"

namespace lca {

constexpr int kGT = 128, kGK = 64, kGS = 80;  // tile rows / columns, K slice, LDS row stride
constexpr int kGemvRows = 4;                  // M at most this: the streaming kernel
constexpr int64_t kGemmBigTiles = 256;        // 256 x 256 tiles from which a map takes gemm_big

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
    // (32-bit element offsets from the operands' bases: loads then take the scalar-base form)
    uint32_t xo[4], wo[4];
    int kk[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i, r = q >> 3;
        kk[i] = 8 * (q & 7);
        lo[i] = r * kGS + kk[i];
        xo[i] = (uint32_t)((int64_t)min(m0 + r, M - 1) * a.ldx);
        wo[i] = (uint32_t)((int64_t)min(n0 + r, N - 1) * a.ldw);
    }
    // two register sets: the slice after next is loaded while the next one waits for its LDS buffer
    u32x4 rx[2][4], rw[2][4];
    // (chunks past K are zeroed when stored, not when loaded: a use right after the load would make
    // the wave wait for it)
    auto load = [&](int st, int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t kc = (uint32_t)min(k0 + kk[i], K - 8);
            rx[st][i] = *(const u32x4*)(X + (xo[i] + kc));
            rw[st][i] = *(const u32x4*)(W + (wo[i] + kc));
        }
    };
    auto store = [&](int st, int buf, int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = k0 + kk[i] < K;
            *(u32x4*)&As[buf][lo[i]] = ok ? rx[st][i] : u32x4{0u, 0u, 0u, 0u};
            *(u32x4*)&Bs[buf][lo[i]] = ok ? rw[st][i] : u32x4{0u, 0u, 0u, 0u};
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int fr = (lane & 15) * kGS + 8 * (lane >> 4);  // this lane's fragment offset in a block
    auto compute = [&](int buf) {
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
    };
    // slice kt is in LDS buffer kt mod 2, slice kt + 1 in register set (kt + 1) mod 2
    // (no branches in the loop body: slices past the end are loaded again from the last slice and
    // stored into the free buffer, so the compiler counts the loads in flight exactly)
    const int nk = (K + kGK - 1) / kGK, klast = (nk - 1) * kGK;
    // (compiler barriers keep the phases in this order: the stores of the next slice must not move
    // up, where they would wait for its loads)
    auto step = [&](int kt, int cur, int nxt) {
        load(cur, min((kt + 2) * kGK, klast));
        asm volatile("" ::: "memory");
        compute(cur);
        asm volatile("" ::: "memory");
        store(nxt, nxt, (kt + 1) * kGK);
        __syncthreads();
    };
    load(0, 0);
    store(0, 0, 0);
    load(1, min(kGK, klast));
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        step(kt, 0, 1);
        step(kt + 1, 1, 0);
    }
    if (kt < nk) compute(0);  // an odd slice count: the last slice is in buffer 0

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

// Large maps (enough 256 x 256 tiles to fill the GPU): a 512-thread workgroup computes a 256 x 256 tile
// of Y, each of its eight waves a 64 x 128 part as 4 x 8 blocks of v_mfma_f32_16x16x32_bf16 (128
// accumulator registers, two waves per SIMD).  Per byte brought in from L2 the tile does twice the
// work of gemm_mfma's 128 x 128 one, whose operand traffic (64 flop per byte) bounds it on this GPU.
// 64-deep K slices in two LDS buffers (rows padded to 72 elements); the next slice's global loads go
// out before a slice's products (one register set: a second, for loads two slices ahead, spills), one
// barrier per slice.  (A four-wave form with 128 x 128 per wave needs all 256 AGPRs for its
// accumulators, and the register allocator then moved them through VGPRs on every MFMA.)
constexpr int kBT = 256, kBS = 72;  // tile rows / columns, LDS row stride
template <typename TY>
__global__ void __launch_bounds__(512) gemm_big(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBT * kBS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBT * kBS];
    const int b = blockIdx.z;
    const int m0 = blockIdx.y * kBT, n0 = blockIdx.x * kBT;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = (wv >> 1) * 64, wn = (wv & 1) * 128;
    const int M = a.M, N = a.N, K = a.K;
    const uint16_t* X = (const uint16_t*)a.x + (int64_t)b * a.sx;
    const uint16_t* W = (const uint16_t*)a.w + (int64_t)b * a.sw;

    // chunk q = tid + 512 i (i < 4) of a slice: row tid / 8 + 64 i, elements kk = 8 (tid mod 8) ..; rows past
    // M / N re-read the last row (not stored), chunks past K read the last chunk and are zeroed when stored
    const int r0 = tid >> 3, kk = 8 * (tid & 7);
    const int lo0 = r0 * kBS + kk;
    uint32_t xo[4], wo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xo[i] = (uint32_t)((int64_t)min(m0 + r0 + 64 * i, M - 1) * a.ldx);
        wo[i] = (uint32_t)((int64_t)min(n0 + r0 + 64 * i, N - 1) * a.ldw);
    }
    u32x4 rx[4], rw[4];
    auto load = [&](int k0) {
        const uint32_t kc = (uint32_t)min(k0 + kk, K - 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rx[i] = *(const u32x4*)(X + (xo[i] + kc));
            rw[i] = *(const u32x4*)(W + (wo[i] + kc));
        }
    };
    auto store = [&](int buf, int k0) {
        const bool ok = k0 + kk < K;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)&As[buf][lo0 + 64 * kBS * i] = ok ? rx[i] : u32x4{0u, 0u, 0u, 0u};
            *(u32x4*)&Bs[buf][lo0 + 64 * kBS * i] = ok ? rw[i] : u32x4{0u, 0u, 0u, 0u};
        }
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int fr = (lane & 15) * kBS + 8 * (lane >> 4);  // this lane's fragment offset in a block
    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 af[4], bw[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)&As[buf][(wm + 16 * i) * kBS + fr + 32 * s];
#pragma unroll
            for (int j = 0; j < 8; ++j) bw[j] = *(const bf16x8*)&Bs[buf][(wn + 16 * j) * kBS + fr + 32 * s];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
        }
    };
    // slice kt is in LDS buffer kt mod 2; past the last slice the loads re-read it (branch-free) and the
    // store goes to the free buffer
    const int nk = (K + kGK - 1) / kGK, klast = (nk - 1) * kGK;
    load(0);
    store(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        load(min((kt + 1) * kGK, klast));
        asm volatile("" ::: "memory");
        compute(cur);
        asm volatile("" ::: "memory");
        store(cur ^ 1, (kt + 1) * kGK);
        __syncthreads();
    }

    TY* Y = (TY*)a.y + (int64_t)b * a.sy;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                if (m < M && n < N) put_y<TY>(Y + (int64_t)m * a.ldy + n, acc[i][j][r]);
            }
        }
}

// KS: the four waves split K over the workgroup's 4 outputs (few outputs: more workgroups); else
// each wave takes 4 outputs of its own over all of K (16 per workgroup).
template <int MR, typename TY, bool KS>
__global__ void __launch_bounds__(256) gemv_stream(GemmArgs a) {
    __shared__ float red[4][MR][4];
    const int b = blockIdx.z, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int M = a.M, N = a.N, K = a.K;
    // KS: wave wv takes every fourth 512-element step of K, k = 2048 i + 512 wv + 8 lane
    const int n0 = KS ? blockIdx.x * 4 : blockIdx.x * 16 + 4 * wv;
    const int kstep = KS ? 2048 : 512, kfirst = KS ? 512 * wv : 0;
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
    // four steps of this wave per round, loads first (branch-free: chunks past K read the last chunk
    // and count zero)
    for (int kb = kfirst; kb < K; kb += 4 * kstep) {
        u32x4 wv_[4][4], xv[4][MR];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = kb + kstep * u + 8 * lane;
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
    if constexpr (!KS) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float s = wave_sum_dpp(acc[m][r]);
                if (lane == 0 && m < M && n0 + r < N) put_y<TY>(Y + (int64_t)m * a.ldy + n0 + r, s);
            }
        return;
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = wave_sum_dpp(acc[m][r]);
            if (lane == 0) red[wv][m][r] = s;
        }
    __syncthreads();
    // the four waves' partial sums in a fixed order
    const int t = threadIdx.x;
    if (t < MR * 4) {
        const int m = t >> 2, r = t & 3;
        const float s = (red[0][m][r] + red[1][m][r]) + (red[2][m][r] + red[3][m][r]);
        if (m < M && n0 + r < N) put_y<TY>(Y + (int64_t)m * a.ldy + n0 + r, s);
    }
}

template <typename TY>
static void launch_gemm_t(const GemmArgs& a, hipStream_t st) {
    if (a.M <= kGemvRows) {
        // outputs per workgroup: 4 (K split over the waves) while that leaves fewer than ~2048
        // workgroups, else 16
        const bool ks = (int64_t)a.N * a.batch < 8192;
        dim3 grid((unsigned)(ks ? (a.N + 3) / 4 : (a.N + 15) / 16), 1, (unsigned)a.batch);
        if (trace_on()) trace("  gemv_stream<%d>: grid (%u, 1, %u) x 256%s", a.M, grid.x, grid.z, ks ? ", K split over waves" : "");
        if (ks) {
            if (a.M == 1) hipLaunchKernelGGL((gemv_stream<1, TY, true>), grid, dim3(256), 0, st, a);
            else if (a.M == 2) hipLaunchKernelGGL((gemv_stream<2, TY, true>), grid, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((gemv_stream<4, TY, true>), grid, dim3(256), 0, st, a);
        } else {
            if (a.M == 1) hipLaunchKernelGGL((gemv_stream<1, TY, false>), grid, dim3(256), 0, st, a);
            else if (a.M == 2) hipLaunchKernelGGL((gemv_stream<2, TY, false>), grid, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((gemv_stream<4, TY, false>), grid, dim3(256), 0, st, a);
        }
        return;
    }
    const int64_t big = (int64_t)((a.N + kBT - 1) / kBT) * ((a.M + kBT - 1) / kBT) * a.batch;
    if (big >= kGemmBigTiles) {  // enough 256 x 256 tiles to fill the GPU
        dim3 grid((unsigned)((a.N + kBT - 1) / kBT), (unsigned)((a.M + kBT - 1) / kBT), (unsigned)a.batch);
        if (trace_on()) trace("  gemm_big: grid (%u, %u, %u) x 512, 256 x 256 tiles", grid.x, grid.y, grid.z);
        hipLaunchKernelGGL((gemm_big<TY>), grid, dim3(512), 0, st, a);
        return;
    }
    dim3 grid((unsigned)((a.N + kGT - 1) / kGT), (unsigned)((a.M + kGT - 1) / kGT), (unsigned)a.batch);
    if (trace_on()) trace("  gemm_mfma: grid (%u, %u, %u) x 256, 128 x 128 tiles", grid.x, grid.y, grid.z);
    hipLaunchKernelGGL((gemm_mfma<TY>), grid, dim3(256), 0, st, a);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
    if (a.y_dtype == LCA_F32) launch_gemm_t<float>(a, st);
    else launch_gemm_t<uint16_t>(a, st);
    return hipGetLastError();
}

}  // namespace lca
