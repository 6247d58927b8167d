// kernels.h -- launch entry points of the HIP kernels (host side), called by
// the C ABI in capi.cpp after it has validated every argument.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lca.h"

namespace lca {

struct Pos {
    int64_t v[LCA_MAX_BATCH];
};

// theta^(-2i/d_rope) for i < d_rope / 2, computed on the host in fp64
constexpr int kMaxRopeHalf = 64;
struct RopeTab {
    double inv[kMaxRopeHalf];
};

// kv_compress: entries [s_lo[b], s_hi[b]) of each sequence.
struct CompressArgs {
    const void* c_a;
    const void* z_a;
    const void* c_b;
    const void* z_b;
    const float* bias_a;
    const float* bias_b;
    const float* gamma;
    float eps;
    double rope_theta;
    RopeTab rope;
    int32_t in_dtype;
    int32_t m, overlap, B;
    int64_t n_rows, in_stride;
    lca_kv out;
    int32_t ring;
    Pos first_pos;
    Pos s_lo;
    int64_t max_entries;
    // bf16 rows of few entries split over workgroups (parts > 1): ws holds the parts' channel states
    float* ws;
    int32_t parts, part_len;
};
hipError_t launch_kv_compress(const CompressArgs& a, hipStream_t st);
// Entry parts of a split compression: (entries x sequences) units share kCompressUnits workgroups, at most
// kCompressMaxParts per entry, each part at least kCompressMinRows rows of the entry's list.
constexpr int kCompressUnits = 256, kCompressMaxParts = 16, kCompressMinRows = 8, kCompressMinList = 64;

struct IndexerArgs {
    const void* q;
    const float* w;
    const void* k;
    const void* k_scale;  // E8M0 bytes of MXFP4 keys (in_dtype == LCA_MXFP4: bf16 q, MXFP4 keys)
    int32_t in_dtype;
    int64_t k_cap;
    int32_t H_I, d_I, B, T, m;
    void* scores;
    int32_t score_dtype;
    int64_t s_stride;
    Pos q_pos;
    int64_t max_vis;
    // Fused first pass of the top-k (bf16 scores): the high-byte histograms of each query row's visible
    // scores, added with device atomics into th_h1 (row r = b T + i at th_h1 + r * th_row; zero on
    // entry) -- per kTopkChunk-key chunk when th_chunked (the top-k's split schedule: chunk g at
    // + kTopkHistWords g in 16-bit counts, th_row = kTopkHistWords G), else one per row in 32-bit
    // counts (its row schedule, th_row = 256).  NULL = off.
    uint32_t* th_h1;
    int64_t th_row;
    int32_t th_chunked;
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st);

// Keys per chunk of the top-k's split schedule (one workgroup each, a power of two).
constexpr int kTopkChunkLog2 = 12;
constexpr int kTopkChunk = 1 << kTopkChunkLog2;
// A chunk's 256-bin histogram holds 16-bit counts (at most kTopkChunk per bin), two bins per word:
// bin 2j in the low half of word j, bin 2j + 1 in the high half.
constexpr int kTopkHistWords = 128;

struct TopkArgs {
    const void* scores;
    int32_t score_dtype;
    int64_t s_stride;
    int32_t B, T, m, k;
    int32_t* idx;
    void* ws;
    int64_t max_n;   // largest candidate count over the rows
    Pos q_pos;
    // The split schedule's high-byte histograms were made by the indexer (IndexerArgs::th_h1, at the
    // workspace's start): only the last two launches run, and the last one clears those histograms
    // for the next call.
    int32_t split_fused;
    // The row schedule's first pass was made by the indexer: row r's high-byte histogram at
    // row_h1 + 256 r (zero on entry); the row's workgroup reads it instead of the pass and zeroes it.
    uint32_t* row_h1;
};
size_t topk_ws_bytes(int32_t B, int32_t T, int64_t s_stride, int32_t score_dtype);
// chunks per row of the split schedule for these rows, 0 when the rows take the row schedule
int topk_split_chunks(int32_t rows, int64_t max_n, int64_t s_stride, int32_t score_dtype);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

struct AttnArgs {
    const void* q;
    int32_t q_dtype;
    int32_t H, B, T, m;
    lca_kv comp;
    const int32_t* idx;  // NULL: dense over every visible entry (HCA)
    int32_t k;
    lca_kv win;
    int32_t n_win;
    const float* sink;
    float sm_scale;
    double rope_theta;
    RopeTab rope;
    void* out;
    int32_t out_dtype;
    float* lse;
    void* ws;
    Pos q_pos;
    Pos w_base;         // (q_pos[b] - n_win + 1) mod win.cap, where that position is >= 0
    int32_t m_shift;    // log2(m) when m is a power of two, else -1
    int64_t max_keys;   // attended rows per query, upper bound
    // Window store fused into a decode launch (T = 1, bf16 raw rows): app_x holds the raw row
    // of each query position, stored into the window ring (RMSNorm with app_gamma / app_eps, RoPE
    // with rope_theta) by the launch itself; NULL = the window already holds it.
    const void* app_x;
    const float* app_gamma;
    float app_eps;
    int64_t app_stride;  // rows of app_x between sequences
};
// fp8 rows -> bf16 rows (nope codes times their scale, RoPE dims copied): for each sequence b,
// positions p in [first[b], first[b] + count[b]) of src (row b * src.cap + (p mod src.cap)) go to
// dst row b * dst.cap + (p mod dst.cap).  Used to expand a dense (HCA) launch's rows once when
// many query rows share them.
struct ExpandArgs {
    lca_kv src, dst;
    Pos first, count;
    int32_t B;
    int64_t max_count;
};
hipError_t launch_kv_expand(const ExpandArgs& a, hipStream_t st);
constexpr int64_t kExpandMinRows = 128;  // query rows from which a dense launch expands its rows
// workspace bytes a launch with this max_keys needs, and an upper bound for every launch with at
// most max_keys attended rows per query
size_t attn_ws_need(int64_t rows, int32_t H, int32_t c, int64_t max_keys);
size_t attn_ws_bytes(int64_t rows, int32_t H, int32_t c, int64_t max_keys);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
// whether launch_attn runs a.app_x's window store inside the attention launch (else the caller
// stores first)
bool attn_fuses_store(const AttnArgs& a);

// Linear map Y[b][m][n] = sum_k X[b][m][k] W[b][n][k] (bf16 X, W; f32 accumulation).  Element
// strides in elements: X (b, m, k) at x + b sx + m ldx + k, W (b, n, k) at w + b sw + n ldw + k,
// Y (b, m, n) at y + b sy + m ldy + n.  K, ldx, ldw, sx, sw multiples of 8 (16-byte rows); K >= 8.
struct GemmArgs {
    const void* x;
    const void* w;
    void* y;
    int64_t ldx, sx, ldw, sw, ldy, sy;
    int32_t M, N, K, batch;
    int32_t y_dtype;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

}  // namespace lca
