// capi.cpp -- the library's C ABI (declared in include/lca.h): host-side
// validation of every argument, then one launch on the caller's stream.
// Nothing is launched when validation fails.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/lca.h"
#include "kernels.h"
#include "status.h"
#include "trace.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    if (lca::trace_on()) lca::trace("  -> error %d: %s", code, g_err);
    return code;
}

// one trace line per call (LCA_TRACE)
#define LCA_TRACE_CALL(...)                         \
    do {                                            \
        if (lca::trace_on()) lca::trace(__VA_ARGS__); \
    } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

long long pos0(const int64_t* p) { return p ? (long long)p[0] : -1; }  // (traces only)

int check_kv(const lca_kv& kv, const char* name, bool need_rows, bool allow_fp4) {
    if (kv.fmt == LCA_MXFP4 && !allow_fp4)
        return fail(LCA_EDTYPE, "%s: MXFP4 storage holds indexer keys only", name);
    if (kv.fmt != LCA_F32 && kv.fmt != LCA_BF16 && kv.fmt != LCA_FP8 && kv.fmt != LCA_MXFP4)
        return fail(LCA_EDTYPE, "%s: unknown storage format %d", name, kv.fmt);
    if (kv.d_nope < 0 || kv.d_rope < 0 || (kv.d_rope & 1) || kv.d_nope + kv.d_rope < 1 ||
        kv.d_nope + kv.d_rope > 1024)
        return fail(LCA_ESHAPE, "%s: bad dims d_nope=%d d_rope=%d", name, kv.d_nope, kv.d_rope);
    if (kv.fmt == LCA_FP8 && (kv.d_nope % 128 != 0 || kv.d_nope == 0))
        return fail(LCA_ESHAPE, "%s: fp8 storage needs d_nope a positive multiple of 128", name);
    if (kv.fmt == LCA_MXFP4 && (kv.d_rope != 0 || kv.d_nope % 32 != 0))
        return fail(LCA_ESHAPE, "%s: MXFP4 storage needs d_rope = 0 and d_nope a multiple of 32", name);
    if (need_rows && kv.cap < 1) return fail(LCA_ESHAPE, "%s: cap must be >= 1", name);
    if (!kv.nope && kv.d_nope > 0) return fail(LCA_EINVAL, "%s: nope plane is NULL", name);
    if (!kv.rope && kv.d_rope > 0) return fail(LCA_EINVAL, "%s: rope plane is NULL", name);
    if ((kv.fmt == LCA_FP8 || kv.fmt == LCA_MXFP4) && !kv.scale)
        return fail(LCA_EINVAL, "%s: fp8 / MXFP4 storage needs scales", name);
    if (!aligned16(kv.nope) || !aligned16(kv.rope) || !aligned16(kv.scale))
        return fail(LCA_EALIGN, "%s: planes must be 16-byte aligned", name);
    return LCA_OK;
}

int check_batch(int32_t B, const int64_t* pos, const char* name) {
    if (B < 1 || B > LCA_MAX_BATCH) return fail(LCA_ESHAPE, "B=%d outside [1, %d]", B, LCA_MAX_BATCH);
    if (!pos) return fail(LCA_EINVAL, "%s is NULL", name);
    for (int b = 0; b < B; ++b)
        if (pos[b] < 0) return fail(LCA_ESHAPE, "%s[%d] = %lld is negative", name, b, (long long)pos[b]);
    return LCA_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return LCA_OK;
    return fail(LCA_EHIP, "HIP launch failed: %s", hipGetErrorString(e));
}

lca::RopeTab rope_tab(double theta, int d_rope) {
    lca::RopeTab r;
    memset(&r, 0, sizeof r);
    if (theta > 0.0)
        for (int i = 0; i < d_rope / 2 && i < lca::kMaxRopeHalf; ++i) r.inv[i] = pow(theta, -2.0 * i / d_rope);
    return r;
}

lca::Pos to_pos(const int64_t* p, int32_t B) {
    lca::Pos r;
    memset(&r, 0, sizeof r);
    for (int b = 0; b < B; ++b) r.v[b] = p[b];
    return r;
}

}  // namespace

namespace lca {
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    if (trace_on()) trace("  -> error %d: %s", code, g_err);
    return code;
}
bool trace_on() {
    static const bool on = [] {
        const char* e = getenv("LCA_TRACE");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return on;
}
void trace(const char* fmt, ...) {
    char line[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(line, sizeof line, fmt, ap);
    va_end(ap);
    fprintf(stderr, "[lca] %s\n", line);
}
void clear_error() { g_err[0] = 0; }
}  // namespace lca

extern "C" {

int lca_version(void) { return LCA_VERSION; }

const char* lca_last_error(void) { return g_err; }

// lca_kv_compress_ws splits entries when the pooled row list is long and the inputs take kv_pool_wide
static bool compress_splits(int32_t in_dtype, int32_t m, int32_t overlap, int32_t c) {
    return in_dtype == LCA_BF16 && c > 0 && c % 8 == 0 && c <= 576 && (int64_t)m * (1 + overlap) >= lca::kCompressMinList;
}

size_t lca_compress_workspace_size(int32_t in_dtype, int32_t m, int32_t overlap, int32_t d_nope, int32_t d_rope) {
    if (m < 1 || (overlap != 0 && overlap != 1) || d_nope < 0 || d_rope < 0) return 0;
    const int32_t c = d_nope + d_rope;
    if (!compress_splits(in_dtype, m, overlap, c)) return 0;
    return (size_t)lca::kCompressUnits * 3 * (size_t)c * sizeof(float);
}

static int kv_compress_common(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                              int32_t in_dtype, const float* bias_a, const float* bias_b, const float* gamma,
                              float eps, double rope_theta, int32_t m, int32_t overlap, int32_t B, int64_t n_rows,
                              int64_t in_stride, const int64_t* first_pos, lca_kv out, int32_t ring, void* ws,
                              size_t ws_bytes, void* stream) {
    if (!c_a || !z_a) return fail(LCA_EINVAL, "c_a / z_a is NULL");
    if (m < 1) return fail(LCA_EINVAL, "m must be >= 1 (got %d)", m);
    if (overlap != 0 && overlap != 1) return fail(LCA_EINVAL, "overlap must be 0 or 1");
    if (overlap && (!c_b || !z_b)) return fail(LCA_EINVAL, "overlap needs c_b and z_b");
    if (ring != 0 && ring != 1) return fail(LCA_EINVAL, "ring must be 0 or 1");
    if (in_dtype != LCA_F32 && in_dtype != LCA_BF16) return fail(LCA_EDTYPE, "in_dtype must be f32 or bf16");
    if (n_rows < 0) return fail(LCA_ESHAPE, "n_rows < 0");
    if (in_stride < 0 || (in_stride > 0 && in_stride < n_rows))
        return fail(LCA_ESHAPE, "in_stride %lld is smaller than n_rows %lld", (long long)in_stride, (long long)n_rows);
    if (!(rope_theta >= 0.0)) return fail(LCA_EINVAL, "rope_theta must be >= 0");
    if (!(eps >= 0.0f)) return fail(LCA_EINVAL, "eps must be >= 0");
    int rc = check_batch(B, first_pos, "first_pos");
    if (rc) return rc;
    if ((rc = check_kv(out, "out", true, true))) return rc;
    if (rope_theta > 0.0 && out.d_rope > 2 * lca::kMaxRopeHalf)
        return fail(LCA_ESHAPE, "RoPE supports d_rope <= %d", 2 * lca::kMaxRopeHalf);
    for (const void* p : {c_a, z_a, c_b, z_b, (const void*)bias_a, (const void*)bias_b, (const void*)gamma})
        if (!aligned16(p)) return fail(LCA_EALIGN, "input pointers must be 16-byte aligned");

    lca::CompressArgs a;
    memset(&a, 0, sizeof a);
    a.c_a = c_a; a.z_a = z_a; a.c_b = c_b; a.z_b = z_b;
    a.bias_a = bias_a; a.bias_b = bias_b; a.gamma = gamma;
    a.eps = eps; a.rope_theta = rope_theta; a.in_dtype = in_dtype;
    a.rope = rope_tab(rope_theta, out.d_rope);
    a.m = m; a.overlap = overlap; a.B = B; a.n_rows = n_rows; a.out = out; a.ring = ring;
    a.in_stride = in_stride > 0 ? in_stride : n_rows;
    a.first_pos = to_pos(first_pos, B);
    int64_t most = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t p0 = first_pos[b];
        int64_t s_lo = (p0 + m - 1) / m;
        if (overlap && s_lo > 0) s_lo += 1;
        const int64_t s_hi = (p0 + n_rows) / m;
        if (ring && s_hi - s_lo > out.cap) s_lo = s_hi - out.cap;
        a.s_lo.v[b] = s_lo;
        if (s_hi > s_lo) {
            if (!ring && s_hi > out.cap)
                return fail(LCA_ESHAPE, "entry %lld of sequence %d does not fit cap %lld",
                            (long long)(s_hi - 1), b, (long long)out.cap);
            if (s_hi - s_lo > most) most = s_hi - s_lo;
        }
    }
    if (most > 0x7fffffff) return fail(LCA_ESHAPE, "too many entries in one call");
    a.max_entries = most;
    const int32_t c = out.d_nope + out.d_rope;
    if (ws && most > 0 && compress_splits(in_dtype, m, overlap, c) && !(m == 1 && !overlap) &&
        (int64_t)B * most * 2 <= lca::kCompressUnits) {
        if (!aligned16(ws)) return fail(LCA_EALIGN, "ws must be 16-byte aligned");
        const int64_t list = (int64_t)m * (1 + overlap);  // rows of an entry's list, at most
        int64_t parts = lca::kCompressUnits / ((int64_t)B * most);
        if (parts > lca::kCompressMaxParts) parts = lca::kCompressMaxParts;
        if (parts > list / lca::kCompressMinRows) parts = list / lca::kCompressMinRows;
        const int64_t len = (list + parts - 1) / parts;
        parts = (list + len - 1) / len;
        const size_t need = (size_t)B * (size_t)most * (size_t)parts * 3 * (size_t)c * sizeof(float);
        if (ws_bytes < need)
            return fail(LCA_EWORKSPACE, "compressor workspace too small: %zu < %zu bytes", ws_bytes, need);
        if (parts > 1) {
            a.ws = (float*)ws;
            a.parts = (int32_t)parts;
            a.part_len = (int32_t)len;
        }
    }
    return hip_status(lca::launch_kv_compress(a, (hipStream_t)stream));
}

int lca_kv_compress(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                    int32_t in_dtype, const float* bias_a, const float* bias_b, const float* gamma,
                    float eps, double rope_theta, int32_t m, int32_t overlap, int32_t B, int64_t n_rows,
                    int64_t in_stride, const int64_t* first_pos, lca_kv out, int32_t ring, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_kv_compress B=%d rows=%lld in_dtype=%d m=%d overlap=%d out fmt=%d dims=%d+%d cap=%lld ring=%d "
                   "first_pos[0]=%lld", B, (long long)n_rows, in_dtype, m, overlap, out.fmt, out.d_nope, out.d_rope,
                   (long long)out.cap, ring, pos0(first_pos));
    return kv_compress_common(c_a, z_a, c_b, z_b, in_dtype, bias_a, bias_b, gamma, eps, rope_theta, m, overlap, B,
                              n_rows, in_stride, first_pos, out, ring, nullptr, 0, stream);
}

int lca_kv_compress_ws(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                       int32_t in_dtype, const float* bias_a, const float* bias_b, const float* gamma,
                       float eps, double rope_theta, int32_t m, int32_t overlap, int32_t B, int64_t n_rows,
                       int64_t in_stride, const int64_t* first_pos, lca_kv out, int32_t ring, void* ws,
                       size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_kv_compress_ws B=%d rows=%lld in_dtype=%d m=%d overlap=%d out fmt=%d dims=%d+%d cap=%lld "
                   "ring=%d ws=%zu first_pos[0]=%lld", B, (long long)n_rows, in_dtype, m, overlap, out.fmt, out.d_nope,
                   out.d_rope, (long long)out.cap, ring, ws_bytes, pos0(first_pos));
    return kv_compress_common(c_a, z_a, c_b, z_b, in_dtype, bias_a, bias_b, gamma, eps, rope_theta, m, overlap, B,
                              n_rows, in_stride, first_pos, out, ring, ws, ws_bytes, stream);
}

int lca_indexer_score(const void* q, const float* w, const void* k, int32_t in_dtype, int64_t k_cap,
                      int32_t H_I, int32_t d_I, int32_t B, int32_t T, const int64_t* q_pos, int32_t m,
                      void* scores, int32_t score_dtype, int64_t s_stride, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_indexer_score B=%d T=%d keys fmt=%d k_cap=%lld H_I=%d d_I=%d m=%d score_dtype=%d s_stride=%lld "
                   "q_pos[0]=%lld", B, T, in_dtype, (long long)k_cap, H_I, d_I, m, score_dtype, (long long)s_stride,
                   pos0(q_pos));
    if (!q || !k || !scores) return fail(LCA_EINVAL, "q, k and scores must be non-NULL");
    if (m < 1) return fail(LCA_EINVAL, "m must be >= 1");
    if (in_dtype != LCA_BF16 && in_dtype != LCA_F32) return fail(LCA_EDTYPE, "in_dtype must be bf16 or f32");
    if (score_dtype != LCA_BF16 && score_dtype != LCA_F32) return fail(LCA_EDTYPE, "score_dtype must be bf16 or f32");
    if (T < 0 || k_cap < 1 || s_stride < 1) return fail(LCA_ESHAPE, "bad T / k_cap / s_stride");
    if (in_dtype == LCA_BF16 && (H_I != 16 || d_I != 128))
        return fail(LCA_ESHAPE, "bf16 indexer supports H_I = 16, d_I = 128 (got %d x %d)", H_I, d_I);
    if (H_I < 1 || H_I > 64 || d_I < 1 || d_I > 1024) return fail(LCA_ESHAPE, "bad H_I / d_I");
    int rc = check_batch(B, q_pos, "q_pos");
    if (rc) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(w) || !aligned16(scores))
        return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    int64_t max_vis = 0;
    for (int b = 0; b < B && T > 0; ++b) {
        const int64_t vis = (q_pos[b] + T) / m;
        if (vis > k_cap || vis > s_stride)
            return fail(LCA_ESHAPE, "sequence %d sees %lld entries: more than k_cap %lld or s_stride %lld", b,
                        (long long)vis, (long long)k_cap, (long long)s_stride);
        if (vis > max_vis) max_vis = vis;
    }
    lca::IndexerArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.w = w; a.k = k; a.in_dtype = in_dtype; a.k_cap = k_cap; a.H_I = H_I; a.d_I = d_I;
    a.B = B; a.T = T; a.m = m; a.scores = scores; a.score_dtype = score_dtype; a.s_stride = s_stride;
    a.q_pos = to_pos(q_pos, B);
    a.max_vis = max_vis;
    return hip_status(lca::launch_indexer(a, (hipStream_t)stream));
}

int lca_indexer_score_mxfp4(const void* q, const float* w, lca_kv k, int32_t H_I, int32_t d_I, int32_t B,
                            int32_t T, const int64_t* q_pos, int32_t m, void* scores, int32_t score_dtype,
                            int64_t s_stride, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_indexer_score_mxfp4 B=%d T=%d k_cap=%lld H_I=%d d_I=%d m=%d score_dtype=%d s_stride=%lld "
                   "q_pos[0]=%lld", B, T, (long long)k.cap, H_I, d_I, m, score_dtype, (long long)s_stride, pos0(q_pos));
    if (!q || !scores) return fail(LCA_EINVAL, "q and scores must be non-NULL");
    if (m < 1) return fail(LCA_EINVAL, "m must be >= 1");
    if (k.fmt != LCA_MXFP4) return fail(LCA_EDTYPE, "keys must be stored MXFP4 (fmt %d)", LCA_MXFP4);
    int rc = check_kv(k, "k", true, true);
    if (rc) return rc;
    if (score_dtype != LCA_BF16 && score_dtype != LCA_F32) return fail(LCA_EDTYPE, "score_dtype must be bf16 or f32");
    if (H_I != 16 || d_I != 128 || k.d_nope != d_I)
        return fail(LCA_ESHAPE, "MXFP4 indexer supports H_I = 16, d_I = k.d_nope = 128 (got %d x %d, keys %d)", H_I,
                    d_I, k.d_nope);
    if (T < 0 || s_stride < 1) return fail(LCA_ESHAPE, "bad T / s_stride");
    if ((rc = check_batch(B, q_pos, "q_pos"))) return rc;
    if (!aligned16(q) || !aligned16(w) || !aligned16(scores)) return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    int64_t max_vis = 0;
    for (int b = 0; b < B && T > 0; ++b) {
        const int64_t vis = (q_pos[b] + T) / m;
        if (vis > k.cap || vis > s_stride)
            return fail(LCA_ESHAPE, "sequence %d sees %lld entries: more than k.cap %lld or s_stride %lld", b,
                        (long long)vis, (long long)k.cap, (long long)s_stride);
        if (vis > max_vis) max_vis = vis;
    }
    lca::IndexerArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.w = w; a.k = k.nope; a.k_scale = k.scale; a.in_dtype = LCA_MXFP4; a.k_cap = k.cap;
    a.H_I = H_I; a.d_I = d_I; a.B = B; a.T = T; a.m = m; a.scores = scores; a.score_dtype = score_dtype;
    a.s_stride = s_stride; a.q_pos = to_pos(q_pos, B); a.max_vis = max_vis;
    return hip_status(lca::launch_indexer(a, (hipStream_t)stream));
}

size_t lca_topk_workspace_size(int32_t B, int32_t T, int64_t s_stride, int32_t) {
    if (B < 1 || T < 1 || s_stride < 1) return 0;
    return lca::topk_ws_bytes(B, T, s_stride, LCA_BF16);
}

int lca_topk_select(const void* scores, int32_t score_dtype, int64_t s_stride, int32_t B, int32_t T,
                    const int64_t* q_pos, int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                    void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_topk_select B=%d T=%d score_dtype=%d s_stride=%lld m=%d k=%d ws=%zu q_pos[0]=%lld", B, T,
                   score_dtype, (long long)s_stride, m, k, ws_bytes, pos0(q_pos));
    if (!scores || !idx) return fail(LCA_EINVAL, "scores and idx must be non-NULL");
    if (m < 1) return fail(LCA_EINVAL, "m must be >= 1");
    if (k < 1) return fail(LCA_EINVAL, "k must be >= 1");
    if (score_dtype != LCA_BF16 && score_dtype != LCA_F32) return fail(LCA_EDTYPE, "score_dtype must be bf16 or f32");
    if (T < 0 || s_stride < 1) return fail(LCA_ESHAPE, "bad T / s_stride");
    int rc = check_batch(B, q_pos, "q_pos");
    if (rc) return rc;
    if (!aligned16(scores) || !aligned16(idx) || !aligned16(ws)) return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    int64_t max_n = 0;
    for (int b = 0; b < B && T > 0; ++b) {
        const int64_t n = (q_pos[b] + T) / m;
        if (n > s_stride) return fail(LCA_ESHAPE, "sequence %d sees more entries than s_stride", b);
        if (n > max_n) max_n = n;
    }
    if (T == 0) return LCA_OK;
    const size_t need = lca::topk_ws_bytes(B, T, s_stride, score_dtype);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(LCA_EWORKSPACE, "top-k workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    lca::TopkArgs a;
    memset(&a, 0, sizeof a);
    a.scores = scores; a.score_dtype = score_dtype; a.s_stride = s_stride; a.B = B; a.T = T; a.m = m;
    a.k = k; a.idx = idx; a.ws = ws; a.max_n = max_n; a.q_pos = to_pos(q_pos, B);
    return hip_status(lca::launch_topk(a, (hipStream_t)stream));
}

// Workspace of lca_indexer_topk for B x T query rows: the top-k's first-pass histograms as the indexer
// builds them, from the workspace's first byte.  Split schedule (few long rows): per row its
// kTopkChunk-key chunks' histograms, then the top-k's own second-pass histograms and figures (which need
// no zeros).  Row schedule: one histogram per row.  A call clears the first-pass histograms again.

static int indexer_topk_launch(lca::IndexerArgs ia, int32_t topk, int32_t* idx, void* ws, size_t ws_bytes,
                               void* stream);

size_t lca_indexer_topk_workspace_size(int32_t B, int32_t T, int64_t s_stride, int32_t k) {
    if (B < 1 || T < 1 || s_stride < 1 || k < 1) return 0;
    const int32_t rows = B * T;
    size_t split = 0;
    if (lca::topk_split_chunks(rows, s_stride, s_stride, LCA_BF16) > 0)
        split = lca::topk_ws_bytes(rows, 1, s_stride, LCA_BF16);
    const size_t row = (size_t)rows * 256 * sizeof(uint32_t);
    return split > row ? split : row;
}

// the validation both forms share: shapes, positions, alignment; fills max_vis
static int indexer_topk_check(const void* q, const void* scores, const int32_t* idx, const float* w, const void* ws,
                              int32_t m, int32_t topk, int32_t B, int32_t T, const int64_t* q_pos, int64_t k_cap,
                              int64_t s_stride, int64_t* max_vis) {
    if (!q || !scores || !idx) return fail(LCA_EINVAL, "q, scores and idx must be non-NULL");
    if (m < 1) return fail(LCA_EINVAL, "m must be >= 1");
    if (topk < 1) return fail(LCA_EINVAL, "k must be >= 1");
    if (T < 0) return fail(LCA_ESHAPE, "T < 0");
    if (k_cap < 1 || s_stride < 1) return fail(LCA_ESHAPE, "bad k_cap / s_stride");
    int rc = check_batch(B, q_pos, "q_pos");
    if (rc) return rc;
    if (!aligned16(q) || !aligned16(w) || !aligned16(scores) || !aligned16(idx) || !aligned16(ws))
        return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    *max_vis = 0;
    for (int b = 0; b < B && T > 0; ++b) {
        const int64_t vis = (q_pos[b] + T) / m;
        if (vis > k_cap || vis > s_stride)
            return fail(LCA_ESHAPE, "sequence %d sees %lld entries: more than k_cap %lld or s_stride %lld", b,
                        (long long)vis, (long long)k_cap, (long long)s_stride);
        if (vis > *max_vis) *max_vis = vis;
    }
    return LCA_OK;
}

int lca_indexer_topk(const void* q, const float* w, const void* k, int64_t k_cap, int32_t H_I, int32_t d_I,
                     int32_t B, int32_t T, const int64_t* q_pos, int32_t m, void* scores, int64_t s_stride,
                     int32_t topk, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_indexer_topk B=%d T=%d k_cap=%lld H_I=%d d_I=%d m=%d s_stride=%lld k=%d ws=%zu q_pos[0]=%lld",
                   B, T, (long long)k_cap, H_I, d_I, m, (long long)s_stride, topk, ws_bytes, pos0(q_pos));
    if (!k) return fail(LCA_EINVAL, "k must be non-NULL");
    if (H_I != 16 || d_I != 128)
        return fail(LCA_ESHAPE, "the indexer supports H_I = 16, d_I = 128 (got %d x %d)", H_I, d_I);
    int64_t max_vis = 0;
    int rc = indexer_topk_check(q, scores, idx, w, ws, m, topk, B, T, q_pos, k_cap, s_stride, &max_vis);
    if (rc) return rc;
    if (!aligned16(k)) return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    if (T == 0) return LCA_OK;
    lca::IndexerArgs ia;
    memset(&ia, 0, sizeof ia);
    ia.q = q; ia.w = w; ia.k = k; ia.in_dtype = LCA_BF16; ia.k_cap = k_cap; ia.H_I = H_I; ia.d_I = d_I;
    ia.B = B; ia.T = T; ia.m = m; ia.scores = scores; ia.score_dtype = LCA_BF16; ia.s_stride = s_stride;
    ia.q_pos = to_pos(q_pos, B);
    ia.max_vis = max_vis;
    return indexer_topk_launch(ia, topk, idx, ws, ws_bytes, stream);
}

// the shared part of lca_indexer_topk(_mxfp4): the workspace check and the launches
static int indexer_topk_launch(lca::IndexerArgs ia, int32_t topk, int32_t* idx, void* ws, size_t ws_bytes,
                               void* stream) {
    const int32_t B = ia.B, T = ia.T, rows = B * T;
    const int64_t s_stride = ia.s_stride, max_vis = ia.max_vis;
    const size_t need = lca_indexer_topk_workspace_size(B, T, s_stride, topk);
    if (!ws || ws_bytes < need)
        return fail(LCA_EWORKSPACE, "indexer + top-k workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    lca::TopkArgs ta;
    memset(&ta, 0, sizeof ta);
    ta.scores = ia.scores; ta.score_dtype = LCA_BF16; ta.s_stride = s_stride; ta.B = B; ta.T = T; ta.m = ia.m;
    ta.k = topk; ta.idx = idx; ta.ws = ws; ta.max_n = max_vis; ta.q_pos = ia.q_pos;
    ia.th_h1 = (uint32_t*)ws;
    const int G = lca::topk_split_chunks(rows, max_vis, s_stride, LCA_BF16);
    LCA_TRACE_CALL("  indexer_topk: %s schedule%s, %d chunk(s) of %d keys per row", G > 0 ? "split" : "row",
                   G > 0 ? " (top-k: second-digit and emission launches)" : "", G > 0 ? G : 1,
                   G > 0 ? lca::kTopkChunk : (int)s_stride);
    if (G > 0) {  // split schedule: the chunks' histograms; the top-k runs its last two launches
        ia.th_row = (int64_t)G * lca::kTopkHistWords;
        ia.th_chunked = 1;
        ta.split_fused = 1;
    } else {      // row schedule: one histogram per row; the top-k skips its first pass
        ia.th_row = 256;
        ia.th_chunked = 0;
        ta.row_h1 = (uint32_t*)ws;
    }
    if (max_vis > 0) {
        hipError_t e = lca::launch_indexer(ia, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(lca::launch_topk(ta, (hipStream_t)stream));
}

int lca_indexer_topk_mxfp4(const void* q, const float* w, lca_kv k, int32_t H_I, int32_t d_I, int32_t B,
                           int32_t T, const int64_t* q_pos, int32_t m, void* scores, int64_t s_stride, int32_t topk,
                           int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_indexer_topk_mxfp4 B=%d T=%d k_cap=%lld H_I=%d d_I=%d m=%d s_stride=%lld k=%d ws=%zu "
                   "q_pos[0]=%lld", B, T, (long long)k.cap, H_I, d_I, m, (long long)s_stride, topk, ws_bytes, pos0(q_pos));
    if (k.fmt != LCA_MXFP4) return fail(LCA_EDTYPE, "keys must be stored MXFP4 (fmt %d)", LCA_MXFP4);
    int rc = check_kv(k, "k", true, true);
    if (rc) return rc;
    if (H_I != 16 || d_I != 128 || k.d_nope != d_I)
        return fail(LCA_ESHAPE, "MXFP4 indexer supports H_I = 16, d_I = k.d_nope = 128 (got %d x %d, keys %d)", H_I,
                    d_I, k.d_nope);
    int64_t max_vis = 0;
    if ((rc = indexer_topk_check(q, scores, idx, w, ws, m, topk, B, T, q_pos, k.cap, s_stride, &max_vis))) return rc;
    if (T == 0) return LCA_OK;
    lca::IndexerArgs ia;
    memset(&ia, 0, sizeof ia);
    ia.q = q; ia.w = w; ia.k = k.nope; ia.k_scale = k.scale; ia.in_dtype = LCA_MXFP4; ia.k_cap = k.cap;
    ia.H_I = H_I; ia.d_I = d_I; ia.B = B; ia.T = T; ia.m = m; ia.scores = scores; ia.score_dtype = LCA_BF16;
    ia.s_stride = s_stride; ia.q_pos = to_pos(q_pos, B); ia.max_vis = max_vis;
    return indexer_topk_launch(ia, topk, idx, ws, ws_bytes, stream);
}

// Bytes of one expanded (bf16) row, and the expansion's bound: at most max_keys compressed rows
// plus a window ring of at most max_keys + T - 1 rows per sequence.
static constexpr size_t kExpandRowBytes = (512 + 64) * sizeof(uint16_t);
static size_t expand_bound(int64_t B, int64_t T, int64_t max_keys) {
    if (B * T < lca::kExpandMinRows) return 0;
    return (size_t)B * (size_t)(2 * max_keys + T) * kExpandRowBytes;
}

size_t lca_attn_workspace_size(int32_t B, int32_t T, int32_t H, int32_t c, int64_t max_keys) {
    if (B < 1 || T < 1 || H < 1 || c < 1 || max_keys < 1) return 0;
    const size_t split = lca::attn_ws_bytes((int64_t)B * T, H, c, max_keys);
    const size_t expand = c == 576 ? expand_bound(B, T, max_keys) : 0;
    return split > expand ? split : expand;
}

// The m = 1 ring store of rows q_pos[b] .. q_pos[b] + T - 1 of x (x_stride rows per sequence) into win (what
// lca_kv_compress does with m = 1, overlap = 0, ring = 1 and first_pos = q_pos).
static hipError_t store_window_rows(const void* x, int32_t x_dtype, int64_t x_stride, const float* gamma, float eps,
                                    double rope_theta, int32_t B, int32_t T, const int64_t* q_pos, const lca_kv& win,
                                    hipStream_t st) {
    lca::CompressArgs c;
    memset(&c, 0, sizeof c);
    c.c_a = x; c.z_a = x; c.gamma = gamma; c.eps = eps; c.rope_theta = rope_theta; c.in_dtype = x_dtype;
    c.rope = rope_tab(rope_theta, win.d_rope);
    c.m = 1; c.overlap = 0; c.B = B; c.n_rows = T; c.in_stride = x_stride; c.out = win; c.ring = 1;
    c.first_pos = to_pos(q_pos, B);
    int64_t most = 0;
    for (int b = 0; b < B; ++b) {
        int64_t s_lo = q_pos[b];
        if (T > win.cap) s_lo = q_pos[b] + T - win.cap;
        c.s_lo.v[b] = s_lo;
        const int64_t n = q_pos[b] + T - s_lo;
        if (n > most) most = n;
    }
    c.max_entries = most;
    return lca::launch_kv_compress(c, st);
}

static int attn_common(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T,
                       const int64_t* q_pos, lca_kv comp, int32_t m, const int32_t* idx, int32_t k,
                       lca_kv win, int32_t n_win, const float* sink, float sm_scale, double rope_theta,
                       void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream,
                       const void* x_win = nullptr, int32_t x_dtype = 0, int64_t x_stride = 0,
                       const float* x_gamma = nullptr, float x_eps = 0.0f) {
    if (!q || !out) return fail(LCA_EINVAL, "q and out must be non-NULL");
    if (m < 1) return fail(LCA_EINVAL, "m must be >= 1");
    if (H < 1 || T < 0) return fail(LCA_ESHAPE, "bad H / T");
    if (n_win < 0) return fail(LCA_EINVAL, "n_win must be >= 0");
    if (!(rope_theta >= 0.0)) return fail(LCA_EINVAL, "rope_theta must be >= 0");
    if (!(sm_scale == sm_scale)) return fail(LCA_EINVAL, "sm_scale is NaN");
    if (out_dtype != LCA_F32 && out_dtype != LCA_BF16) return fail(LCA_EDTYPE, "out_dtype must be f32 or bf16");
    int rc = check_batch(B, q_pos, "q_pos");
    if (rc) return rc;
    if ((rc = check_kv(comp, "comp", true, false))) return rc;
    if (n_win > 0) {
        if ((rc = check_kv(win, "win", true, false))) return rc;
        if (win.fmt != comp.fmt || win.d_nope != comp.d_nope || win.d_rope != comp.d_rope)
            return fail(LCA_ESHAPE, "window and compressed caches must share format and dims");
        for (int b = 0; b < B; ++b) {  // rows [q_pos - n_win + 1, q_pos + T - 1] that exist
            const int64_t back = (int64_t)n_win - 1 < q_pos[b] ? (int64_t)n_win - 1 : q_pos[b];
            if (back + T > win.cap)
                return fail(LCA_ESHAPE, "window ring too small for sequence %d: %lld rows > cap %lld", b,
                            (long long)(back + T), (long long)win.cap);
        }
    }
    const int c = comp.d_nope + comp.d_rope;
    if (rope_theta > 0.0 && comp.d_rope > 2 * lca::kMaxRopeHalf)
        return fail(LCA_ESHAPE, "RoPE supports d_rope <= %d", 2 * lca::kMaxRopeHalf);
    if (comp.fmt == LCA_F32) {
        if (q_dtype != LCA_F32) return fail(LCA_EDTYPE, "f32 caches need f32 queries");
    } else {
        if (q_dtype != LCA_BF16) return fail(LCA_EDTYPE, "bf16 / fp8 caches need bf16 queries");
        if (comp.d_nope != 512 || comp.d_rope != 64)
            return fail(LCA_ESHAPE, "bf16 / fp8 caches support d_nope = 512, d_rope = 64");
        if (H > 64) return fail(LCA_ESHAPE, "bf16 / fp8 caches support H <= 64");
    }
    if (!aligned16(q) || !aligned16(out) || !aligned16(lse) || !aligned16(idx) || !aligned16(sink) ||
        !aligned16(ws) || !aligned16(x_win) || !aligned16(x_gamma))
        return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    if (x_win) {
        if (n_win < 1) return fail(LCA_EINVAL, "the window store needs n_win >= 1");
        if (x_dtype != LCA_F32 && x_dtype != LCA_BF16) return fail(LCA_EDTYPE, "x_dtype must be f32 or bf16");
        if (!(x_eps >= 0.0f)) return fail(LCA_EINVAL, "eps must be >= 0");
        if (x_stride < 0 || (x_stride > 0 && x_stride < T))
            return fail(LCA_ESHAPE, "x_stride %lld is smaller than T %d", (long long)x_stride, T);
        if (rope_theta > 0.0 && win.d_rope > 2 * lca::kMaxRopeHalf)
            return fail(LCA_ESHAPE, "RoPE supports d_rope <= %d", 2 * lca::kMaxRopeHalf);
    }
    if (T == 0) return LCA_OK;
    int64_t max_keys = 1;
    for (int b = 0; b < B; ++b) {
        const int64_t t_last = q_pos[b] + T - 1;
        int64_t keys = n_win > 0 ? (n_win < t_last + 1 ? n_win : t_last + 1) : 0;
        if (idx) {
            keys += k;
        } else {
            const int64_t vis = (t_last + 1) / m;
            if (vis > comp.cap)
                return fail(LCA_ESHAPE, "sequence %d sees %lld entries, cap is %lld", b, (long long)vis,
                            (long long)comp.cap);
            keys += vis;
        }
        if (keys > max_keys) max_keys = keys;
    }
    const size_t need = lca::attn_ws_need((int64_t)B * T, H, c, max_keys);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(LCA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    lca::AttnArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.q_dtype = q_dtype; a.H = H; a.B = B; a.T = T; a.m = m; a.comp = comp; a.idx = idx; a.k = k;
    a.win = win; a.n_win = n_win; a.sink = sink; a.sm_scale = sm_scale; a.rope_theta = rope_theta;
    a.rope = rope_tab(rope_theta, comp.d_rope);
    a.out = out; a.out_dtype = out_dtype; a.lse = lse; a.ws = ws; a.q_pos = to_pos(q_pos, B);
    a.max_keys = max_keys;
    a.m_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if (((int64_t)1 << sh) == m) a.m_shift = sh;
    for (int b = 0; b < B; ++b) {
        const int64_t d = q_pos[b] - n_win + 1;
        a.w_base.v[b] = d >= 0 && win.cap > 0 ? d % win.cap : 0;
    }
    if (n_win == 0) a.win = comp;  // never read
    if (x_win) {
        // the window store of the call's own rows: inside a decode launch when it can take it, else
        // as its own launch before anything reads the window
        a.app_x = x_win;
        a.app_gamma = x_gamma;
        a.app_eps = x_eps;
        a.app_stride = x_stride > 0 ? x_stride : T;
        if (x_dtype != LCA_BF16 || !lca::attn_fuses_store(a)) {
            a.app_x = nullptr;
            hipError_t e = store_window_rows(x_win, x_dtype, a.app_stride, x_gamma, x_eps, rope_theta, B, T, q_pos,
                                             win, (hipStream_t)stream);
            if (e != hipSuccess) return hip_status(e);
        }
    }

    // Dense fp8 launches with many query rows share every row: expand the rows they read to bf16
    // once (compressed rows [0, vis) and the window positions the rows need, into a ring of
    // min(n_win - 1, q_pos) + T rows), when the workspace holds them; otherwise the attention
    // expands per tile.
    if (!idx && comp.fmt == LCA_FP8 && (int64_t)B * T >= lca::kExpandMinRows &&
        lca::attn_ws_need((int64_t)B * T, H, c, max_keys) == 0) {
        int64_t cap_c = 1, cap_w = 1;
        for (int b = 0; b < B; ++b) {
            const int64_t vis = (q_pos[b] + T) / m;
            if (vis > cap_c) cap_c = vis;
        }
        if (n_win > 0) {  // the ring rule: min(n_win - 1, q_pos) + T rows
            int64_t back = 0;
            for (int b = 0; b < B; ++b) {
                const int64_t k1 = (int64_t)n_win - 1 < q_pos[b] ? (int64_t)n_win - 1 : q_pos[b];
                if (k1 > back) back = k1;
            }
            cap_w = back + T;
        }
        const size_t bytes = (size_t)B * (size_t)(cap_c + (n_win > 0 ? cap_w : 0)) * kExpandRowBytes;
        if (ws && ws_bytes >= bytes) {
            uint16_t* base = (uint16_t*)ws;
            lca_kv ec;
            ec.fmt = LCA_BF16; ec.d_nope = 512; ec.d_rope = 64; ec.scale = nullptr; ec.cap = cap_c;
            ec.nope = base;
            ec.rope = base + (size_t)B * cap_c * 512;
            lca::ExpandArgs x;
            memset(&x, 0, sizeof x);
            x.src = comp; x.dst = ec; x.B = B;
            for (int b = 0; b < B; ++b) {
                x.first.v[b] = 0;
                x.count.v[b] = (q_pos[b] + T) / m;
                if (x.count.v[b] > x.max_count) x.max_count = x.count.v[b];
            }
            hipError_t e = lca::launch_kv_expand(x, (hipStream_t)stream);
            if (e != hipSuccess) return hip_status(e);
            a.comp = ec;
            if (n_win > 0) {
                lca_kv ew = ec;
                ew.cap = cap_w;
                ew.nope = base + (size_t)B * cap_c * 576;
                ew.rope = (uint16_t*)ew.nope + (size_t)B * cap_w * 512;
                x.src = win; x.dst = ew; x.max_count = 0;
                for (int b = 0; b < B; ++b) {
                    const int64_t lo = q_pos[b] - n_win + 1 < 0 ? 0 : q_pos[b] - n_win + 1;
                    x.first.v[b] = lo;
                    x.count.v[b] = q_pos[b] + T - lo;
                    if (x.count.v[b] > x.max_count) x.max_count = x.count.v[b];
                    const int64_t d = q_pos[b] - n_win + 1;
                    a.w_base.v[b] = d >= 0 ? d % cap_w : 0;
                }
                if ((e = lca::launch_kv_expand(x, (hipStream_t)stream)) != hipSuccess) return hip_status(e);
                a.win = ew;
            } else {
                a.win = ec;
            }
        }
    }
    return hip_status(lca::launch_attn(a, (hipStream_t)stream));
}

int lca_csa_attn(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T, const int64_t* q_pos,
                 lca_kv comp, int32_t m, const int32_t* idx, int32_t k, lca_kv win, int32_t n_win,
                 const float* sink, float sm_scale, double rope_theta, void* out, int32_t out_dtype,
                 float* lse, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_csa_attn B=%d T=%d H=%d q_dtype=%d comp fmt=%d cap=%lld m=%d k=%d win cap=%lld n_win=%d out_dtype=%d "
                   "ws=%zu q_pos[0]=%lld", B, T, H, q_dtype, comp.fmt, (long long)comp.cap, m, k, (long long)win.cap, n_win,
                   out_dtype, ws_bytes, pos0(q_pos));
    if (!idx) return fail(LCA_EINVAL, "idx is NULL");
    if (k < 1) return fail(LCA_EINVAL, "k must be >= 1");
    return attn_common(q, q_dtype, H, B, T, q_pos, comp, m, idx, k, win, n_win, sink, sm_scale, rope_theta,
                       out, out_dtype, lse, ws, ws_bytes, stream);
}

int lca_csa_attn_append(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T, const int64_t* q_pos,
                        lca_kv comp, int32_t m, const int32_t* idx, int32_t k, lca_kv win, int32_t n_win,
                        const void* x_win, int32_t x_dtype, int64_t x_stride, const float* gamma, float eps,
                        const float* sink, float sm_scale, double rope_theta, void* out, int32_t out_dtype,
                        float* lse, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_csa_attn_append B=%d T=%d H=%d q_dtype=%d comp fmt=%d cap=%lld m=%d k=%d win cap=%lld n_win=%d out_dtype=%d "
                   "ws=%zu q_pos[0]=%lld", B, T, H, q_dtype, comp.fmt, (long long)comp.cap, m, k, (long long)win.cap, n_win,
                   out_dtype, ws_bytes, pos0(q_pos));
    if (!idx) return fail(LCA_EINVAL, "idx is NULL");
    if (k < 1) return fail(LCA_EINVAL, "k must be >= 1");
    if (!x_win) return fail(LCA_EINVAL, "x_win is NULL");
    return attn_common(q, q_dtype, H, B, T, q_pos, comp, m, idx, k, win, n_win, sink, sm_scale, rope_theta, out,
                       out_dtype, lse, ws, ws_bytes, stream, x_win, x_dtype, x_stride, gamma, eps);
}

int lca_hca_attn_append(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T, const int64_t* q_pos,
                        lca_kv comp, int32_t m, lca_kv win, int32_t n_win, const void* x_win, int32_t x_dtype,
                        int64_t x_stride, const float* gamma, float eps, const float* sink, float sm_scale,
                        double rope_theta, void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                        void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_hca_attn_append B=%d T=%d H=%d q_dtype=%d comp fmt=%d cap=%lld m=%d k=%d win cap=%lld n_win=%d out_dtype=%d "
                   "ws=%zu q_pos[0]=%lld", B, T, H, q_dtype, comp.fmt, (long long)comp.cap, m, 0, (long long)win.cap, n_win,
                   out_dtype, ws_bytes, pos0(q_pos));
    if (!x_win) return fail(LCA_EINVAL, "x_win is NULL");
    return attn_common(q, q_dtype, H, B, T, q_pos, comp, m, nullptr, 0, win, n_win, sink, sm_scale, rope_theta,
                       out, out_dtype, lse, ws, ws_bytes, stream, x_win, x_dtype, x_stride, gamma, eps);
}

int lca_hca_attn(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T, const int64_t* q_pos,
                 lca_kv comp, int32_t m, lca_kv win, int32_t n_win, const float* sink, float sm_scale,
                 double rope_theta, void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                 void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_hca_attn B=%d T=%d H=%d q_dtype=%d comp fmt=%d cap=%lld m=%d k=%d win cap=%lld n_win=%d out_dtype=%d "
                   "ws=%zu q_pos[0]=%lld", B, T, H, q_dtype, comp.fmt, (long long)comp.cap, m, 0, (long long)win.cap, n_win,
                   out_dtype, ws_bytes, pos0(q_pos));
    return attn_common(q, q_dtype, H, B, T, q_pos, comp, m, nullptr, 0, win, n_win, sink, sm_scale,
                       rope_theta, out, out_dtype, lse, ws, ws_bytes, stream);
}

// Scratch of lca_hca_attn_noalloc: one static array per GPU (each device that loads the library holds its own
// copy until the process ends).  In host code `scratch` names a host-side stand-in, not device memory: every
// use goes through the device address hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[LCA_NOALLOC_SCRATCH_BYTES];
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LCA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LCA_EINVAL, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(LCA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LCA_OK;
}
}  // namespace

int lca_hca_attn_noalloc(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T, const int64_t* q_pos,
                         lca_kv comp, int32_t m, lca_kv win, int32_t n_win, const float* sink, float sm_scale,
                         double rope_theta, void* out, int32_t out_dtype, float* lse, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_hca_attn_noalloc B=%d T=%d H=%d q_dtype=%d comp fmt=%d cap=%lld m=%d win cap=%lld n_win=%d "
                   "out_dtype=%d q_pos[0]=%lld", B, T, H, q_dtype, comp.fmt, (long long)comp.cap, m, (long long)win.cap,
                   n_win, out_dtype, pos0(q_pos));
    void* ws = nullptr;
    const int rc = scratch_for_current_device(&ws);
    if (rc) return rc;
    // (attn_common checks the launch's split partials against the array's size: LCA_EWORKSPACE beyond it)
    return attn_common(q, q_dtype, H, B, T, q_pos, comp, m, nullptr, 0, win, n_win, sink, sm_scale, rope_theta,
                       out, out_dtype, lse, ws, LCA_NOALLOC_SCRATCH_BYTES, stream);
}

// The MFMA GEMM kernels address the rows of one batch entry with 32-bit element offsets from its base:
// (rows - 1) * ld + K must stay below 2^32.
static bool gemm_offsets_fit(int64_t rows, int64_t ld, int64_t K) {
    return rows < 1 || (rows - 1) * ld + K <= (int64_t)UINT32_MAX;
}

int lca_linear(const void* x, int64_t ldx, int64_t sx, const void* w, int64_t ldw, int64_t sw, void* y,
               int32_t y_dtype, int64_t ldy, int64_t sy, int32_t M, int32_t N, int32_t K, int32_t batch,
               void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_linear M=%d N=%d K=%d batch=%d y_dtype=%d", M, N, K, batch, y_dtype);
    if (!x || !w || !y) return fail(LCA_EINVAL, "x, w and y must be non-NULL");
    if (y_dtype != LCA_F32 && y_dtype != LCA_BF16) return fail(LCA_EDTYPE, "y_dtype must be f32 or bf16");
    if (M < 0 || N < 1 || batch < 1) return fail(LCA_ESHAPE, "bad M / N / batch");
    if (K < 8 || K % 8) return fail(LCA_ESHAPE, "K must be a positive multiple of 8 (got %d)", K);
    if (ldx < K || ldw < K || ldy < N || sx < 0 || sw < 0 || sy < 0)
        return fail(LCA_ESHAPE, "row strides must cover the rows (ldx, ldw >= K, ldy >= N)");
    if (ldx % 8 || ldw % 8 || sx % 8 || sw % 8)
        return fail(LCA_EALIGN, "x and w strides must be multiples of 8 elements (16-byte rows)");
    if (!aligned16(x) || !aligned16(w) || ((uintptr_t)y & (y_dtype == LCA_F32 ? 3u : 1u)))
        return fail(LCA_EALIGN, "x and w must be 16-byte aligned, y aligned to its element");
    if (!gemm_offsets_fit(M, ldx, K) || !gemm_offsets_fit(N, ldw, K))
        return fail(LCA_ESHAPE, "one batch entry of x or w spans 2^32 elements or more");
    lca::GemmArgs a;
    memset(&a, 0, sizeof a);
    a.x = x; a.w = w; a.y = y; a.ldx = ldx; a.sx = sx; a.ldw = ldw; a.sw = sw; a.ldy = ldy; a.sy = sy;
    a.M = M; a.N = N; a.K = K; a.batch = batch; a.y_dtype = y_dtype;
    return hip_status(lca::launch_gemm(a, (hipStream_t)stream));
}

int lca_grouped_out_proj(const void* o, int32_t T, int32_t H, int32_t c, int32_t g, const void* wg, int32_t d_g,
                         const void* wo, int32_t d, void* mid, void* out, int32_t out_dtype, void* stream) {
    g_err[0] = 0;
    LCA_TRACE_CALL("lca_grouped_out_proj T=%d H=%d c=%d g=%d d_g=%d d=%d out_dtype=%d", T, H, c, g, d_g, d, out_dtype);
    if (!o || !wg || !wo || !mid || !out) return fail(LCA_EINVAL, "o, wg, wo, mid and out must be non-NULL");
    if (out_dtype != LCA_F32 && out_dtype != LCA_BF16) return fail(LCA_EDTYPE, "out_dtype must be f32 or bf16");
    if (T < 0 || H < 1 || c < 1 || g < 1 || H % g || d_g < 1 || d < 1)
        return fail(LCA_ESHAPE, "bad T / H / c / g / d_g / d (H must be a multiple of g)");
    const int64_t kg = (int64_t)(H / g) * c;
    if (kg % 8 || d_g % 8 || kg > INT32_MAX || (int64_t)g * d_g > INT32_MAX)
        return fail(LCA_ESHAPE, "(H / g) * c and d_g must be multiples of 8");
    if (!aligned16(o) || !aligned16(wg) || !aligned16(wo) || !aligned16(mid) || !aligned16(out))
        return fail(LCA_EALIGN, "pointers must be 16-byte aligned");
    if (!gemm_offsets_fit(T, (int64_t)H * c, kg) || !gemm_offsets_fit(d_g, kg, kg) ||
        !gemm_offsets_fit(T, (int64_t)g * d_g, (int64_t)g * d_g) || !gemm_offsets_fit(d, (int64_t)g * d_g, (int64_t)g * d_g))
        return fail(LCA_ESHAPE, "an operand spans 2^32 elements or more");
    if (T == 0) return LCA_OK;
    lca::GemmArgs a;
    memset(&a, 0, sizeof a);
    // the g group projections: one batch entry per group
    a.x = o; a.ldx = (int64_t)H * c; a.sx = kg;
    a.w = wg; a.ldw = kg; a.sw = (int64_t)d_g * kg;
    a.y = mid; a.y_dtype = LCA_BF16; a.ldy = (int64_t)g * d_g; a.sy = d_g;
    a.M = T; a.N = d_g; a.K = (int32_t)kg; a.batch = g;
    hipError_t e = lca::launch_gemm(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    // the dense projection of the concatenated intermediate
    a.x = mid; a.ldx = (int64_t)g * d_g; a.sx = 0;
    a.w = wo; a.ldw = (int64_t)g * d_g; a.sw = 0;
    a.y = out; a.y_dtype = out_dtype; a.ldy = d; a.sy = 0;
    a.M = T; a.N = d; a.K = g * d_g; a.batch = 1;
    return hip_status(lca::launch_gemm(a, (hipStream_t)stream));
}

}  // extern "C"
