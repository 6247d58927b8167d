/*
 * lca.h -- C ABI of the MI355X (gfx950) compressed-attention library.
 *
 * The library implements the data-parallel hot path of the hybrid attention
 * described on the DeepSeek-V4 pages:
 *   [R] "DeepSeek-V4 中文翻译" (cnblogs translation of the technical report
 *       "DeepSeek-V4: Towards Highly Efficient Million-Token Context
 *       Intelligence"), section 2.3 and 5.2.1;
 *   [H] "DeepSeek-V4：百万 token 上下文，真正可供 Agent 使用" (translation of the
 *       Hugging Face blog post), section "混合注意力：CSA 与 HCA".
 * CSA = compressor (m = 4) -> lightning indexer -> top-k -> shared-KV MQA over
 * the selected entries plus a sliding window; HCA = compressor (m' = 128) ->
 * dense shared-KV MQA over every visible entry plus the window.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor argument is DEVICE memory owned by the caller, row-major and
 *   contiguous, 16-byte aligned.  The library never allocates, frees or
 *   synchronises; each call enqueues its kernels on `stream` (a hipStream_t
 *   passed as void*, NULL = the null stream) and returns at once.
 * - Position arrays (`first_pos`, `q_pos`, length B) are HOST memory, read
 *   during the call; B <= LCA_MAX_BATCH.
 * - All arguments are validated on the host before anything is launched: on
 *   error the call returns a nonzero status, enqueues nothing and leaves every
 *   output untouched; lca_last_error() then describes the problem.
 * - Raw position p of a sequence is the p-th token.  Compressed entry s of a
 *   stream with ratio m pools raw rows [s*m, s*m + m).  Entry s is visible to
 *   a query at position t iff its last row is not after t:
 *   vis(t) = floor((t + 1) / m) entries are visible.
 *
 * KV storage (lca_kv) -- [R] 2.3.4: FP8 storage for most dims, BF16 for the
 * RoPE dims; [R] 5.2.1: the indexer's QK path in FP4 (MXFP4).  Four formats,
 * as planes of one row per entry:
 *   LCA_F32 : nope f32 [B][cap][d_nope], rope f32 [B][cap][d_rope]
 *   LCA_BF16: nope bf16, rope bf16
 *   LCA_FP8 : nope OCP e4m3fn bytes [B][cap][d_nope] with one f32 power-of-two
 *             scale per 128 nope dims, scale [B][cap][d_nope/128]; rope bf16.
 *             Stored value = code * scale (exact in bf16).
 *   LCA_MXFP4: OCP MXFP4 (Microscaling Formats v1.0), indexer keys only:
 *             nope = bytes [B][cap][d_nope/2] holding two FP4 E2M1 codes each
 *             (element 2i in the low nibble of byte i), scale = uint8 E8M0
 *             bytes [B][cap][d_nope/32] (block exponent e stored as e + 127);
 *             d_rope = 0, d_nope % 32 == 0.  Stored value = E2M1(code) * 2^e.
 *             Rows are written by lca_kv_compress, read by
 *             lca_indexer_score_mxfp4; the attention calls reject them.
 * The attended vector of a row is nope ++ rope (c = d_nope + d_rope dims).
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCA_VERSION 1
#define LCA_MAX_BATCH 64

/* status codes */
#define LCA_OK 0
#define LCA_EINVAL 1      /* null pointer, bad flag or enum value          */
#define LCA_ESHAPE 2      /* inconsistent or unsupported sizes             */
#define LCA_EDTYPE 3      /* unsupported dtype / storage format            */
#define LCA_EALIGN 4      /* pointer not 16-byte aligned                   */
#define LCA_EWORKSPACE 5  /* workspace missing or too small                */
#define LCA_EHIP 6        /* the HIP runtime refused a launch              */
#define LCA_ENOMEM 7      /* the paged cache has no free page or slot      */

/* dtypes / storage formats */
#define LCA_F32 0
#define LCA_BF16 1
#define LCA_FP8 2         /* KV storage only (see above)                   */
#define LCA_MXFP4 3       /* indexer-key storage only (see above)          */

typedef struct lca_kv {
    void* nope;       /* [B][cap][d_nope]                                  */
    void* rope;       /* [B][cap][d_rope]; may be NULL when d_rope == 0    */
    void* scale;      /* f32 [B][cap][d_nope/128] for LCA_FP8, uint8
                         [B][cap][d_nope/32] for LCA_MXFP4, else NULL      */
    int32_t fmt;      /* LCA_F32 / LCA_BF16 / LCA_FP8 / LCA_MXFP4          */
    int32_t d_nope;
    int32_t d_rope;   /* even                                              */
    int64_t cap;      /* rows per sequence (batch stride = cap rows)       */
} lca_kv;

/*
 * lca_kv_compress -- the compressor of [R] 2.3.1 ("compressed KV entries")
 * and 2.3.2, [H] CSA/HCA: softmax-gated pooling with a learnable
 * per-position bias, then RMSNorm ([R] 2.3.3), partial RoPE ([R] 2.3.3) and
 * the store into `out`.
 *
 * Inputs c_a, z_a, c_b, z_b: B sequences of n_rows rows of c values, dtype
 * in_dtype (LCA_F32 or LCA_BF16), c = out.d_nope + out.d_rope; sequence b
 * starts in_stride rows after sequence b-1 (in_stride = 0 means n_rows, i.e.
 * [B][n_rows][c]); row i of sequence b is position first_pos[b] + i.  bias_a, bias_b: f32 [m][c] (NULL = zero).  For entry s
 * and channel j the logits are z_a[s*m+i][j] + bias_a[i][j] (i < m) and, when
 * overlap != 0 and s >= 1, z_b[(s-1)*m+i][j] + bias_b[i][j]; one softmax over
 * them weights the matching c_a / c_b values.  c_b, z_b may be NULL when
 * overlap == 0.  gamma: f32 [c] RMSNorm weight over all c dims with epsilon
 * eps, NULL = no norm.  rope_theta > 0: rotate dims [d_nope, c) (half-split
 * pairs (i, i + d_rope/2), inverse frequency theta^(-2i/d_rope)) by the
 * entry's first position s*m; 0 = no rotation.
 *
 * Entries written: exactly those s whose rows are all in range -- block s,
 * and block s-1 when overlap != 0 and s >= 1.  Entry s goes to row s of
 * sequence b in `out` (ring != 0: row s mod out.cap, and only the newest
 * out.cap entries of the call are written).  m = 1 with overlap = 0 is the
 * raw-row store used for the sliding window.
 * Errors: LCA_EINVAL (null inputs, m < 1, overlap not 0/1), LCA_EDTYPE,
 * LCA_ESHAPE (0 < in_stride < n_rows, ...),
 * LCA_ESHAPE (B out of range, c != d_nope + d_rope, fp8 with d_nope % 128,
 * a non-ring entry row >= cap), LCA_EALIGN.
 * MXFP4 output (the indexer keys): every 32 dims share the exponent
 * e = floor(log2 amax) - 2 of their largest magnitude (clamped to [-127, 127];
 * 0 for an all-zero block) and each value is stored as the E2M1 code nearest
 * to value * 2^-e (ties to the even code, saturating at 6).  Needs
 * out.d_rope == 0 and out.d_nope % 32 == 0 (else LCA_ESHAPE).
 */
int lca_kv_compress(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                    int32_t in_dtype, const float* bias_a, const float* bias_b,
                    const float* gamma, float eps, double rope_theta,
                    int32_t m, int32_t overlap, int32_t B, int64_t n_rows, int64_t in_stride,
                    const int64_t* first_pos, lca_kv out, int32_t ring, void* stream);

/*
 * lca_kv_compress_ws -- lca_kv_compress with a caller workspace (the same
 * entries, the same arithmetic up to the order in which the rows' softmax
 * states are merged).  With ws != NULL a call of few long entries -- bf16
 * inputs, c % 8 == 0, c <= 576, at least 64 rows per entry (m * (1 + overlap))
 * and at most 128 (entry, sequence) pairs, e.g. a 4096-token chunk's m = 128
 * blocks -- cuts each entry's rows into ranges pooled by separate workgroups
 * (at most 256 workgroups in all) and merges the ranges' per-channel states
 * in a fixed order; other calls ignore ws.  ws: device memory of at least
 * lca_compress_workspace_size(in_dtype, m, overlap, d_nope, d_rope) bytes,
 * 16-byte aligned, owned by the caller, no initialisation needed; calls on
 * one workspace must not overlap.  ws == NULL: exactly lca_kv_compress.
 * Errors: as lca_kv_compress; LCA_EWORKSPACE when ws is non-NULL but
 * ws_bytes is below the size the call needs; LCA_EALIGN for a misaligned ws.
 */
int lca_kv_compress_ws(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                       int32_t in_dtype, const float* bias_a, const float* bias_b,
                       const float* gamma, float eps, double rope_theta,
                       int32_t m, int32_t overlap, int32_t B, int64_t n_rows, int64_t in_stride,
                       const int64_t* first_pos, lca_kv out, int32_t ring, void* ws, size_t ws_bytes,
                       void* stream);
/* Workspace bytes for lca_kv_compress_ws over any number of rows and
 * sequences (256 x 3 x c floats), or 0 when such calls never split. */
size_t lca_compress_workspace_size(int32_t in_dtype, int32_t m, int32_t overlap, int32_t d_nope, int32_t d_rope);

/*
 * lca_indexer_score -- the lightning indexer of [R] 2.3.1 and [H] CSA: a
 * multi-head dot product scored by ReLU between each query and every
 * compressed indexer key, with BF16 scores as in [R] 5.2.1.
 *   S[b][i][s] = sum_h w[b][i][h] * max(0, q[b][i][h] . k[b][s])   for s < vis(t)
 * with t = q_pos[b] + i; columns s >= vis(t) are left unspecified (a call
 * with several rows per sequence may write scores there, for columns below
 * the visible count of the call's last row of that sequence).
 * q: [B][T][H_I][d_I], k: [B][k_cap][d_I] (one key per compressed entry,
 * shared by all indexer heads), both in_dtype (LCA_BF16, or LCA_F32);
 * w: f32 [B][T][H_I] (NULL = all ones).  scores: [B][T][s_stride] of
 * score_dtype (LCA_F32, or LCA_BF16 = nearest-even rounding of the f32
 * score, -0 stored as +0).  Arithmetic: products accumulated in f32.
 * Requires vis(q_pos[b] + T - 1) <= min(k_cap, s_stride); d_I % 32 == 0,
 * H_I <= 64.
 */
int lca_indexer_score(const void* q, const float* w, const void* k, int32_t in_dtype,
                      int64_t k_cap, int32_t H_I, int32_t d_I, int32_t B, int32_t T,
                      const int64_t* q_pos, int32_t m, void* scores, int32_t score_dtype,
                      int64_t s_stride, void* stream);

/*
 * lca_indexer_score_mxfp4 -- the same scores with the QK path in FP4
 * ([R] 5.2.1: the indexer's query and key activations are cached, loaded and
 * multiplied in MXFP4).  q: bf16 [B][T][H_I][d_I]; each head's 32-element
 * blocks are quantised to MXFP4 inside the call by the rule stated for
 * lca_kv_compress (bf16 in, so the codes are exact functions of the input).
 * k: MXFP4 key rows (k.fmt == LCA_MXFP4, k.d_nope == d_I, k.d_rope == 0,
 * k.cap rows per sequence), as written by lca_kv_compress.  The products of
 * the decoded values are accumulated in f32; w, scores, s_stride and the
 * visibility rule as for lca_indexer_score.  Supports H_I = 16, d_I = 128.
 * Errors: LCA_EINVAL (NULL pointers, m < 1), LCA_EDTYPE (k not MXFP4, score
 * dtype), LCA_ESHAPE (H_I / d_I, vis beyond k.cap or s_stride, B), LCA_EALIGN.
 */
int lca_indexer_score_mxfp4(const void* q, const float* w, lca_kv k, int32_t H_I, int32_t d_I, int32_t B,
                            int32_t T, const int64_t* q_pos, int32_t m, void* scores, int32_t score_dtype,
                            int64_t s_stride, void* stream);

/*
 * lca_topk_select -- the top-k selector of [R] 2.3.1 (keeps a subset of the
 * compressed entries for the core attention).  For row (b, i) with
 * t = q_pos[b] + i the candidates are s < vis(t); the K = min(k, vis(t))
 * entries with the largest scores are kept, ties broken by the lower index
 * (-0 equals +0); idx[b][i][0..K) lists them in ascending order and the rest
 * of the row is -1.  scores: [B][T][s_stride] (LCA_F32 or LCA_BF16, finite);
 * idx: int32 [B][T][k].  ws: device workspace of at least
 * lca_topk_workspace_size(B, T, s_stride, k) bytes (may be NULL when that
 * is 0; nonzero only for few long rows, where each row is split across
 * workgroups).  The workspace needs no initialisation.
 */
int lca_topk_select(const void* scores, int32_t score_dtype, int64_t s_stride, int32_t B,
                    int32_t T, const int64_t* q_pos, int32_t m, int32_t k, int32_t* idx,
                    void* ws, size_t ws_bytes, void* stream);
size_t lca_topk_workspace_size(int32_t B, int32_t T, int64_t s_stride, int32_t k);

/*
 * lca_indexer_topk -- lca_indexer_score followed by lca_topk_select, with the top-k's first pass
 * fused into the indexer.  [R] 2.3.1 (indexer, then top-k) and 5.2.1 (bf16 scores).  For each
 * sequence b the query rows are positions q_pos[b] .. q_pos[b] + T - 1: scores [B][T][s_stride]
 * bf16 get the scores of lca_indexer_score (q, w, k bf16 as there; H_I = 16, d_I = 128) and idx
 * [B][T][k] int32 the selection of lca_topk_select on those scores, bit for bit.  While it stores
 * the scores, the indexer also counts their high bytes (the top-k's first radix digit) with LDS and
 * device atomics: per row and 4096-key chunk when the rows are few and long (the top-k's split
 * schedule: its last two launches run), else per row (its row schedule: each row's workgroup skips
 * the first of its passes over the scores).
 * ws: device workspace of lca_indexer_topk_workspace_size(B, T, s_stride, k) bytes.  It must be
 * ZEROED BEFORE ITS FIRST USE and must not be shared with other calls (lca_topk_select writes the
 * same histograms without clearing them): every call leaves it ready for the next one, also inside
 * a captured graph -- the first-pass histograms, at the workspace's start, are zeroed again (per
 * row 128 words of 16-bit counts per 4096-key chunk in the split schedule, 256 words in the row
 * schedule); what follows them holds the top-k's own per-call figures, which need no
 * initialisation.  Errors as
 * lca_indexer_score and lca_topk_select; LCA_EWORKSPACE when ws is NULL or too small.
 */
int lca_indexer_topk(const void* q, const float* w, const void* k, int64_t k_cap, int32_t H_I, int32_t d_I,
                     int32_t B, int32_t T, const int64_t* q_pos, int32_t m, void* scores, int64_t s_stride,
                     int32_t topk, int32_t* idx, void* ws, size_t ws_bytes, void* stream);
size_t lca_indexer_topk_workspace_size(int32_t B, int32_t T, int64_t s_stride, int32_t k);

/*
 * lca_indexer_topk_mxfp4 -- the same fused call with the QK path in MXFP4 ([R] 5.2.1): the scores
 * of lca_indexer_score_mxfp4 (k: MXFP4 key rows, k.cap rows per sequence) and the selection of
 * lca_topk_select on them, with the same workspace (lca_indexer_topk_workspace_size) and rules.
 */
int lca_indexer_topk_mxfp4(const void* q, const float* w, lca_kv k, int32_t H_I, int32_t d_I, int32_t B,
                           int32_t T, const int64_t* q_pos, int32_t m, void* scores, int64_t s_stride, int32_t topk,
                           int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * lca_csa_attn -- CSA core attention, [R] 2.3.1 (shared-KV MQA: each stored
 * row is both key and value, one KV head for all H query heads) and 2.3.3
 * (sliding-window branch, attention sink, output RoPE).  For query row
 * (b, i), t = q_pos[b] + i, head h, the attended rows are
 *   comp rows e = idx[b][i][j] (j < k) with 0 <= e < vis(t) = min(floor((t + 1) / m),
 *   comp.cap)  and  window rows p in [max(0, t - n_win + 1), t], stored at win
 *   row p mod win.cap,
 * under one softmax with logits sm_scale * <q[b][i][h], row> and an optional
 * sink logit sink[h] that adds e^sink[h] to the denominator only:
 *   o = sum_j e^(l_j - mu) row_j / (e^(sink - mu) + sum_j e^(l_j - mu)).
 * rope_theta > 0: the last d_rope dims of o are rotated by -t (same pairing
 * as lca_kv_compress).  lse (f32 [B][T][H], NULL = skip) = mu + ln(den).
 * An empty set without a sink gives o = 0, lse = -inf.
 * q: [B][T][H][c] (LCA_BF16, or LCA_F32 with f32 caches); out: [B][T][H][c]
 * of out_dtype (LCA_F32 or LCA_BF16).  comp and win share d_nope / d_rope;
 * supported shapes: (d_nope, d_rope) = (512, 64) with 1 <= H <= 64 for
 * bf16/fp8 caches (the kernels take heads 16 at a time; a last partial
 * group computes on zero queries and stores nothing), any c <= 1024 for f32.  The window ring must hold every
 * needed row: min(n_win - 1, q_pos[b]) + T <= win.cap (n_win = 0: no window).  idx
 * values that are negative (padding) or not visible (e >= vis(t): a block
 * ending after t, or a row past the cache) are skipped, never read: block-level
 * causality holds whatever the list names.  ws: device workspace of at least
 * lca_attn_workspace_size(B, T, H, c, max keys per query) bytes.
 */
int lca_csa_attn(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T,
                 const int64_t* q_pos, lca_kv comp, int32_t m, const int32_t* idx, int32_t k,
                 lca_kv win, int32_t n_win, const float* sink, float sm_scale, double rope_theta,
                 void* out, int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * lca_hca_attn -- HCA core attention, [R] 2.3.2 and [H] HCA: as lca_csa_attn
 * but over EVERY visible compressed entry s < vis(t) (dense attention over the
 * heavily compressed stream) plus the same window.  Requires
 * vis(q_pos[b] + T - 1) <= comp.cap.
 */
int lca_hca_attn(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T,
                 const int64_t* q_pos, lca_kv comp, int32_t m, lca_kv win, int32_t n_win,
                 const float* sink, float sm_scale, double rope_theta, void* out,
                 int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * lca_hca_attn_noalloc -- lca_hca_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and results.  Its scratch (the split partials of decode-sized
 * launches, and the once-per-launch fp8 expansion of long ones when it fits)
 * is one static device array of LCA_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the library's load on that device until the process ends; the call never
 * allocates or frees.  A launch whose split partials need more than that
 * (lca_attn_workspace_size's split part, e.g. more rows x longer contexts
 * than one 1M-token decode row) fails with LCA_EWORKSPACE before anything
 * runs; a long launch whose expansion does not fit expands per tile as
 * lca_hca_attn does with a small workspace.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (two streams, two
 * threads) race and must be serialised by the caller.  The first call on a
 * device looks up the array's device address (hipGetSymbolAddress) with that
 * device current; errors as lca_hca_attn, plus LCA_EHIP if that lookup fails.
 */
#define LCA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int lca_hca_attn_noalloc(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T,
                         const int64_t* q_pos, lca_kv comp, int32_t m, lca_kv win, int32_t n_win,
                         const float* sink, float sm_scale, double rope_theta, void* out,
                         int32_t out_dtype, float* lse, void* stream);

/*
 * lca_csa_attn_append / lca_hca_attn_append -- the window store of the call's
 * own rows, then the attention: first rows q_pos[b] .. q_pos[b] + T - 1 of
 * x_win (x_dtype LCA_F32 or LCA_BF16; the raw rows of those positions: T
 * rows of c values per sequence, sequence b starting x_stride rows after
 * sequence b - 1, x_stride = 0 meaning T) are stored into the window ring win
 * exactly as
 * lca_kv_compress(x_win, ..., m = 1, overlap = 0, gamma, eps, rope_theta,
 * ring = 1, first_pos = q_pos) stores them ([R] 2.3.3 and 3.5.1: the
 * sliding-window rows live in the state cache), then the call is
 * lca_csa_attn / lca_hca_attn with the same arguments, so each query row
 * attends to its own freshly stored row.  Decode launches (T = 1, bf16
 * x_win, bf16 / fp8 caches of 512 + 64 dims, at most 64 rows x 16-head
 * groups) do the store inside the attention launch: one launch fewer per
 * layer and token.  Requires n_win >= 1; gamma: f32 [c] or NULL; x_win and
 * gamma 16-byte aligned.  Errors as lca_csa_attn / lca_hca_attn, plus
 * LCA_EINVAL (NULL x_win, n_win < 1, eps < 0), LCA_EDTYPE (x_dtype) and
 * LCA_ESHAPE (0 < x_stride < T).
 */
int lca_csa_attn_append(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T,
                        const int64_t* q_pos, lca_kv comp, int32_t m, const int32_t* idx, int32_t k,
                        lca_kv win, int32_t n_win, const void* x_win, int32_t x_dtype,
                        int64_t x_stride, const float* gamma, float eps, const float* sink,
                        float sm_scale, double rope_theta, void* out, int32_t out_dtype, float* lse,
                        void* ws, size_t ws_bytes, void* stream);
int lca_hca_attn_append(const void* q, int32_t q_dtype, int32_t H, int32_t B, int32_t T,
                        const int64_t* q_pos, lca_kv comp, int32_t m, lca_kv win, int32_t n_win,
                        const void* x_win, int32_t x_dtype, int64_t x_stride, const float* gamma,
                        float eps, const float* sink, float sm_scale, double rope_theta, void* out,
                        int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * lca_linear -- the linear maps around the attention ([R] 2.3.1: the
 * compressor inputs C_a, Z_a, C_b, Z_b, the low-rank queries and the indexer
 * queries are projections of the hidden state):
 *   y[b][m][n] = sum_k x[b][m][k] w[b][n][k]      (b < batch, m < M, n < N)
 * x and w bf16 (w holds one output per row, as a weight matrix), accumulated
 * in f32, y of y_dtype (LCA_F32, or LCA_BF16 = nearest-even rounding of the
 * f32 sum).  Element (b, m, k) of x is at x + b sx + m ldx + k, (b, n, k) of
 * w at w + b sw + n ldw + k, (b, m, n) of y at y + b sy + m ldy + n (strides
 * in elements).  Requires K a positive multiple of 8; ldx, ldw >= K and,
 * with sx and sw, multiples of 8; ldy >= N; x, w 16-byte aligned; one batch
 * entry of x and of w below 2^32 elements ((M - 1) ldx + K and (N - 1) ldw
 * + K), else LCA_ESHAPE (the MFMA kernels use 32-bit row offsets).  M <= 4
 * takes a kernel that streams w once (decode); larger M, MFMA tiles.
 */
int lca_linear(const void* x, int64_t ldx, int64_t sx, const void* w, int64_t ldw, int64_t sw, void* y,
               int32_t y_dtype, int64_t ldy, int64_t sy, int32_t M, int32_t N, int32_t K,
               int32_t batch, void* stream);

/*
 * lca_grouped_out_proj -- the grouped output projection of [R] 2.3.1: the H
 * head outputs of each of T tokens (o: bf16 [T][H][c]) form g groups of H/g
 * heads; group j is projected to d_g dims by wg[j] (bf16 [g][d_g][H/g * c]),
 * the g results are rounded to bf16 into mid (caller buffer, bf16 [T][g *
 * d_g]), and mid is projected to d dims by wo (bf16 [d][g * d_g]) into out
 * ([T][d], out_dtype LCA_F32 or LCA_BF16).  Two lca_linear launches.
 * Requires H % g == 0, (H / g) * c and d_g multiples of 8, 16-byte aligned
 * pointers, and each of o, wg, mid and wo below 2^32 elements as lca_linear
 * addresses them (else LCA_ESHAPE).
 */
int lca_grouped_out_proj(const void* o, int32_t T, int32_t H, int32_t c, int32_t g, const void* wg,
                         int32_t d_g, const void* wo, int32_t d, void* mid, void* out, int32_t out_dtype,
                         void* stream);

/* Workspace bytes for lca_csa_attn / lca_hca_attn with at most max_keys
 * attended rows per query (selected or visible entries + window).  Covers the
 * split partials of short (decode-sized) launches and, from 128 query rows on,
 * room for lca_hca_attn to expand an fp8 launch's rows to bf16 once instead of
 * per query row; with less workspace a long launch expands per tile (same
 * results).  No initialisation is needed. */
size_t lca_attn_workspace_size(int32_t B, int32_t T, int32_t H, int32_t c, int64_t max_keys);

/* Message for the last failed call on this thread ("" if none). */
const char* lca_last_error(void);
int lca_version(void);

#ifdef __cplusplus
}
#endif
#endif
