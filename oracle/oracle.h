/*
 * oracle.h -- plain CPU oracle for the CSA / HCA compressed-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library and must never be used as a
 * fallback for it.
 *
 * Everything is computed in fp64 on host arrays, following the method as the
 * DeepSeek-V4 pages state it:
 *   [R]  "DeepSeek-V4 中文翻译" (cnblogs translation of the DeepSeek-V4 technical
 *        report), section 2.3 (2.3.1 CSA, 2.3.2 HCA, 2.3.3 other details,
 *        2.3.4 efficiency) and 5.2.1 (BF16 index scores);
 *   [H]  "DeepSeek-V4：百万 token 上下文，真正可供 Agent 使用" (translation of the
 *        Hugging Face blog post), section "混合注意力：CSA 与 HCA".
 * Where the pages leave a step open the plain reading is taken; each such
 * reading is named at the function that takes it.
 *
 * Storage formats (same meaning as the library's, defined independently):
 *   ORC_F32 : nope f32, rope f32
 *   ORC_BF16: nope bf16, rope bf16
 *   ORC_FP8 : nope OCP e4m3fn with one f32 power-of-two scale per 128 nope
 *             dims, rope bf16.
 *   ORC_MXFP4: nope OCP MXFP4 (E2M1 elements, two per byte with the even
 *             element in the low nibble, and one E8M0 scale byte per 32
 *             elements, stored through the `scale` pointer as uint8_t);
 *             no rope dims.  Used for the indexer keys ([R] 5.2.1: the QK
 *             path of the CSA indexer is cached, loaded and multiplied in
 *             FP4 (MXFP4)).
 * bf16 arrays are passed as uint16_t bit patterns.
 */
#ifndef LCA_ORACLE_H
#define LCA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_MXFP4 = 3 };

typedef struct {
    void*   nope;   /* [B][cap][d_nope]                                   */
    void*   rope;   /* [B][cap][d_rope]                                   */
    float*  scale;  /* [B][cap][d_nope/128] for ORC_FP8; uint8_t E8M0
                       [B][cap][d_nope/32] for ORC_MXFP4; else unused     */
    int32_t fmt;
    int32_t d_nope, d_rope;
    int64_t cap;    /* rows per sequence                                  */
} orc_kv;

/* scalar codecs */
double   orc_bf16_to_f64(uint16_t h);
uint16_t orc_f32_to_bf16(float x);            /* round to nearest even     */
double   orc_fp8_to_f64(uint8_t code);        /* OCP e4m3fn; NaN codes -> NaN */
uint8_t  orc_f64_to_fp8(double x);            /* nearest, ties to even code, saturating at +-448 */

double   orc_e2m1_to_f64(uint8_t code);       /* OCP FP4 E2M1 (low 4 bits)  */
uint8_t  orc_f64_to_e2m1(double x);           /* nearest, ties to even code, saturating at +-6 */
/* One MXFP4 block of 32 values: the E8M0 scale byte and 32 E2M1 codes. */
uint8_t  orc_mxfp4_block(const double* v, uint8_t* codes);

/* decode stored rows [row0, row0+nrows) of sequence b into out[nrows][d_nope+d_rope] */
void orc_kv_decode(orc_kv kv, int64_t b, int64_t row0, int64_t nrows, double* out);

/* Compressor (softmax-gated pooling, optional RMSNorm, partial RoPE, store).
 * Returns the number of entries written, or -1 on bad arguments. */
int64_t orc_kv_compress(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                        int32_t in_fmt, const float* bias_a, const float* bias_b,
                        const float* gamma, double eps, double rope_theta,
                        int32_t m, int32_t overlap, int32_t B, int64_t n_rows,
                        const int64_t* first_pos, orc_kv out, int32_t ring);

/* Lightning indexer scores S[b][t][s] for s < vis(t); other columns untouched. */
int orc_indexer_score(const void* q, int32_t q_fmt, const float* w, const void* k, int32_t k_fmt,
                      int64_t k_cap, int32_t H_I, int32_t d_I, int32_t B, int32_t T,
                      const int64_t* q_pos, int32_t m, void* scores, int32_t score_fmt,
                      int64_t s_stride);

/* The same scores with the QK path in MXFP4 ([R] 5.2.1): q (bf16 or f32) is
 * quantised per head and 32-element block, the keys are stored MXFP4 (k.fmt
 * == ORC_MXFP4, k.d_nope == d_I), and the products of the decoded values are
 * summed exactly (fp64). */
int orc_indexer_score_mxfp4(const void* q, int32_t q_fmt, const float* w, orc_kv k, int32_t H_I,
                            int32_t d_I, int32_t B, int32_t T, const int64_t* q_pos, int32_t m,
                            void* scores, int32_t score_fmt, int64_t s_stride);

/* Top-k selection by (score desc, index asc), emitted ascending, -1 padded. */
int orc_topk_select(const void* scores, int32_t score_fmt, int64_t s_stride, int32_t B, int32_t T,
                    const int64_t* q_pos, int32_t m, int32_t k, int32_t* idx);

/* Core attention.  idx != NULL: CSA (selected entries); idx == NULL: HCA
 * (every visible entry).  Plus the sliding window and the sink. */
int orc_attention(const void* q, int32_t q_fmt, int32_t H, int32_t B, int32_t T,
                  const int64_t* q_pos, orc_kv comp, int32_t m, const int32_t* idx, int32_t k,
                  orc_kv win, int32_t n_win, const float* sink, double sm_scale,
                  double rope_theta, void* out, int32_t out_fmt, float* lse);

/* Linear maps around the path ([R] 2.3.1: the compressor inputs C, Z and the queries are linear
 * projections of the hidden state; the grouped output projection):
 *   Y[b][m][n] = sum_k X[b][m][k] W[b][n][k]
 * X element (b, m, k) at x[b * sx + m * ldx + k], W at w[b * sw + n * ldw + k], Y at
 * y[b * sy + m * ldy + n]; formats ORC_F32 / ORC_BF16; exact products, fp64 sums, one rounding. */
int orc_linear(const void* x, int32_t x_fmt, int64_t ldx, int64_t sx, const void* w, int32_t w_fmt,
               int64_t ldw, int64_t sw, void* y, int32_t y_fmt, int64_t ldy, int64_t sy, int32_t M,
               int32_t N, int32_t K, int32_t batch);

/* Grouped output projection ([R] 2.3.1): the H head outputs of a token (o [T][H][c]) form g groups
 * of H/g heads; group j is projected to d_g dims by wg[j] ([g][d_g][H/g * c]), the g results are
 * stored in mid_fmt and concatenated ([T][g * d_g]), then projected to d dims by wo ([d][g * d_g]). */
int orc_grouped_out_proj(const void* o, int32_t o_fmt, int32_t T, int32_t H, int32_t c, int32_t g,
                         const void* wg, int32_t d_g, const void* wo, int32_t d, int32_t mid_fmt, void* out,
                         int32_t out_fmt);

#ifdef __cplusplus
}
#endif
#endif
