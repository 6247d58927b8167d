/*
 * oracle.c -- plain, slow, fp64 CPU oracle of the CSA / HCA path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  No blocking, fusion or
 * reordering beyond what the method states: every function is the
 * definition written out, one output element at a time.  OpenMP is used
 * only to run independent output rows side by side.
 *
 * Page references:
 *   [R] "DeepSeek-V4 中文翻译" (cnblogs translation of the technical report)
 *   [H] "DeepSeek-V4：百万 token 上下文，真正可供 Agent 使用" (translation of
 *       the Hugging Face blog post), section "混合注意力：CSA 与 HCA"
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* scalar codecs                                                              */
/* ------------------------------------------------------------------------- */

double orc_bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* bf16 keeps the top 16 bits of the fp32 pattern; the dropped half is
 * rounded to nearest, ties to the even kept pattern. */
uint16_t orc_f32_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    uint32_t upper = u >> 16, lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
    return (uint16_t)upper;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities; max 448. */
double orc_fp8_to_f64(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, mt = code & 7;
    double v;
    if (e == 15 && mt == 7) return NAN;
    if (e == 0) v = ldexp((double)mt / 8.0, -6);
    else v = ldexp(1.0 + (double)mt / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest representable magnitude among codes 0..126 (monotone in value),
 * found by bisection; exact ties go to the even code. */
uint8_t orc_f64_to_fp8(double x) {
    int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint8_t c;
    if (!(a == a)) return 0x7f;                 /* NaN */
    if (a >= 448.0) c = 126;                    /* saturate */
    else {
        int lo = 0, hi = 126;                   /* value(lo) <= a < value(hi) */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (orc_fp8_to_f64((uint8_t)mid) <= a) lo = mid; else hi = mid;
        }
        double dl = a - orc_fp8_to_f64((uint8_t)lo), dh = orc_fp8_to_f64((uint8_t)hi) - a;
        if (dl < dh) c = (uint8_t)lo;
        else if (dh < dl) c = (uint8_t)hi;
        else c = (uint8_t)((lo & 1) ? hi : lo);
    }
    return (uint8_t)(c | (neg << 7));
}

/* OCP FP4 E2M1 (OCP Microscaling Formats v1.0): 1 sign, 2 exponent (bias 1),
 * 1 mantissa bit; exponent 0 is subnormal (m/2); no NaN or infinity; max 6. */
double orc_e2m1_to_f64(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, mt = code & 1;
    double v = e == 0 ? 0.5 * mt : ldexp(1.0 + 0.5 * mt, e - 1);
    return s ? -v : v;
}

/* Nearest magnitude among codes 0..7 (monotone in value); exact ties go to the
 * even code; beyond 6 the result saturates. */
uint8_t orc_f64_to_e2m1(double x) {
    int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint8_t c = 7;
    if (a < 6.0) {
        int lo = 0;
        while (lo < 6 && orc_e2m1_to_f64((uint8_t)(lo + 1)) <= a) ++lo;   /* value(lo) <= a < value(lo+1) */
        double dl = a - orc_e2m1_to_f64((uint8_t)lo), dh = orc_e2m1_to_f64((uint8_t)(lo + 1)) - a;
        if (dl < dh) c = (uint8_t)lo;
        else if (dh < dl) c = (uint8_t)(lo + 1);
        else c = (uint8_t)((lo & 1) ? lo + 1 : lo);
    }
    return (uint8_t)(c | (neg << 3));
}

/* MX block conversion (OCP Microscaling Formats v1.0, conversion of a block of
 * 32 values to MXFP4): the shared scale is X = 2^(floor(log2(amax)) - 2), 2
 * being the largest exponent of E2M1, and each element is the E2M1 value
 * nearest to v / X (ties to even, saturating).  Reading: an all-zero block gets
 * scale 2^0 (E8M0 127) and zero codes; the E8M0 byte is clamped to [0, 254]. */
uint8_t orc_mxfp4_block(const double* v, uint8_t* codes) {
    double amax = 0.0;
    for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs(v[j]));
    int sh = 0;
    if (amax > 0.0) sh = ilogb(amax) - 2;
    if (sh < -127) sh = -127;
    if (sh > 127) sh = 127;
    for (int j = 0; j < 32; ++j) codes[j] = orc_f64_to_e2m1(ldexp(v[j], -sh));
    return (uint8_t)(sh + 127);
}

static double load_in(const void* p, int32_t fmt, int64_t i) {
    if (fmt == ORC_F32) return (double)((const float*)p)[i];
    return orc_bf16_to_f64(((const uint16_t*)p)[i]);
}

/* ------------------------------------------------------------------------- */
/* KV storage                                                                 */
/* ------------------------------------------------------------------------- */

void orc_kv_decode(orc_kv kv, int64_t b, int64_t row0, int64_t nrows, double* out) {
    int64_t c = kv.d_nope + kv.d_rope;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t row = b * kv.cap + row0 + r;
        double* o = out + r * c;
        for (int j = 0; j < kv.d_nope; ++j) {
            int64_t e = row * kv.d_nope + j;
            if (kv.fmt == ORC_MXFP4) {
                const uint8_t byte = ((const uint8_t*)kv.nope)[e / 2];
                const uint8_t sc = ((const uint8_t*)kv.scale)[row * (kv.d_nope / 32) + j / 32];
                o[j] = ldexp(orc_e2m1_to_f64((uint8_t)((j & 1) ? byte >> 4 : byte & 15)), (int)sc - 127);
                continue;
            }
            if (kv.fmt == ORC_F32) o[j] = ((const float*)kv.nope)[e];
            else if (kv.fmt == ORC_BF16) o[j] = orc_bf16_to_f64(((const uint16_t*)kv.nope)[e]);
            else o[j] = orc_fp8_to_f64(((const uint8_t*)kv.nope)[e]) *
                        (double)kv.scale[row * (kv.d_nope / 128) + j / 128];
        }
        for (int j = 0; j < kv.d_rope; ++j) {
            int64_t e = row * kv.d_rope + j;
            if (kv.fmt == ORC_F32) o[kv.d_nope + j] = ((const float*)kv.rope)[e];
            else o[kv.d_nope + j] = orc_bf16_to_f64(((const uint16_t*)kv.rope)[e]);
        }
    }
}

/* Store one row y[c] (fp64) into the planes.  f32: nearest fp32.  bf16:
 * nearest fp32, then nearest-even bf16.  fp8 (reading: the pages name only FP8
 * for the non-RoPE dims and BF16 for the RoPE dims, [R] 2.3.4): per group of 128
 * nope dims the scale is the power of two 2^ceil(log2(amax/448)) (1 for an
 * all-zero group) and each code is the nearest e4m3fn value of y/scale. */
static void store_row(orc_kv kv, int64_t row, const double* y) {
    for (int j = 0; j < kv.d_nope; ++j) {
        int64_t e = row * kv.d_nope + j;
        if (kv.fmt == ORC_F32) ((float*)kv.nope)[e] = (float)y[j];
        else if (kv.fmt == ORC_BF16) ((uint16_t*)kv.nope)[e] = orc_f32_to_bf16((float)y[j]);
    }
    if (kv.fmt == ORC_MXFP4) {
        uint8_t codes[32];
        for (int g = 0; g < kv.d_nope / 32; ++g) {
            ((uint8_t*)kv.scale)[row * (kv.d_nope / 32) + g] = orc_mxfp4_block(y + 32 * g, codes);
            for (int j = 0; j < 32; j += 2)
                ((uint8_t*)kv.nope)[(row * kv.d_nope + 32 * g + j) / 2] = (uint8_t)(codes[j] | (codes[j + 1] << 4));
        }
    }
    if (kv.fmt == ORC_FP8) {
        int ng = kv.d_nope / 128;
        for (int g = 0; g < ng; ++g) {
            double amax = 0.0;
            for (int j = g * 128; j < g * 128 + 128; ++j) amax = fmax(amax, fabs(y[j]));
            /* smallest power of two s with amax <= 448 s (exact comparisons) */
            double scale = 1.0;
            if (amax > 0.0) {
                scale = ldexp(1.0, ilogb(amax) - 10);
                while (amax > 448.0 * scale) scale *= 2.0;
            }
            kv.scale[row * ng + g] = (float)scale;
            for (int j = g * 128; j < g * 128 + 128; ++j)
                ((uint8_t*)kv.nope)[row * kv.d_nope + j] = orc_f64_to_fp8(y[j] / scale);
        }
    }
    for (int j = 0; j < kv.d_rope; ++j) {
        int64_t e = row * kv.d_rope + j;
        double v = y[kv.d_nope + j];
        if (kv.fmt == ORC_F32) ((float*)kv.rope)[e] = (float)v;
        else ((uint16_t*)kv.rope)[e] = orc_f32_to_bf16((float)v);
    }
}

/* RoPE on dims [d_nope, d_nope + d_rope) ([R] 2.3.3: RoPE on the last 64 dims of
 * queries and KV entries).  Reading: half-split pairs (i, i + d_rope/2) with
 * inverse frequency theta^(-2i/d_rope); angle = pos * inv_freq in fp64. */
static void rope_rotate(double* y, int d_nope, int d_rope, double theta, double pos) {
    int half = d_rope / 2;
    for (int i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)d_rope);
        double ang = pos * inv_freq;
        double cs = cos(ang), sn = sin(ang);
        double x0 = y[d_nope + i], x1 = y[d_nope + half + i];
        y[d_nope + i] = x0 * cs - x1 * sn;
        y[d_nope + half + i] = x0 * sn + x1 * cs;
    }
}

/* ------------------------------------------------------------------------- */
/* Compressor ([R] 2.3.1 "compressed KV entries", 2.3.2; [H] CSA / HCA)       */
/* ------------------------------------------------------------------------- */
/*
 * Entry s of a sequence pools the block of m raw rows [s*m, s*m+m).  For every
 * channel j the logits are Z_a[row][j] + B_a[i][j] over the block's rows
 * (i = position inside the block; the learnable positional bias), and, when
 * overlap is on and s >= 1, also Z_b[row][j] + B_b[i][j] over the previous
 * block's rows.  One softmax over all these logits weights the matching C_a /
 * C_b values; the weighted sum is the entry's channel j.
 * Readings: Z has C's shape (one gate per channel); the bias is indexed by the
 * position inside the block; CSA's second set (C_b, Z_b) covers the previous
 * block, since HCA is described as the variant without overlapping
 * compression.  After pooling: RMSNorm over all c dims ([R] 2.3.3), then RoPE
 * at the block's first position s*m, then the store.
 *
 * Entries are produced for exactly those s whose needed rows are all inside
 * the given range [first_pos, first_pos + n_rows): block s, and block s-1 too
 * when overlap is on and s >= 1.  Row s of the output (s mod cap if ring; a
 * ring call writes only the newest cap of those entries).
 */
int64_t orc_kv_compress(const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                        int32_t in_fmt, const float* bias_a, const float* bias_b,
                        const float* gamma, double eps, double rope_theta,
                        int32_t m, int32_t overlap, int32_t B, int64_t n_rows,
                        const int64_t* first_pos, orc_kv out, int32_t ring) {
    const int c = out.d_nope + out.d_rope;
    if (m < 1 || B < 1 || n_rows < 0 || !c_a || !z_a || (overlap && (!c_b || !z_b))) return -1;
    int64_t written = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t p0 = first_pos[b];
        int64_t s_lo = (p0 + m - 1) / m;
        if (overlap && s_lo > 0) s_lo += 1;
        const int64_t s_hi = (p0 + n_rows) / m;
        /* a ring keeps only the newest cap entries; older ones would be overwritten */
        if (ring && s_hi - s_lo > out.cap) s_lo = s_hi - out.cap;
        if (s_hi <= s_lo) continue;
        written += s_hi - s_lo;
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t s = s_lo; s < s_hi; ++s) {
            double* y = (double*)malloc(sizeof(double) * (size_t)c);
            double* lg = (double*)malloc(sizeof(double) * (size_t)(2 * m));
            double* cv = (double*)malloc(sizeof(double) * (size_t)(2 * m));
            const int use_b = overlap && s >= 1;
            for (int j = 0; j < c; ++j) {
                int nl = 0;
                for (int i = 0; i < m; ++i) {
                    int64_t r = b * n_rows + (s * m + i - p0);
                    lg[nl] = load_in(z_a, in_fmt, r * c + j) + (bias_a ? (double)bias_a[i * c + j] : 0.0);
                    cv[nl] = load_in(c_a, in_fmt, r * c + j);
                    ++nl;
                }
                if (use_b) {
                    for (int i = 0; i < m; ++i) {
                        int64_t r = b * n_rows + ((s - 1) * m + i - p0);
                        lg[nl] = load_in(z_b, in_fmt, r * c + j) + (bias_b ? (double)bias_b[i * c + j] : 0.0);
                        cv[nl] = load_in(c_b, in_fmt, r * c + j);
                        ++nl;
                    }
                }
                double mx = -INFINITY;
                for (int i = 0; i < nl; ++i) mx = fmax(mx, lg[i]);
                double den = 0.0, num = 0.0;
                for (int i = 0; i < nl; ++i) {
                    double e = exp(lg[i] - mx);
                    den += e;
                    num += e * cv[i];
                }
                y[j] = num / den;
            }
            if (gamma) {
                double ss = 0.0;
                for (int j = 0; j < c; ++j) ss += y[j] * y[j];
                double inv = 1.0 / sqrt(ss / (double)c + eps);
                for (int j = 0; j < c; ++j) y[j] = (double)gamma[j] * y[j] * inv;
            }
            if (rope_theta != 0.0 && out.d_rope > 0)
                rope_rotate(y, out.d_nope, out.d_rope, rope_theta, (double)(s * m));
            int64_t row = ring ? (s % out.cap) : s;
            store_row(out, b * out.cap + row, y);
            free(y);
            free(lg);
            free(cv);
        }
    }
    return written;
}

/* ------------------------------------------------------------------------- */
/* Visibility                                                                 */
/* ------------------------------------------------------------------------- */
/* Reading (the pages do not spell out block-level causality): entry s is
 * visible to query position t iff its last raw token, (s+1)*m - 1, is <= t,
 * so vis(t) = floor((t+1)/m) entries are visible. */
static int64_t vis_count(int64_t t, int32_t m) { return (t + 1) / m; }

/* ------------------------------------------------------------------------- */
/* Lightning indexer ([R] 2.3.1 "lightning indexer"; [H] CSA; [R] 5.2.1)      */
/* ------------------------------------------------------------------------- */
/*
 * S[t][s] = sum_h w[t][h] * ReLU(q_I[t][h] . k_I[s]): a multi-head dot product
 * scored by ReLU.  Readings: one indexer key per compressed entry shared by
 * all indexer heads; w = 1 when not given; no extra scale.  The score is
 * rounded to fp32 and, for bf16 scores ([R] 5.2.1: index scores quantised
 * from FP32 to BF16), to the nearest-even bf16; -0 is stored as +0.
 */
int orc_indexer_score(const void* q, int32_t q_fmt, const float* w, const void* k, int32_t k_fmt,
                      int64_t k_cap, int32_t H_I, int32_t d_I, int32_t B, int32_t T,
                      const int64_t* q_pos, int32_t m, void* scores, int32_t score_fmt,
                      int64_t s_stride) {
    if (!q || !k || !scores || H_I < 1 || d_I < 1 || B < 1 || T < 0 || m < 1) return -1;
    for (int32_t b = 0; b < B; ++b) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t i = 0; i < T; ++i) {
            const int64_t t = q_pos[b] + i;
            int64_t vis = vis_count(t, m);
            if (vis > k_cap) vis = k_cap;
            const int64_t qrow = ((int64_t)b * T + i) * H_I;
            for (int64_t s = 0; s < vis; ++s) {
                double acc = 0.0;
                for (int h = 0; h < H_I; ++h) {
                    double dot = 0.0;
                    for (int d = 0; d < d_I; ++d)
                        dot += load_in(q, q_fmt, (qrow + h) * d_I + d) *
                               load_in(k, k_fmt, ((int64_t)b * k_cap + s) * d_I + d);
                    double wh = w ? (double)w[qrow + h] : 1.0;
                    acc += wh * (dot > 0.0 ? dot : 0.0);
                }
                float f = (float)acc;
                if (f == 0.0f) f = 0.0f;
                int64_t e = ((int64_t)b * T + i) * s_stride + s;
                if (score_fmt == ORC_F32) ((float*)scores)[e] = f;
                else ((uint16_t*)scores)[e] = orc_f32_to_bf16(f);
            }
        }
    }
    return 0;
}

/*
 * The MXFP4 QK path ([R] 5.2.1: QK activations cached, loaded and multiplied
 * in FP4 (MXFP4)): every query head is quantised per 32-element block with
 * the rule of orc_mxfp4_block, the keys are read as stored, and the score is
 * the definition above on the decoded values (exact products, fp64 sums).
 */
int orc_indexer_score_mxfp4(const void* q, int32_t q_fmt, const float* w, orc_kv k, int32_t H_I,
                            int32_t d_I, int32_t B, int32_t T, const int64_t* q_pos, int32_t m,
                            void* scores, int32_t score_fmt, int64_t s_stride) {
    if (!q || !scores || k.fmt != ORC_MXFP4 || k.d_nope != d_I || k.d_rope != 0 || d_I % 32 || H_I < 1 ||
        B < 1 || T < 0 || m < 1)
        return -1;
    for (int32_t b = 0; b < B; ++b) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t i = 0; i < T; ++i) {
            const int64_t t = q_pos[b] + i;
            int64_t vis = vis_count(t, m);
            if (vis > k.cap) vis = k.cap;
            const int64_t qrow = ((int64_t)b * T + i) * H_I;
            double* qd = (double*)malloc(sizeof(double) * (size_t)H_I * d_I);
            double* kd = (double*)malloc(sizeof(double) * (size_t)d_I);
            for (int h = 0; h < H_I; ++h) {
                double blk[32];
                uint8_t codes[32];
                for (int g = 0; g < d_I / 32; ++g) {
                    for (int j = 0; j < 32; ++j) blk[j] = load_in(q, q_fmt, (qrow + h) * d_I + 32 * g + j);
                    const int sc = (int)orc_mxfp4_block(blk, codes) - 127;
                    for (int j = 0; j < 32; ++j) qd[h * d_I + 32 * g + j] = ldexp(orc_e2m1_to_f64(codes[j]), sc);
                }
            }
            for (int64_t s = 0; s < vis; ++s) {
                orc_kv_decode(k, b, s, 1, kd);
                double acc = 0.0;
                for (int h = 0; h < H_I; ++h) {
                    double dot = 0.0;
                    for (int d = 0; d < d_I; ++d) dot += qd[h * d_I + d] * kd[d];
                    double wh = w ? (double)w[qrow + h] : 1.0;
                    acc += wh * (dot > 0.0 ? dot : 0.0);
                }
                float f = (float)acc;
                if (f == 0.0f) f = 0.0f;
                int64_t e = ((int64_t)b * T + i) * s_stride + s;
                if (score_fmt == ORC_F32) ((float*)scores)[e] = f;
                else ((uint16_t*)scores)[e] = orc_f32_to_bf16(f);
            }
            free(qd);
            free(kd);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Top-k selector ([R] 2.3.1: a top-k selector keeps a subset for the core    */
/* attention)                                                                 */
/* ------------------------------------------------------------------------- */
/*
 * Reading: K = min(k, vis(t)) entries with the largest scores, ties broken
 * by the lower entry index; emitted in ascending index order and padded
 * with -1.  Implemented as a stable sort of the visible candidates.
 */
typedef struct { double v; int64_t s; } cand_t;

static int cand_cmp(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->s < b->s) ? -1 : (a->s > b->s);
}

static int idx_cmp(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

int orc_topk_select(const void* scores, int32_t score_fmt, int64_t s_stride, int32_t B, int32_t T,
                    const int64_t* q_pos, int32_t m, int32_t k, int32_t* idx) {
    if (!scores || !idx || k < 1 || B < 1 || T < 0 || m < 1) return -1;
    for (int32_t b = 0; b < B; ++b) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t i = 0; i < T; ++i) {
            const int64_t t = q_pos[b] + i;
            int64_t vis = vis_count(t, m);
            if (vis > s_stride) vis = s_stride;
            const int64_t rowoff = ((int64_t)b * T + i) * s_stride;
            cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * (size_t)(vis > 0 ? vis : 1));
            for (int64_t s = 0; s < vis; ++s) {
                cs[s].v = (score_fmt == ORC_F32) ? (double)((const float*)scores)[rowoff + s]
                                                 : orc_bf16_to_f64(((const uint16_t*)scores)[rowoff + s]);
                cs[s].s = s;
            }
            qsort(cs, (size_t)vis, sizeof(cand_t), cand_cmp);
            int64_t K = vis < k ? vis : k;
            int32_t* o = idx + ((int64_t)b * T + i) * k;
            for (int64_t j = 0; j < K; ++j) o[j] = (int32_t)cs[j].s;
            qsort(o, (size_t)K, sizeof(int32_t), idx_cmp);
            for (int64_t j = K; j < k; ++j) o[j] = -1;
            free(cs);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Core attention ([R] 2.3.1 shared-KV MQA, 2.3.2 HCA, 2.3.3 sliding window,  */
/* attention sink, output RoPE)                                               */
/* ------------------------------------------------------------------------- */
/*
 * For query position t and head h the attended set is the union of
 *   - compressed entries: CSA the entries listed in idx that are visible,
 *     0 <= s < vis(t) (block-level causality: an entry whose block ends after
 *     t is never attended, whatever the selection lists; negative ids are
 *     padding); HCA every visible entry s < vis(t) (dense attention over the
 *     compressed stream);
 *   - window rows: the n_win most recent raw positions ending at t itself,
 *     p in [max(0, t - n_win + 1), t], stored at ring row p mod win.cap.
 * Each stored vector is both key and value (shared-KV MQA: one KV head for all
 * query heads).  logit_j = sm_scale * <q[t][h], kv_j> over all c dims.  The sink
 * is one learnable logit z_h per head that joins the softmax denominator with
 * no value (so a head's weights may sum to less than 1):
 *   mu = max(max_j logit_j, z_h), den = e^(z_h-mu) + sum_j e^(logit_j-mu),
 *   o  = sum_j e^(logit_j-mu) kv_j / den,  lse = mu + ln(den).
 * Output RoPE ([R] 2.3.3: RoPE is also applied to the core-attention output to
 * carry relative position): reading, the last d_rope dims of o are rotated by
 * -t, which turns each entry's absolute rotation into a relative one.
 * An empty set without a sink gives o = 0 and lse = -inf.
 */
int orc_attention(const void* q, int32_t q_fmt, int32_t H, int32_t B, int32_t T,
                  const int64_t* q_pos, orc_kv comp, int32_t m, const int32_t* idx, int32_t k,
                  orc_kv win, int32_t n_win, const float* sink, double sm_scale,
                  double rope_theta, void* out, int32_t out_fmt, float* lse) {
    const int c = comp.d_nope + comp.d_rope;
    if (!q || !out || H < 1 || B < 1 || T < 0 || m < 1) return -1;
    if (n_win > 0 && (win.d_nope + win.d_rope != c)) return -1;
    for (int32_t b = 0; b < B; ++b) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t i = 0; i < T; ++i) {
            const int64_t t = q_pos[b] + i;
            /* gather the attended vectors */
            int64_t vis = vis_count(t, m);
            if (vis > comp.cap) vis = comp.cap;
            int64_t ncomp = 0;
            if (idx) {
                for (int j = 0; j < k; ++j) {
                    const int32_t s = idx[((int64_t)b * T + i) * k + j];
                    if (s >= 0 && s < vis) ++ncomp;
                }
            } else {
                ncomp = vis;
            }
            int64_t w_lo = t - n_win + 1;
            if (w_lo < 0) w_lo = 0;
            int64_t nwin = n_win > 0 ? t - w_lo + 1 : 0;
            int64_t nkv = ncomp + nwin;
            double* kv = (double*)malloc(sizeof(double) * (size_t)((nkv > 0 ? nkv : 1) * c));
            int64_t r = 0;
            if (idx) {
                for (int j = 0; j < k; ++j) {
                    int32_t s = idx[((int64_t)b * T + i) * k + j];
                    if (s >= 0 && s < vis) orc_kv_decode(comp, b, s, 1, kv + (r++) * c);
                }
            } else {
                for (int64_t s = 0; s < vis; ++s) orc_kv_decode(comp, b, s, 1, kv + (r++) * c);
            }
            for (int64_t p = w_lo; p <= t && n_win > 0; ++p)
                orc_kv_decode(win, b, p % win.cap, 1, kv + (r++) * c);

            double* lg = (double*)malloc(sizeof(double) * (size_t)(nkv > 0 ? nkv : 1));
            double* o = (double*)malloc(sizeof(double) * (size_t)c);
            double* qv = (double*)malloc(sizeof(double) * (size_t)c);
            for (int h = 0; h < H; ++h) {
                const int64_t qoff = (((int64_t)b * T + i) * H + h) * c;
                for (int d = 0; d < c; ++d) qv[d] = load_in(q, q_fmt, qoff + d);
                double mu = sink ? (double)sink[h] : -INFINITY;
                for (int64_t j = 0; j < nkv; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < c; ++d) dot += qv[d] * kv[j * c + d];
                    lg[j] = sm_scale * dot;
                    mu = fmax(mu, lg[j]);
                }
                double den = sink ? exp((double)sink[h] - mu) : 0.0;
                for (int d = 0; d < c; ++d) o[d] = 0.0;
                for (int64_t j = 0; j < nkv; ++j) {
                    double e = exp(lg[j] - mu);
                    den += e;
                    for (int d = 0; d < c; ++d) o[d] += e * kv[j * c + d];
                }
                double l;
                if (den > 0.0) {
                    for (int d = 0; d < c; ++d) o[d] /= den;
                    l = mu + log(den);
                } else {
                    l = -INFINITY;
                }
                if (rope_theta != 0.0 && comp.d_rope > 0)
                    rope_rotate(o, comp.d_nope, comp.d_rope, rope_theta, -(double)t);
                for (int d = 0; d < c; ++d) {
                    if (out_fmt == ORC_F32) ((float*)out)[qoff + d] = (float)o[d];
                    else ((uint16_t*)out)[qoff + d] = orc_f32_to_bf16((float)o[d]);
                }
                if (lse) lse[((int64_t)b * T + i) * H + h] = (float)l;
            }
            free(kv);
            free(lg);
            free(o);
            free(qv);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Linear maps ([R] 2.3.1: projections of the hidden state; grouped output   */
/* projection)                                                               */
/* ------------------------------------------------------------------------- */

int orc_linear(const void* x, int32_t x_fmt, int64_t ldx, int64_t sx, const void* w, int32_t w_fmt,
               int64_t ldw, int64_t sw, void* y, int32_t y_fmt, int64_t ldy, int64_t sy, int32_t M,
               int32_t N, int32_t K, int32_t batch) {
    if (!x || !w || !y || M < 0 || N < 0 || K < 0 || batch < 1) return -1;
    for (int32_t b = 0; b < batch; ++b) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int32_t m = 0; m < M; ++m) {
            double* xr = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
            for (int32_t k = 0; k < K; ++k) xr[k] = load_in(x, x_fmt, b * sx + m * ldx + k);
            for (int32_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int32_t k = 0; k < K; ++k) acc += xr[k] * load_in(w, w_fmt, b * sw + n * ldw + k);
                const int64_t e = b * sy + m * ldy + n;
                if (y_fmt == ORC_F32) ((float*)y)[e] = (float)acc;
                else ((uint16_t*)y)[e] = orc_f32_to_bf16((float)acc);
            }
            free(xr);
        }
    }
    return 0;
}

int orc_grouped_out_proj(const void* o, int32_t o_fmt, int32_t T, int32_t H, int32_t c, int32_t g,
                         const void* wg, int32_t d_g, const void* wo, int32_t d, int32_t mid_fmt, void* out,
                         int32_t out_fmt) {
    if (g < 1 || H % g || T < 0 || d_g < 1 || d < 1) return -1;
    const int32_t kg = H / g * c;  /* inputs of one group */
    void* mid = malloc((mid_fmt == ORC_F32 ? 4 : 2) * (size_t)(T > 0 ? T : 1) * g * d_g);
    if (!mid) return -1;
    /* group j: rows t, inputs o[t][j * kg ..], weights wg[j] -> mid[t][j * d_g ..] */
    int rc = orc_linear(o, o_fmt, (int64_t)H * c, kg, wg, ORC_BF16, kg, (int64_t)d_g * kg, mid, mid_fmt,
                        (int64_t)g * d_g, d_g, T, d_g, kg, g);
    if (rc == 0)
        rc = orc_linear(mid, mid_fmt, (int64_t)g * d_g, 0, wo, ORC_BF16, (int64_t)g * d_g, 0, out, out_fmt, d, 0, T,
                        d, g * d_g, 1);
    free(mid);
    return rc;
}
