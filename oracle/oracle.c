/*
 * DSA oracle: a plain, slow CPU implementation of the DeepSeek Sparse Attention hot path
 * (lightning indexer -> top-k selection -> sparse MQA over the MLA latent cache).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header or table with the
 * HIP library; the two meet only through the byte-exact inputs produced by the seeded
 * input generator.
 *
 * Everything is computed in double precision with straightforward loops.  OpenMP is used
 * only to spread independent query rows over host cores.
 *
 * Sources (page titles as printed on the pages):
 *  - "DeepSeek-V3.2-Exp" overview, section "架构 & 背后实现" and module table (indexer
 *    score with ReLU, H_I indexer heads, one key per earlier token; top-k selection of
 *    key-value entries; core attention in MQA mode over the selected latent entries).
 *  - "DeepSeek-V3.2-Exp解析" section 一.1 (64 indexer heads of dim 128, FP8, top-k = 2048)
 *    and 一.2 (ReLU replaces softmax in the indexer).
 *  - Lightning-indexer walk-through, steps 2-4 (FP8 codes with cached key scales; per-head
 *    dot product, ReLU, weighted head sum; top-k positions).
 *  - "DeepSeek-V3.2 explained", sections 二.1-二.4 (DSA = attention over the top-k index
 *    set; 576-wide latent row = 512 latent + 64 rope; selected entries shared by all heads).
 *  - Lightning-indexer walk-through, step 2 (rotary encoding of the indexer query and key,
 *    FP8 quantisation of both, key codes and scale cached): the cache producer, in float32.
 *  - "DeepSeek-V3.2-Exp" overview, "训练"; "DeepSeek-V3.2-Exp解析" section 二; deep dive
 *    section 3 (indexer trained towards the head-summed, L1-normalised main attention with a
 *    KL divergence): the indexer training target, forward only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------ */
/* Codecs                                                                               */
/* ------------------------------------------------------------------------------------ */

/* OCP FP8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
 * the single NaN pattern S.1111.111, subnormals M * 2^-9, largest finite 448. */
double orc_e4m3(uint8_t b) {
    int s = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* The same value scaled by 2^9: always an integer, so products of two codes are exact
 * integers in units of 2^-18. */
int64_t orc_e4m3_fixed(uint8_t b) {
    int s = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    int64_t v = (e == 0) ? (int64_t)m : ((int64_t)(8 + m) << (e - 1));
    return s ? -v : v;
}

/* bf16 is the upper half of an IEEE binary32. */
double orc_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void orc_decode_e4m3(int64_t n, const uint8_t* in, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3(in[i]);
}

void orc_decode_bf16(int64_t n, const uint16_t* in, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16(in[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Lightning indexer                                                                    */
/* ------------------------------------------------------------------------------------ */

/* Dot product of two FP8 code vectors of length d, as a double (exact: every product is a
 * multiple of 2^-18 below 448^2, and the sum of at most 2^10 of them stays far below 2^53
 * units). */
double orc_dot_e4m3(int d, const uint8_t* a, const uint8_t* b) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += orc_e4m3(a[i]) * orc_e4m3(b[i]);
    return acc;
}

/* The same dot product in int64 fixed point, units of 2^-18. */
int64_t orc_dot_e4m3_fixed(int d, const uint8_t* a, const uint8_t* b) {
    int64_t acc = 0;
    for (int i = 0; i < d; ++i) acc += orc_e4m3_fixed(a[i]) * orc_e4m3_fixed(b[i]);
    return acc;
}

/* Index score of one (query row, key row) pair:
 *   I = sum_{j < H} w[j] * ReLU( qs[j] * ks * D_j ),  D_j = q8[j, :] . k8[:]
 * q8: [H][d] codes of the query row, qs: [H] query scales, w: [H] head weights,
 * k8: [d] codes of the key row, ks: the key scale.  Summed over j = 0..H-1 in order. */
double orc_index_score(int H, int d, const uint8_t* q8, const float* qs, const float* w,
                       const uint8_t* k8, float ks) {
    double total = 0.0;
    for (int j = 0; j < H; ++j) {
        double dj = orc_dot_e4m3(d, q8 + (int64_t)j * d, k8);
        double logit = (double)qs[j] * (double)ks * dj;
        double relu = logit > 0.0 ? logit : 0.0;
        total += (double)w[j] * relu;
    }
    return total;
}

/* Index scores for a list of query rows of one sequence.
 * q8: [T][H][d], qs: [T][H], w: [T][H]  (rows of the query side)
 * k8: [S][d], ks: [S]                   (key cache of the same sequence, position = row)
 * rows[i]: which query row; pos[i]: its absolute position p (keys 0..p are scored).
 * out: row i at out + i*out_stride, entries 0..pos[i] written, the rest untouched.
 * The codes are decoded to double once up front; the per-pair arithmetic is exactly that of
 * orc_index_score (same products, same head order), so the results are bit-identical. */
void orc_indexer_rows(int H, int d, const uint8_t* q8, const float* qs, const float* w,
                      const uint8_t* k8, const float* ks, int nrows, const int32_t* rows,
                      const int32_t* pos, double* out, int64_t out_stride) {
    int64_t smax = 0;
    for (int i = 0; i < nrows; ++i)
        if ((int64_t)pos[i] + 1 > smax) smax = (int64_t)pos[i] + 1;
    double* kd = (double*)malloc(sizeof(double) * (size_t)(smax > 0 ? smax : 1) * (size_t)d);
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < smax; ++s)
        for (int i = 0; i < d; ++i) kd[s * d + i] = orc_e4m3(k8[s * d + i]);
#pragma omp parallel
    {
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < nrows; ++i) {
            int64_t t = rows[i];
            for (int64_t x = 0; x < (int64_t)H * d; ++x) qd[x] = orc_e4m3(q8[t * H * d + x]);
            for (int64_t s = 0; s <= pos[i]; ++s) {
                const double* kr = kd + s * d;
                double total = 0.0;
                for (int j = 0; j < H; ++j) {
                    const double* qr = qd + (int64_t)j * d;
                    double dj = 0.0;
                    for (int x = 0; x < d; ++x) dj += qr[x] * kr[x];
                    double logit = (double)qs[t * H + j] * (double)ks[s] * dj;
                    double relu = logit > 0.0 ? logit : 0.0;
                    total += (double)w[t * H + j] * relu;
                }
                out[i * out_stride + s] = total;
            }
        }
        free(qd);
    }
    free(kd);
}

/* ------------------------------------------------------------------------------------ */
/* Top-k selection                                                                      */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    double v;
    int32_t pos;
} orc_cand;

/* Ranking rule: larger score first; -0 equals +0; NaN ranks below every number (including
 * -inf); equal scores rank the lower position first. */
static int orc_cand_cmp(const void* pa, const void* pb) {
    const orc_cand* a = (const orc_cand*)pa;
    const orc_cand* b = (const orc_cand*)pb;
    int an = isnan(a->v), bn = isnan(b->v);
    if (an != bn) return an ? 1 : -1;
    if (!an) {
        if (a->v > b->v) return -1;
        if (a->v < b->v) return 1;
    }
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos) ? 1 : 0;
}

static int orc_int_cmp(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a < b) ? -1 : (a > b);
}

/* Select the k best of the n scores x[0..n-1] under the ranking rule, write their positions
 * in ascending order to out[0..min(k,n)-1] and -1 to the remaining slots up to k. */
static void orc_topk_row(int64_t n, const double* x, int k, int32_t* out, orc_cand* buf) {
    for (int64_t s = 0; s < n; ++s) {
        buf[s].v = x[s];
        buf[s].pos = (int32_t)s;
    }
    qsort(buf, (size_t)n, sizeof(orc_cand), orc_cand_cmp);
    int64_t m = n < k ? n : k;
    for (int64_t i = 0; i < m; ++i) out[i] = buf[i].pos;
    qsort(out, (size_t)m, sizeof(int32_t), orc_int_cmp);
    for (int64_t i = m; i < k; ++i) out[i] = -1;
}

/* Rows of double scores: row i has n[i] valid entries at x + i*stride. */
void orc_topk_rows_f64(int nrows, const int64_t* n, const double* x, int64_t stride, int k,
                       int32_t* out) {
#pragma omp parallel
    {
        int64_t nmax = 1;
        for (int i = 0; i < nrows; ++i)
            if (n[i] > nmax) nmax = n[i];
        orc_cand* buf = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)nmax);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < nrows; ++i)
            orc_topk_row(n[i], x + (int64_t)i * stride, k, out + (int64_t)i * k, buf);
        free(buf);
    }
}

/* Rows of float scores (the exact arrays a GPU kernel saw), widened to double exactly. */
void orc_topk_rows_f32(int nrows, const int64_t* n, const float* x, int64_t stride, int k,
                       int32_t* out) {
#pragma omp parallel
    {
        int64_t nmax = 1;
        for (int i = 0; i < nrows; ++i)
            if (n[i] > nmax) nmax = n[i];
        orc_cand* buf = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)nmax);
        double* row = (double*)malloc(sizeof(double) * (size_t)nmax);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < nrows; ++i) {
            const float* xr = x + (int64_t)i * stride;
            for (int64_t s = 0; s < n[i]; ++s) row[s] = (double)xr[s];
            orc_topk_row(n[i], row, k, out + (int64_t)i * k, buf);
        }
        free(row);
        free(buf);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Sparse MQA over the latent cache                                                     */
/* ------------------------------------------------------------------------------------ */

/* For every query row t and head h, attention over the selected latent rows:
 *   z_s = sm * <q[t,h,:Dqk], c[s,:Dqk]>   for s in idx[t] (slots holding -1 are empty)
 *   o[t,h,:] = sum_s softmax(z)_s * c[s,:Dv],   lse[t,h] = log sum_s exp(z_s)
 * q: [T][H][Dqk] bf16 bits, kv: [S][Dqk] bf16 bits, idx: [T][k].
 * A row with no valid slot gets o = 0 and lse = -inf. */
void orc_sparse_mqa(int H, int Dqk, int Dv, double sm, int T, const uint16_t* q,
                    const uint16_t* kv, int k, const int32_t* idx, double* out, double* lse) {
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        double* qd = (double*)malloc(sizeof(double) * (size_t)Dqk);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < T; ++t) {
            const int32_t* sel = idx + (int64_t)t * k;
            for (int h = 0; h < H; ++h) {
                const uint16_t* qrow = q + ((int64_t)t * H + h) * Dqk;
                double* o = out + ((int64_t)t * H + h) * Dv;
                for (int d = 0; d < Dqk; ++d) qd[d] = orc_bf16(qrow[d]);
                double m = -INFINITY;
                for (int i = 0; i < k; ++i) {
                    z[i] = -INFINITY;
                    if (sel[i] < 0) continue;
                    const uint16_t* crow = kv + (int64_t)sel[i] * Dqk;
                    double acc = 0.0;
                    for (int d = 0; d < Dqk; ++d) acc += qd[d] * orc_bf16(crow[d]);
                    z[i] = sm * acc;
                    if (z[i] > m) m = z[i];
                }
                for (int v = 0; v < Dv; ++v) o[v] = 0.0;
                if (m == -INFINITY) {
                    lse[(int64_t)t * H + h] = -INFINITY;
                    continue;
                }
                double denom = 0.0;
                for (int i = 0; i < k; ++i) {
                    if (sel[i] < 0) continue;
                    double e = exp(z[i] - m);
                    denom += e;
                    const uint16_t* crow = kv + (int64_t)sel[i] * Dqk;
                    for (int v = 0; v < Dv; ++v) o[v] += e * orc_bf16(crow[v]);
                }
                for (int v = 0; v < Dv; ++v) o[v] /= denom;
                lse[(int64_t)t * H + h] = m + log(denom);
            }
        }
        free(qd);
        free(z);
    }
}

/* Dense causal attention in MQA mode, written independently of orc_sparse_mqa as the
 * textbook two-pass softmax: for query row t at position pos[t], every key s in [0, pos[t]]
 * takes part.  Used to pin the sparse path (the two agree whenever k >= pos + 1). */
void orc_dense_causal(int H, int Dqk, int Dv, double sm, int T, const int32_t* pos,
                      const uint16_t* q, const uint16_t* kv, double* out, double* lse) {
#pragma omp parallel
    {
        int64_t smax = 1;
        for (int t = 0; t < T; ++t)
            if (pos[t] + 1 > smax) smax = pos[t] + 1;
        double* p = (double*)malloc(sizeof(double) * (size_t)smax);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < T; ++t) {
            int64_t n = (int64_t)pos[t] + 1;
            for (int h = 0; h < H; ++h) {
                const uint16_t* qrow = q + ((int64_t)t * H + h) * Dqk;
                /* pass 1: logits and their maximum */
                double mx = -INFINITY;
                for (int64_t s = 0; s < n; ++s) {
                    double acc = 0.0;
                    for (int d = 0; d < Dqk; ++d)
                        acc += orc_bf16(qrow[d]) * orc_bf16(kv[s * Dqk + d]);
                    p[s] = acc * sm;
                    mx = p[s] > mx ? p[s] : mx;
                }
                /* pass 2: probabilities */
                double sum = 0.0;
                for (int64_t s = 0; s < n; ++s) {
                    p[s] = exp(p[s] - mx);
                    sum += p[s];
                }
                for (int64_t s = 0; s < n; ++s) p[s] /= sum;
                /* weighted sum of values */
                double* o = out + ((int64_t)t * H + h) * Dv;
                for (int v = 0; v < Dv; ++v) {
                    double acc = 0.0;
                    for (int64_t s = 0; s < n; ++s) acc += p[s] * orc_bf16(kv[s * Dqk + v]);
                    o[v] = acc;
                }
                lse[(int64_t)t * H + h] = mx + log(sum);
            }
        }
        free(p);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Cache producer: RoPE, FP8 encoding, per-row quantiser                                */
/* ------------------------------------------------------------------------------------ */

/* Lightning-indexer walk-through, step 2: the indexer query and key get a rotary encoding
 * of their first dims, are quantised to FP8 and the key codes are cached with their scale.
 * Everything here runs in float32 with each product, sum and quotient rounded on its own
 * (this file is built with -ffp-contract=off), the precision in which the GPU path decides
 * each FP8 code, so that both sides take the same rounding decisions. */

/* Nearest e4m3fn code of x: a search over the 127 non-negative finite codes for the value
 * closest to |x| (|x| above 448 saturates to 448: the format has no infinity); of two equally
 * close neighbours the one with an even code (mantissa bit 0 clear) wins.  The sign bit is
 * copied from x, so -0 and negative values that round to zero give 0x80.  NaN gives 0x7f. */
uint8_t orc_encode_e4m3(float x) {
    if (isnan(x)) return 0x7F;
    double a = fabs((double)x);
    if (a > 448.0) a = 448.0;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(signbit(x) ? (best | 0x80) : best);
}

void orc_encode_e4m3_n(int64_t n, const float* x, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode_e4m3(x[i]);
}

/* Rotary encoding of rows x[r, 0..d-1] (float32) at position pos: the pairs (2i, 2i+1) with
 * 2i < rope_dim rotate by the angle whose cosine and sine are cos_tab / sin_tab[pos *
 * tab_stride + i]:
 *     r0 = x0*c - x1*s,   r1 = x0*s + x1*c     (each product and difference rounded to fp32);
 * the dims from rope_dim on are copied unchanged. */
void orc_rope_f32(int n_rows, int d, const float* x, int64_t pos, const float* cos_tab,
                  const float* sin_tab, int64_t tab_stride, int rope_dim, float* out) {
    const float* c = cos_tab + pos * tab_stride;
    const float* s = sin_tab + pos * tab_stride;
    for (int r = 0; r < n_rows; ++r) {
        const float* xr = x + (int64_t)r * d;
        float* o = out + (int64_t)r * d;
        for (int i = 0; i < d; ++i) o[i] = xr[i];
        for (int i = 0; 2 * i + 1 < rope_dim; ++i) {
            float x0 = xr[2 * i], x1 = xr[2 * i + 1];
            float a = x0 * c[i], b = x1 * s[i];
            float e = x0 * s[i], f = x1 * c[i];
            o[2 * i] = a - b;
            o[2 * i + 1] = e + f;
        }
    }
}

/* One scale per row of x[r, 0..d-1] (float32): amax/448 (1 for an all-zero row), then the
 * codes of x / scale, clamped to +-448. */
void orc_quantize_rows_e4m3(int n_rows, int d, const float* x, uint8_t* codes, float* scale) {
    for (int r = 0; r < n_rows; ++r) {
        const float* xr = x + (int64_t)r * d;
        float amax = 0.0f;
        for (int i = 0; i < d; ++i) {
            float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        scale[r] = sc;
        for (int i = 0; i < d; ++i) {
            float y = xr[i] / sc;
            if (y > 448.0f) y = 448.0f;
            if (y < -448.0f) y = -448.0f;
            codes[(int64_t)r * d + i] = orc_encode_e4m3(y);
        }
    }
}

/* The cache producer for n new tokens at positions pos[i]: RoPE on the indexer query
 * q_idx[i] ([H][d]) and key k_idx[i] ([d]) over the first rope_dim dims, then one scale and
 * code row per query head and for the key.  Outputs q8 [n][H][d], q_scale [n][H],
 * k8 [n][d], k_scale [n]. */
void orc_cache_append(int n, int H, int d, const float* q_idx, const float* k_idx, const int64_t* pos,
                      const float* cos_tab, const float* sin_tab, int64_t tab_stride, int rope_dim,
                      uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale) {
#pragma omp parallel
    {
        float* rot = (float*)malloc(sizeof(float) * (size_t)H * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            orc_rope_f32(H, d, q_idx + (int64_t)i * H * d, pos[i], cos_tab, sin_tab, tab_stride, rope_dim, rot);
            orc_quantize_rows_e4m3(H, d, rot, q8 + (int64_t)i * H * d, q_scale + (int64_t)i * H);
            orc_rope_f32(1, d, k_idx + (int64_t)i * d, pos[i], cos_tab, sin_tab, tab_stride, rope_dim, rot);
            orc_quantize_rows_e4m3(1, d, rot, k8 + (int64_t)i * d, k_scale + i);
        }
        free(rot);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Indexer training target (forward only)                                               */
/* ------------------------------------------------------------------------------------ */

/* DeepSeek-V3.2-Exp overview, "训练"; 解析 section 二; deep dive section 3: the indexer is
 * trained towards the main attention summed over heads and L1-normalised along the keys,
 * with a KL divergence; in the sparse stage both sides are restricted to the selected set.
 * For query row t over its slots (entries of slots[t*k ..] that are not -1):
 *     P[s] = sum_h exp(sm * q[t,h,:] . kv[s,:] - lse[t,h]),   P /= sum_s P[s]
 *     Q    = softmax over the slots of the indexer scores I[t,s] = scores[t*score_stride + s]
 *     kl[t] = sum_{P>0} P (ln P - ln Q),   rev[t] = sum Q (ln Q - ln P)  (+inf if some P = 0)
 * A row without slots gets 0 and 0.  q: [T][H][Dqk] bf16 bits, kv: rows of the sequence. */
void orc_indexer_kl(int H, int Dqk, double sm, int T, const uint16_t* q, const uint16_t* kv,
                    const double* lse, int k, const int32_t* slots, const double* scores,
                    int64_t score_stride, double* kl, double* rev) {
#pragma omp parallel
    {
        double* P = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        double* lq = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)Dqk);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < T; ++t) {
            const int32_t* sel = slots + (int64_t)t * k;
            const double* I = scores + (int64_t)t * score_stride;
            kl[t] = 0.0;
            rev[t] = 0.0;
            for (int x = 0; x < H * Dqk; ++x) qd[x] = orc_bf16(q[(int64_t)t * H * Dqk + x]);
            int n = 0;
            double psum = 0.0, imax = -INFINITY;
            for (int i = 0; i < k; ++i) {
                if (sel[i] < 0) continue;
                const uint16_t* crow = kv + (int64_t)sel[i] * Dqk;
                double p = 0.0;
                for (int h = 0; h < H; ++h) {
                    double z = 0.0;
                    for (int dd = 0; dd < Dqk; ++dd) z += qd[(int64_t)h * Dqk + dd] * orc_bf16(crow[dd]);
                    p += exp(sm * z - lse[(int64_t)t * H + h]);
                }
                P[n] = p;
                lq[n] = I[sel[i]];
                psum += p;
                if (lq[n] > imax) imax = lq[n];
                ++n;
            }
            if (n == 0) continue;
            double esum = 0.0;
            for (int i = 0; i < n; ++i) esum += exp(lq[i] - imax);
            const double lse_i = imax + log(esum);
            double a = 0.0, b = 0.0;
            for (int i = 0; i < n; ++i) {
                const double p = P[i] / psum;
                const double lQ = lq[i] - lse_i;
                const double lP = log(p);  /* -inf for p = 0 */
                if (p > 0.0) a += p * (lP - lQ);
                b += exp(lQ) * (lQ - lP);
            }
            kl[t] = a;
            rev[t] = b;
        }
        free(qd);
        free(lq);
        free(P);
    }
}

/* Threads used by the OpenMP loops from now on (the benchmark times the oracle on one core
 * as well as on all of them). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
