/* Memory and undefined-behaviour check of the CPU oracle: built together with oracle/oracle.c
 * under AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py, it calls
 * every oracle function on small inputs with the edge cases of the method (one key, k above
 * and equal to the row length, empty and out-of-order slots, rows without slots, all-zero
 * quantiser rows, NaN and infinite scores) and checks a few results that are fixed by
 * definition.  Correctness itself is pinned by the Python tests; this program exists so that
 * any out-of-bounds access or undefined operation in the oracle aborts a run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e4m3(uint8_t b);
int64_t orc_e4m3_fixed(uint8_t b);
double orc_bf16(uint16_t h);
void orc_decode_e4m3(int64_t n, const uint8_t* in, double* out);
void orc_decode_bf16(int64_t n, const uint16_t* in, double* out);
double orc_dot_e4m3(int d, const uint8_t* a, const uint8_t* b);
int64_t orc_dot_e4m3_fixed(int d, const uint8_t* a, const uint8_t* b);
double orc_index_score(int H, int d, const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8, float ks);
void orc_indexer_rows(int H, int d, const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                      const float* ks, int nrows, const int32_t* rows, const int32_t* pos, double* out,
                      int64_t out_stride);
void orc_topk_rows_f64(int nrows, const int64_t* n, const double* x, int64_t stride, int k, int32_t* out);
void orc_topk_rows_f32(int nrows, const int64_t* n, const float* x, int64_t stride, int k, int32_t* out);
void orc_sparse_mqa(int H, int Dqk, int Dv, double sm, int T, const uint16_t* q, const uint16_t* kv, int k,
                    const int32_t* idx, double* out, double* lse);
void orc_dense_causal(int H, int Dqk, int Dv, double sm, int T, const int32_t* pos, const uint16_t* q,
                      const uint16_t* kv, double* out, double* lse);
uint8_t orc_encode_e4m3(float x);
void orc_encode_e4m3_n(int64_t n, const float* x, uint8_t* out);
void orc_rope_f32(int n_rows, int d, const float* x, int64_t pos, const float* cos_tab, const float* sin_tab,
                  int64_t tab_stride, int rope_dim, float* out);
void orc_quantize_rows_e4m3(int n_rows, int d, const float* x, uint8_t* codes, float* scale);
void orc_cache_append(int n, int H, int d, const float* q_idx, const float* k_idx, const int64_t* pos,
                      const float* cos_tab, const float* sin_tab, int64_t tab_stride, int rope_dim, uint8_t* q8,
                      float* q_scale, uint8_t* k8, float* k_scale);
void orc_indexer_kl(int H, int Dqk, double sm, int T, const uint16_t* q, const uint16_t* kv, const double* lse,
                    int k, const int32_t* slots, const double* scores, int64_t score_stride, double* kl,
                    double* rev);
int orc_num_threads(void);

static int failures = 0;
#define CHECK(c)                                                     \
    do {                                                             \
        if (!(c)) {                                                  \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                              \
        }                                                            \
    } while (0)

static uint32_t rng = 12345u;
static uint32_t next(void) {
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return rng;
}
static uint8_t code(void) {
    uint8_t c = (uint8_t)(next() & 0xff);
    return (c & 0x7f) == 0x7f ? 0x38 : c;
}
static uint16_t bf(void) { return (uint16_t)(0x3c00 + (next() & 0x03ff)) ^ (uint16_t)((next() & 1) << 15); }

int main(void) {
    /* codecs */
    double dec[256];
    uint8_t all[256];
    for (int i = 0; i < 256; ++i) all[i] = (uint8_t)i;
    orc_decode_e4m3(256, all, dec);
    CHECK(dec[0x7e] == 448.0 && isnan(dec[0x7f]) && orc_e4m3_fixed(0x01) == 1);
    uint16_t hb[3] = {0x3f80, 0xc000, 0x0000};
    double hd[3];
    orc_decode_bf16(3, hb, hd);
    CHECK(hd[0] == 1.0 && hd[1] == -2.0 && hd[2] == 0.0 && orc_bf16(0x3f80) == 1.0);

    /* indexer: H = 4 heads of d = 32, 10 keys, rows at positions 0, 5 and 9 */
    enum { H = 4, D = 32, S = 10 };
    uint8_t q8[3 * H * D], k8[S * D];
    float qs[3 * H], w[3 * H], ks[S];
    for (int i = 0; i < 3 * H * D; ++i) q8[i] = code();
    for (int i = 0; i < S * D; ++i) k8[i] = code();
    for (int i = 0; i < 3 * H; ++i) {
        qs[i] = 0.5f + (float)(next() % 8) / 8.0f;
        w[i] = (float)((int)(next() % 9) - 4) / 4.0f;
    }
    for (int i = 0; i < S; ++i) ks[i] = 0.25f + (float)(next() % 4) / 4.0f;
    CHECK(orc_dot_e4m3(D, q8, k8) * 262144.0 == (double)orc_dot_e4m3_fixed(D, q8, k8));
    int32_t rows[3] = {0, 1, 2}, pos[3] = {0, 5, 9};
    double sc[3 * S];
    for (int i = 0; i < 3 * S; ++i) sc[i] = -7.0;
    orc_indexer_rows(H, D, q8, qs, w, k8, ks, 3, rows, pos, sc, S);
    CHECK(sc[0] == orc_index_score(H, D, q8, qs, w, k8, ks[0]) && sc[1] == -7.0 && sc[2 * S + 9] != -7.0);

    /* top-k: row lengths 1, 3, 10 at k = 1, 3, 4, 16; NaN, infinities and ties */
    int64_t n[3] = {1, 3, 10};
    double x[3 * S];
    float xf[3 * S];
    for (int i = 0; i < 3 * S; ++i) x[i] = (double)(next() % 5);
    x[S + 1] = NAN;
    x[2 * S + 3] = INFINITY;
    x[2 * S + 4] = -INFINITY;
    for (int i = 0; i < 3 * S; ++i) xf[i] = (float)x[i];
    int ks_[4] = {1, 3, 4, 16};
    for (int t = 0; t < 4; ++t) {
        int32_t out[3 * 16], out2[3 * 16];
        orc_topk_rows_f64(3, n, x, S, ks_[t], out);
        orc_topk_rows_f32(3, n, xf, S, ks_[t], out2);
        CHECK(memcmp(out, out2, sizeof(int32_t) * 3 * (size_t)ks_[t]) == 0);
        CHECK(out[0] == 0 && (ks_[t] < 2 || out[1] == -1));
    }

    /* sparse MQA and dense causal attention: H = 2 heads, 6-wide keys, 4-wide values */
    enum { HH = 2, DQ = 6, DV = 4, T = 4, K = 5 };
    uint16_t q[T * HH * DQ], kv[S * DQ];
    for (int i = 0; i < T * HH * DQ; ++i) q[i] = bf();
    for (int i = 0; i < S * DQ; ++i) kv[i] = bf();
    int32_t idx[T * K] = {0, -1, -1, -1, -1,   /* one key */
                          3, 1, -1, 2, 0,      /* unordered, an empty slot in between */
                          -1, -1, -1, -1, -1,  /* no slot */
                          0, 1, 2, 3, 4};
    double o[T * HH * DV], lse[T * HH], o2[T * HH * DV], lse2[T * HH];
    orc_sparse_mqa(HH, DQ, DV, 0.3, T, q, kv, K, idx, o, lse);
    CHECK(lse[2 * HH] == -INFINITY && o[2 * HH * DV] == 0.0);
    CHECK(fabs(o[0] - orc_bf16(kv[0])) < 1e-15);
    int32_t dpos[T] = {0, 3, 0, 4};
    orc_dense_causal(HH, DQ, DV, 0.3, T, dpos, q, kv, o2, lse2);
    for (int i = 0; i < HH * DV; ++i) CHECK(fabs(o2[3 * HH * DV + i] - o[3 * HH * DV + i]) < 1e-12);

    /* cache producer: an all-zero row, NaN, saturation, RoPE on 16 of 32 dims */
    float xs[3] = {NAN, 1e30f, -0.0f};
    uint8_t cs[3];
    orc_encode_e4m3_n(3, xs, cs);
    CHECK(cs[0] == 0x7f && cs[1] == 0x7e && cs[2] == 0x80 && orc_encode_e4m3(1.0f) == 0x38);
    enum { NP = 8, R = 16 };
    float cosv[NP * (R / 2)], sinv[NP * (R / 2)];
    for (int p = 0; p < NP; ++p)
        for (int i = 0; i < R / 2; ++i) {
            cosv[p * (R / 2) + i] = cosf(0.1f * (float)(p * (i + 1)));
            sinv[p * (R / 2) + i] = sinf(0.1f * (float)(p * (i + 1)));
        }
    float qf[2 * H * D], kf[2 * D], rot[H * D];
    for (int i = 0; i < 2 * H * D; ++i) qf[i] = (float)((int)(next() % 200) - 100) / 16.0f;
    for (int i = 0; i < 2 * D; ++i) kf[i] = (float)((int)(next() % 200) - 100) / 16.0f;
    for (int i = 0; i < D; ++i) qf[i] = 0.0f; /* head 0 of token 0: all zero */
    orc_rope_f32(H, D, qf, 3, cosv, sinv, R / 2, R, rot);
    CHECK(rot[D - 1] == qf[D - 1]);
    uint8_t c8[H * D];
    float scl[H];
    orc_quantize_rows_e4m3(H, D, qf, c8, scl);
    CHECK(scl[0] == 1.0f && c8[0] == 0);
    int64_t npos[2] = {0, 7};
    uint8_t oq8[2 * H * D], ok8[2 * D];
    float oqs[2 * H], oks[2];
    orc_cache_append(2, H, D, qf, kf, npos, cosv, sinv, R / 2, R, oq8, oqs, ok8, oks);
    CHECK(oqs[0] == 1.0f && memcmp(oq8, c8, D) == 0);

    /* indexer KL target: a row with one slot, a row without slots, a row with gaps */
    double lsek[3 * HH], sck[3 * S], kl[3], rv[3];
    for (int i = 0; i < 3 * HH; ++i) lsek[i] = 1.0;
    for (int i = 0; i < 3 * S; ++i) sck[i] = (double)(next() % 7) - 3.0;
    int32_t slots[3 * 4] = {2, -1, -1, -1, -1, -1, -1, -1, 0, -1, 5, 9};
    orc_indexer_kl(HH, DQ, 0.3, 3, q, kv, lsek, 4, slots, sck, S, kl, rv);
    CHECK(kl[0] == 0.0 && rv[0] == 0.0 && kl[1] == 0.0 && rv[1] == 0.0 && kl[2] >= 0.0 && rv[2] >= 0.0);

    CHECK(orc_num_threads() >= 1);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle under sanitizers: ok\n");
    return 0;
}
