/* Memory and undefined-behaviour check of the C ABI's host layer: built with the library's
 * host code under AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py,
 * it calls every entry point of include/dsa.h on the argument errors each one rejects (bad
 * dims, malformed batches, null and misaligned pointers, short strides and workspaces, paged
 * batches that do not fit their table) and checks the documented status.  No call gets past
 * validation, so nothing is enqueued and no device memory is touched (the pointers are fake,
 * 16-byte aligned host addresses that are never dereferenced); the program runs without a GPU. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsa.h"

static int failures = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        dsa_status got_ = (call);                                                           \
        if (got_ != (want)) {                                                               \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, (int)got_, \
                    (int)(want));                                                           \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

#define F ((void*)(uintptr_t)(1u << 20))        /* aligned fake pointer */
#define M ((void*)(uintptr_t)((1u << 20) + 4)) /* misaligned */

static dsa_dims prod(void) {
    dsa_dims d = {64, 128, 2048, 128, 576, 512, 0.0721f};
    return d;
}

typedef struct {
    int32_t q[40], k[40];
    dsa_batch b;
} host_batch;

static void make(host_batch* h, int n, const int32_t* cq, const int32_t* ck) {
    memcpy(h->q, cq, sizeof(int32_t) * (size_t)(n + 1));
    memcpy(h->k, ck, sizeof(int32_t) * (size_t)(n + 1));
    memset(&h->b, 0, sizeof h->b);
    h->b.n_seqs = n;
    h->b.cu_q_host = h->q;
    h->b.cu_k_host = h->k;
    h->b.cu_q_dev = (const int32_t*)F;
    h->b.cu_k_dev = (const int32_t*)F;
}

static dsa_status fwd(const dsa_dims* d, const dsa_batch* b, void* p, void* ws, size_t wsb) {
    return dsa_forward(d, b, p, p, p, p, p, p, p, p, NULL, NULL, ws, wsb, NULL);
}

int main(void) {
    dsa_dims d = prod();
    host_batch pre, dec, bad;
    const int32_t pq[2] = {0, 4096}, pk[2] = {0, 4096};
    make(&pre, 1, pq, pk);
    int32_t dq[33], dk[33];
    for (int i = 0; i <= 32; ++i) {
        dq[i] = i;
        dk[i] = 40000 * i;
    }
    make(&dec, 32, dq, dk);
    size_t lo = 0, hi = 0, tk = 0;
    EXPECT(dsa_workspace_min(&d, &pre.b, &lo), DSA_OK);
    EXPECT(dsa_workspace_size(&d, &pre.b, &hi), DSA_OK);
    EXPECT(dsa_topk_workspace_size(&d, &dec.b, &tk), DSA_OK);
    EXPECT(dsa_workspace_size(&d, &pre.b, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_workspace_size(NULL, &pre.b, &hi), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_workspace_size(&d, NULL, &hi), DSA_ERR_INVALID_ARG);

    /* dims */
    dsa_dims x = d;
    x.topk = 0;
    EXPECT(fwd(&x, &pre.b, F, F, hi), DSA_ERR_INVALID_ARG);
    x = d;
    x.topk = 8193;
    EXPECT(fwd(&x, &pre.b, F, F, hi), DSA_ERR_INVALID_ARG);
    x = d;
    x.sm_scale = 0.0f;
    EXPECT(fwd(&x, &pre.b, F, F, hi), DSA_ERR_INVALID_ARG);
    x = d;
    x.n_heads = 64;
    EXPECT(fwd(&x, &pre.b, F, F, hi), DSA_ERR_UNSUPPORTED);
    x = d;
    x.idx_dim = 64;
    EXPECT(dsa_workspace_min(&x, &pre.b, &lo), DSA_ERR_UNSUPPORTED);

    /* batches */
    const int32_t nz_q[2] = {1, 4}, nz_k[2] = {0, 4};
    make(&bad, 1, nz_q, nz_k);
    EXPECT(fwd(&d, &bad.b, F, F, hi), DSA_ERR_INVALID_ARG);
    const int32_t mq[2] = {0, 8}, mk[2] = {0, 4};
    make(&bad, 1, mq, mk);
    EXPECT(fwd(&d, &bad.b, F, F, hi), DSA_ERR_INVALID_ARG);
    const int32_t dq3[3] = {0, 4, 2}, dk3[3] = {0, 4, 8};
    make(&bad, 2, dq3, dk3);
    EXPECT(fwd(&d, &bad.b, F, F, hi), DSA_ERR_INVALID_ARG);
    bad = pre;
    bad.b.cu_q_host = pre.q;
    bad.b.cu_k_host = pre.k;
    bad.b.n_seqs = 0;
    EXPECT(fwd(&d, &bad.b, F, F, hi), DSA_ERR_INVALID_ARG);
    bad.b.n_seqs = 1;
    bad.b.cu_q_dev = NULL;
    EXPECT(fwd(&d, &bad.b, F, F, hi), DSA_ERR_INVALID_ARG);

    /* pointers and workspace */
    EXPECT(fwd(&d, &pre.b, NULL, F, hi), DSA_ERR_INVALID_ARG);
    EXPECT(fwd(&d, &pre.b, M, F, hi), DSA_ERR_INVALID_ARG);
    EXPECT(fwd(&d, &pre.b, F, NULL, hi), DSA_ERR_WORKSPACE);
    EXPECT(fwd(&d, &pre.b, F, F, lo - 1), DSA_ERR_WORKSPACE);
    EXPECT(dsa_forward(&d, &pre.b, F, F, F, F, F, F, F, F, M, NULL, F, hi, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_scores(&d, &pre.b, F, F, F, F, F, M, 4096, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_scores(&d, &pre.b, F, F, F, F, F, F, 4094, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_scores_counted(&d, &pre.b, F, F, F, F, F, F, 4096, NULL, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_scores_counted(&d, &dec.b, F, F, F, F, F, F, 40000, F, NULL), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_topk(&d, &pre.b, F, 4096, NULL, NULL, 0, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_topk(&d, &pre.b, F, 4000, F, NULL, 0, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_topk(&d, &pre.b, F, 4096, F, M, 1 << 20, NULL), DSA_ERR_WORKSPACE);
    EXPECT(dsa_topk_counted(&d, &pre.b, F, 4096, NULL, F, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_sparse_mqa(&d, &pre.b, F, F, NULL, F, NULL, NULL, 0, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_sparse_mqa(&d, &dec.b, F, F, F, F, NULL, F, 16, NULL), DSA_ERR_WORKSPACE);
    EXPECT(dsa_dense_mqa(&d, &pre.b, F, M, F, NULL, F, hi, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_kl(&d, &pre.b, F, F, F, NULL, F, 4094, F, NULL, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_kl(&d, &pre.b, F, F, NULL, NULL, F, 4096, F, NULL, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_cache_append(&d, &dec.b, F, F, F, F, F, 1 << 20, F, F, F, F, NULL, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_cache_append(&d, &dec.b, F, F, NULL, F, F, 100, F, F, F, F, NULL, NULL), DSA_ERR_INVALID_ARG);

    /* paged batches: the table must cover the longest sequence */
    host_batch pg;
    const int32_t gq[3] = {0, 1, 2}, gk[3] = {0, 257, 300};
    make(&pg, 2, gq, gk);
    pg.b.page_table_dev = (const int32_t*)F;
    pg.b.pages_per_seq = 4;
    EXPECT(fwd(&d, &pg.b, F, F, hi), DSA_ERR_INVALID_ARG);
    pg.b.pages_per_seq = 0;
    EXPECT(fwd(&d, &pg.b, F, F, hi), DSA_ERR_INVALID_ARG);

    /* no-allocation forward: a batch beyond the scratch array is rejected before any launch */
    int32_t bq[65], bk[65];
    host_batch big;
    for (int i = 0; i <= 64; ++i) {
        bq[i] = i;
        bk[i] = 131072 * i;
    }
    memset(&big, 0, sizeof big);
    big.b.n_seqs = 64;
    big.b.cu_q_host = bq;
    big.b.cu_k_host = bk;
    big.b.cu_q_dev = (const int32_t*)F;
    big.b.cu_k_dev = (const int32_t*)F;
    EXPECT(dsa_forward_noalloc(&d, &big.b, F, F, F, F, F, F, F, F, NULL, NULL, NULL), DSA_ERR_WORKSPACE);
    EXPECT(dsa_forward_noalloc(&x, &pre.b, F, F, F, F, F, F, F, F, NULL, NULL, NULL), DSA_ERR_UNSUPPORTED);

    /* index check and debug flags */
    EXPECT(dsa_check_indices(&d, &pre.b, NULL, F, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_check_indices(&d, &pre.b, F, M, NULL), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_check_indices(&x, &pre.b, F, F, NULL), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_debug_flags(NULL, 1), DSA_ERR_INVALID_ARG);
    /* a page pool of negative size; a sequence past 32-bit latent row offsets */
    const int32_t oq[2] = {0, 1}, ok_[2] = {0, 3728270};
    host_batch lng;
    make(&lng, 1, oq, ok_);
    EXPECT(fwd(&d, &lng.b, F, F, hi), DSA_ERR_UNSUPPORTED);
    make(&pg, 2, gq, gk);
    pg.b.page_table_dev = (const int32_t*)F;
    pg.b.pages_per_seq = 5;
    pg.b.pool_rows = -64;
    EXPECT(fwd(&d, &pg.b, F, F, hi), DSA_ERR_INVALID_ARG);

    /* status strings */
    for (int s = 0; s <= 4; ++s)
        if (dsa_status_string((dsa_status)s) == NULL || strncmp(dsa_status_string((dsa_status)s), "DSA_", 4) != 0)
            ++failures;
    if (dsa_status_string((dsa_status)77) == NULL) ++failures;

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("C ABI host layer under sanitizers: ok\n");
    return 0;
}
