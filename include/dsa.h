/*
 * dsa.h - C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * The path has three stages, as the DeepSeek-V3.2-Exp pages describe DSA:
 *   1. the lightning indexer scores every earlier key for each query token
 *      ("DeepSeek-V3.2-Exp" overview, section "架构 & 背后实现"; lightning-indexer
 *      walk-through, step 3 "相关性得分计算"),
 *   2. a per-query top-k keeps the k best-scoring positions
 *      (walk-through step 4; "DeepSeek-V3.2-Exp解析" section 一.1),
 *   3. MQA-mode attention over the MLA latent cache runs on the selected rows only
 *      ("DeepSeek-V3.2 explained", sections 二.1 and 二.4: DSA(q_t,K,V) = attention of q_t over
 *      the rows picked by TopK(Indexer(q_t,K)); one 576-wide latent row per token shared by
 *      every head).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: the caller allocates every buffer (inputs, outputs, workspace) in device
 *    memory.  The library never allocates, frees or synchronises; all work is enqueued on
 *    the caller's stream.  Apart from dsa_forward_noalloc's per-device scratch array (see
 *    there), the library keeps no mutable global state and is thread-safe.
 *  - Batches: a batch holds n_seqs sequences.  Sequence b owns query rows
 *    [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]) of the packed arrays.  Its
 *    queries are the last len_q(b) tokens of its key sequence, so query row i of b sits at
 *    position p = len_k(b) - len_q(b) + (i - cu_q[b]) and sees keys at positions 0..p
 *    (causal, the query's own position included).  Prefill is one sequence with
 *    len_q = len_k; decode is len_q = 1 per sequence.
 *  - Validation: every argument is checked on the host before anything is enqueued (null
 *    pointers, unsupported dims, topk outside [1, 8192], len_q > len_k, non-monotone or
 *    non-zero-based offsets, pointers not 16-byte aligned, strides too small or not a
 *    multiple of 4, workspace too small).  On error nothing is enqueued and nothing is
 *    written.  A failed kernel launch returns DSA_ERR_HIP.
 *  - Supported dims: (n_idx_heads, idx_dim, n_heads, qk_dim, v_dim) is either the
 *    DeepSeek-V3.2-Exp shape (64, 128, 128, 576, 512) or the tiny test shape
 *    (4, 32, 8, 80, 64); topk may be any value in [1, 8192]; sm_scale any positive
 *    finite number.  Anything else returns DSA_ERR_UNSUPPORTED.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,
    DSA_ERR_UNSUPPORTED = 2,
    DSA_ERR_WORKSPACE = 3,
    DSA_ERR_HIP = 4
} dsa_status;

/* Shape of one DSA layer. */
typedef struct {
    int32_t n_idx_heads; /* H_I: indexer heads (64)                                  */
    int32_t idx_dim;     /* d_I: indexer head dim (128)                              */
    int32_t topk;        /* k: selected positions per query (2048; at most 8192)      */
    int32_t n_heads;     /* H: attention heads sharing each latent row (128)         */
    int32_t qk_dim;      /* latent row width used for the logits (576 = 512 + 64)    */
    int32_t v_dim;       /* value width = leading part of the latent row (512)       */
    float sm_scale;      /* softmax scale applied to q.c (1/sqrt(192))               */
} dsa_dims;

/* Sequence layout of a batch.  The host and device arrays must hold the same values.
 * Caches (k8, k_scale, kv) are packed by default: sequence b's positions 0 .. len_k-1 are
 * rows cu_k[b] .. cu_k[b+1]-1.  With page_table_dev set they are paged instead, in pages
 * of DSA_PAGE_SIZE positions (the serving setups on the DeepSeek-V3.2-Exp pages use page
 * size 64): position p of sequence b is cache row
 *     page_table_dev[b * pages_per_seq + p / 64] * 64 + p % 64
 * of the caller's page pool of pool_rows rows.  With pool_rows > 0 the gathers treat a slot
 * whose page lies outside the pool as empty (dsa_check_indices reports it); with pool_rows = 0
 * page ids are trusted.  Paged caches are read by the decode paths (every sequence with one query
 * row), dsa_sparse_mqa, dsa_indexer_kl and dsa_cache_append; prefill with paged caches returns
 * DSA_ERR_UNSUPPORTED.  A sequence may hold at most 3,728,269 positions (2^32 bytes of latent
 * rows); longer ones return DSA_ERR_UNSUPPORTED. */
#define DSA_PAGE_SIZE 64
typedef struct {
    int32_t n_seqs;                 /* B >= 1                                          */
    const int32_t* cu_q_host;       /* [B+1] query row offsets, host memory, cu_q[0] = 0 */
    const int32_t* cu_k_host;       /* [B+1] key row offsets, host memory, cu_k[0] = 0   */
    const int32_t* cu_q_dev;        /* [B+1] the same offsets in device memory         */
    const int32_t* cu_k_dev;        /* [B+1]                                           */
    const int32_t* page_table_dev;  /* [B, pages_per_seq] page ids, or NULL (packed)    */
    int32_t pages_per_seq;          /* >= ceil(max len_k / 64) when paged               */
    int64_t pool_rows;              /* rows in the page pool, or 0 (not given)          */
} dsa_batch;

/* Bytes of workspace that dsa_forward uses by default for this batch (also enough for
 * dsa_sparse_mqa and dsa_dense_mqa on the whole batch): room for the scores, index rows and
 * score counts of 8192 query rows of the longest sequence.  dsa_forward runs a prefill in
 * passes of query rows sized by area, each as many rows as the workspace holds at the pass's
 * own row length, so early passes of a long sequence take more (shorter) rows.  It also
 * accepts a smaller workspace down to dsa_workspace_min (8 rows of the longest sequence);
 * the passes then hold fewer rows.  Results do not depend on the workspace size. */
dsa_status dsa_workspace_size(const dsa_dims* dims, const dsa_batch* batch, size_t* bytes);
dsa_status dsa_workspace_min(const dsa_dims* dims, const dsa_batch* batch, size_t* bytes);

/* Lightning indexer (stage 1).
 * For every query row i and every key position s in [0, p_i]:
 *   I[i,s] = k_scale[s] * sum_j (w[i,j] * q_scale[i,j]) * ReLU( q8[i,j,:] . k8[s,:] )
 * where the dot product runs over FP8 e4m3fn codes (exact products, fp32 accumulation)
 * and j over the n_idx_heads heads.  Both scales are positive, so they factor out of the
 * ReLU unchanged ("DeepSeek-V3.2-Exp" overview, indexer score; walk-through step 2 for the
 * cached FP8 keys and their scale, step 3 for ReLU and the weighted head sum).
 *   q8      [T, n_idx_heads, idx_dim] uint8 e4m3fn codes (T = cu_q[B])
 *   q_scale [T, n_idx_heads] float32 (> 0),  w [T, n_idx_heads] float32
 *   k8      [S, idx_dim] uint8 e4m3fn codes (S = cu_k[B]),  k_scale [S] float32 (> 0)
 *   scores  float32; row i starts at scores + i*score_stride and receives entries
 *           0..p_i; entries past p_i are left untouched.  score_stride >= max p_i + 1,
 *           multiple of 4. */
dsa_status dsa_indexer_scores(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                              const float* q_scale, const float* w, const uint8_t* k8,
                              const float* k_scale, float* scores, int64_t score_stride,
                              hipStream_t stream);

/* Top-k selection (stage 2).
 * For query row i with n = p_i + 1 valid scores at scores + i*score_stride, select the
 * min(k, n) positions with the largest scores ("DeepSeek-V3.2-Exp" deep dive, section 2.2
 * on fine-grained token selection: only the k best-scoring positions are kept).
 * Ranking: larger first, -0 equals +0, NaN below -inf, equal scores -> lower position first.
 * idx [T, topk] int32 receives the selected positions in ascending order followed by -1
 * in the unused slots.  The result is unique, so it is bit-exact and deterministic.
 *   ws / ws_bytes: optional workspace (NULL/0 allowed, else 16-byte aligned).  With at least
 *   dsa_topk_workspace_size bytes (non-zero only for batches of fewer than 128 rows, e.g.
 *   decode) each row is split over several workgroups; otherwise one workgroup selects each
 *   row.  The result is the same.  The workspace is scratch owned by the caller; its
 *   contents are undefined afterwards. */
dsa_status dsa_topk(const dsa_dims* dims, const dsa_batch* batch, const float* scores,
                    int64_t score_stride, int32_t* idx, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Workspace that lets dsa_topk split rows over several workgroups for this batch (0 when
 * the batch has 128 rows or more, rows longer than 131072 scores, or topk above 2048). */
dsa_status dsa_topk_workspace_size(const dsa_dims* dims, const dsa_batch* batch, size_t* bytes);

/* Fused indexer -> top-k, as two calls (what dsa_forward does in each prefill pass).
 * dsa_indexer_scores_counted: dsa_indexer_scores for a prefill batch (a sequence with several
 *   query rows; decode batches and paged caches: DSA_ERR_UNSUPPORTED) that also counts, per
 *   query row, the scores it stores that are >= +0 by their order-preserving 32-bit key
 *   (bits 30..21, i.e. sign, exponent and two mantissa bits of the score):
 *   counts [T, DSA_COUNT_BINS] uint32, cleared by the call.
 * dsa_topk_counted: dsa_topk from those scores and counts.  The counts give the selection's
 *   first radix digit without reading the row, so each row is read once (rows with fewer
 *   than topk scores >= +0, or too many candidates for on-chip memory, fall back to the
 *   two-read selection).  The result is identical to dsa_topk. */
#define DSA_COUNT_BINS 1024
dsa_status dsa_indexer_scores_counted(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                                      const float* q_scale, const float* w, const uint8_t* k8,
                                      const float* k_scale, float* scores, int64_t score_stride,
                                      uint32_t* counts, hipStream_t stream);
dsa_status dsa_topk_counted(const dsa_dims* dims, const dsa_batch* batch, const float* scores,
                            int64_t score_stride, const uint32_t* counts, int32_t* idx, hipStream_t stream);

/* Sparse MQA over the latent cache (stage 3).
 * For query row i and head h, over the slots of idx[i,:] that hold a position of the row's
 * own sequence, i.e. a value in [0, len_k) (-1 marks an empty slot; any other value is treated
 * as empty too and never loaded; dsa_check_indices reports such rows):
 *   z_s = sm_scale * q[i,h,:qk_dim] . kv[s,:qk_dim]
 *   out[i,h,:] = sum_s softmax(z)_s * kv[s,:v_dim],   lse[i,h] = ln sum_s exp(z_s)
 * Every head reads the same latent rows (MQA mode).  A row without valid slots gets
 * out = 0 and lse = -inf.
 *   q   [T, n_heads, qk_dim] bf16 bits,  kv [S, qk_dim] bf16 bits,  idx [T, topk] int32
 *   out [T, n_heads, v_dim] bf16 bits,   lse [T, n_heads] float32 or NULL
 *   ws / ws_bytes: workspace (may be NULL/0 unless dsa_workspace_size asks for it; it is
 *   used to split rows over several workgroups when T is small, e.g. decode). */
dsa_status dsa_sparse_mqa(const dsa_dims* dims, const dsa_batch* batch, const uint16_t* q,
                          const uint16_t* kv, const int32_t* idx, uint16_t* out, float* lse,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Dense causal MQA: the attention above over every position s in [0, p] of query row i's
 * sequence, without an index row.  For a row with p + 1 <= topk this is exactly what DSA
 * computes (top-k keeps every earlier position); the pages name it the short-sequence
 * masked-MHA mode (DSA deep dive, section 4, efficiency).  dsa_forward uses it for passes
 * whose rows all have p + 1 <= topk.  Same layouts as dsa_sparse_mqa (dims->topk unused
 * beyond validation); ws as there: needed when T < 128 (the rows are then split over
 * workgroups by their length), sized by dsa_workspace_size. */
dsa_status dsa_dense_mqa(const dsa_dims* dims, const dsa_batch* batch, const uint16_t* q,
                         const uint16_t* kv, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* The whole hot path: indexer -> top-k -> sparse MQA, on the caller's stream.
 * Inputs as above.  Scores live only in the workspace, one pass of query rows at a time;
 * the full L x L score matrix never exists.  Rows with p + 1 <= topk skip the indexer and
 * the selection (their index set is every earlier position; the result is the same), and a
 * pass whose rows all have p + 1 <= topk runs the dense causal attention of dsa_dense_mqa
 * (index rows are then written only when idx_out is given).
 *   idx_out [T, topk] int32 or NULL (then the selected positions stay in the workspace). */
dsa_status dsa_forward(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                       const float* q_scale, const float* w, const uint8_t* k8,
                       const float* k_scale, const uint16_t* q, const uint16_t* kv,
                       uint16_t* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* dsa_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation with its workspace
 * taken from a fixed array of DSA_NOALLOC_SCRATCH_BYTES bytes in the library's own device memory
 * (one array per GPU, set up on the first call on that device and held until the process ends).
 * The call allocates and frees nothing.  The caller still passes inputs and outputs; call it with
 * the device of `stream` current.  Batches whose smallest workspace (dsa_workspace_min) exceeds
 * the array return DSA_ERR_WORKSPACE before anything is enqueued; prefill passes are sized to the
 * array.  Every call on a GPU shares that GPU's array: calls that overlap on one GPU (two streams,
 * two threads) race and give undefined results; calls in stream order are safe.  Results equal
 * dsa_forward's. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status dsa_forward_noalloc(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                               const float* q_scale, const float* w, const uint8_t* k8,
                               const float* k_scale, const uint16_t* q, const uint16_t* kv,
                               uint16_t* out, float* lse, int32_t* idx_out, hipStream_t stream);

/* Indexer training target, forward only (DeepSeek-V3.2-Exp overview, "训练": the dense
 * warm-up aligns the indexer with the main attention summed over heads and L1-normalised,
 * and the sparse stage does the same on the selected set only; 解析 §二).  For query row i
 * over its slots S_i (the non-(-1) entries of idx[i,:], or every position s in [0, p] when
 * idx is NULL):
 *   P_i[s] = sum_h exp(sm_scale * q[i,h,:] . kv[s,:] - lse[i,h]),  then P_i /= sum_s P_i[s]
 *   Q_i    = softmax over S_i of the indexer scores I[i,s]
 *   kl[i]  = KL(P_i || Q_i) = sum_s P log(P / Q);  kl_rev[i] = KL(Q_i || P_i)  (+inf if some
 *            slot has P = 0);  0 for a row without slots.
 * The pages write the divergence with its arguments in both orders; both are returned.
 *   q, kv   as for dsa_sparse_mqa (packed or paged caches);  idx [T, topk] int32 or NULL
 *   lse     [T, n_heads] float32: natural-log LSE of the attention over the same slots (what
 *           dsa_sparse_mqa with this idx, or dsa_dense_mqa, return)
 *   scores  float32 row i at scores + i*score_stride, entry s = I[i,s] for every slot s
 *           (what dsa_indexer_scores writes); score_stride >= max len_k, multiple of 4
 *   kl [T] float32;  kl_rev [T] float32 or NULL. */
dsa_status dsa_indexer_kl(const dsa_dims* dims, const dsa_batch* batch, const uint16_t* q,
                          const uint16_t* kv, const float* lse, const int32_t* idx, const float* scores,
                          int64_t score_stride, float* kl, float* kl_rev, hipStream_t stream);

/* Decode cache producer (the indexer's RoPE + FP8 step before the selection: DeepSeek-V3.2-Exp
 * lightning-indexer walk-through, step 2 — rotary encoding of the first 64 dims of the indexer
 * query and key, FP8 quantisation of both, the key codes and their scale kept in the cache).
 * For the len_q new tokens of each sequence (positions len_k - len_q + i, already counted in
 * cu_k):
 *   - RoPE on dims 0 .. R-1 (R = idx_dim / 2: 64 for the production shape): pairs (2i, 2i+1)
 *     rotate by the caller's table angle for (position, i),
 *         r0 = x0*cos - x1*sin,  r1 = x0*sin + x1*cos   (float32, each product and sum rounded);
 *   - per row (each query head, and the key) scale = amax/448 (1 for an all-zero row) and
 *     e4m3fn codes of x/scale (round to nearest even, clamped to +-448), all in float32;
 *   - the key's codes and scale are written to the caches at the token's cache row (packed or
 *     paged, see dsa_batch), and the token's bf16 latent row is copied there when given.
 *   q_idx  [T, n_idx_heads, idx_dim] float32,  k_idx [T, idx_dim] float32  (before RoPE)
 *   kv_new [T, qk_dim] bf16 bits or NULL (then kv_cache may be NULL)
 *   rope_cos, rope_sin [n_pos, R/2] float32, n_pos > every new token's position
 *   q8 [T, n_idx_heads, idx_dim] uint8 and q_scale [T, n_idx_heads] float32 receive the
 *   query codes; k8_cache [rows, idx_dim], k_scale_cache [rows], kv_cache [rows, qk_dim]. */
dsa_status dsa_cache_append(const dsa_dims* dims, const dsa_batch* batch, const float* q_idx,
                            const float* k_idx, const uint16_t* kv_new, const float* rope_cos,
                            const float* rope_sin, int32_t n_pos, uint8_t* q8, float* q_scale,
                            uint8_t* k8_cache, float* k_scale_cache, uint16_t* kv_cache,
                            hipStream_t stream);

/* Index-row check (the selected positions are the attention's gather addresses: lightning-
 * indexer walk-through, step 4).  For each query row i of the batch, row_flags[i] (uint32,
 * device memory) receives the OR of:
 *   DSA_IDX_OUT_OF_RANGE  an entry below -1 or >= len_k of the row's sequence
 *   DSA_IDX_NOT_CAUSAL    an entry in (p_i, len_k): past the query's own position
 *   DSA_IDX_NOT_SORTED    valid entries not strictly ascending, or a valid entry after a -1
 *                         (the form dsa_topk writes; dsa_sparse_mqa accepts any order)
 *   DSA_IDX_BAD_PAGE      paged caches with pool_rows > 0: an entry whose page lies outside the
 *                         pool
 * 0 for a row that dsa_topk could have written.  The gathers of dsa_sparse_mqa and
 * dsa_indexer_kl treat out-of-range entries and bad pages as empty slots, so such rows never
 * make them read outside the caches; this call says whether a row had any.
 *   idx [T, topk] int32 (16-byte aligned), row_flags [T] uint32. */
#define DSA_IDX_OUT_OF_RANGE 1u
#define DSA_IDX_NOT_CAUSAL 2u
#define DSA_IDX_NOT_SORTED 4u
#define DSA_IDX_BAD_PAGE 8u
dsa_status dsa_check_indices(const dsa_dims* dims, const dsa_batch* batch, const int32_t* idx,
                             uint32_t* row_flags, hipStream_t stream);

/* Debug checks.  With the environment variable DSA_DEBUG_CHECKS=1 (read at every call),
 * dsa_sparse_mqa, dsa_indexer_kl and dsa_forward run the check above on every index row before
 * their gathers read it and OR the flags into a per-device word.  dsa_debug_flags copies the
 * current device's word to *flags (host memory; waits for the device) and clears it when clear
 * is non-zero.  Without the variable the word stays 0 and nothing extra is launched. */
dsa_status dsa_debug_flags(uint32_t* flags, int clear);

/* Static description of a status code. */
const char* dsa_status_string(dsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
