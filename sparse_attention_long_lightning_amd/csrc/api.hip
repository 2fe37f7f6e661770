// C ABI of the DSA hot path: argument validation, workspace policy and the launch sequence
// of dsa_forward (lightning indexer -> top-k -> sparse MQA, "DeepSeek-V3.2-Exp解析" section
// 一.1 three-stage workflow).  Nothing here allocates, frees or synchronises.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dsa.h"
#include "internal.hpp"

using namespace dsa;

namespace {

constexpr int kDefaultChunkRows = 8192;  // query rows per prefill pass at the default size
constexpr int kRowGranule = 8;           // prefill passes cover multiples of this many rows
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Batch {
    int B = 0;
    int T = 0;  // total query rows
    int S = 0;  // total key rows
    int max_lk = 0;
    int max_lq = 0;
    bool decode = false;  // every sequence has exactly one query row
    const int32_t* pages = nullptr;  // paged caches (device page table) or nullptr
    int pages_per_seq = 0;
    int64_t pool_rows = 0;           // rows of the page pool (0: not given)
    const dsa_batch* raw = nullptr;
    RowMap map() const {
        return RowMap{raw->cu_q_dev, raw->cu_k_dev, B, 0, 0, 0, pages, pages_per_seq, pool_rows, decode};
    }
    int lq(int b) const { return raw->cu_q_host[b + 1] - raw->cu_q_host[b]; }
    int lk(int b) const { return raw->cu_k_host[b + 1] - raw->cu_k_host[b]; }
};

// Sequences are addressed with 32-bit byte offsets of 1152-byte latent rows from their first row.
constexpr int64_t kMaxLenK = (int64_t(1) << 32) / 1152 - 1;

bool debug_log() {
    static const bool on = [] {
        const char* e = getenv("DSA_LOG");
        return e != nullptr && e[0] == '1';
    }();
    return on;
}

dsa_status check_dims(const dsa_dims* d, Shape* shape) {
    if (d == nullptr) return DSA_ERR_INVALID_ARG;
    if (d->topk < 1 || d->topk > kMaxTopk) return DSA_ERR_INVALID_ARG;
    if (!(d->sm_scale > 0.f) || !std::isfinite(d->sm_scale)) return DSA_ERR_INVALID_ARG;
    if (d->n_idx_heads == 64 && d->idx_dim == 128 && d->n_heads == 128 && d->qk_dim == 576 &&
        d->v_dim == 512) {
        *shape = Shape::Prod;
        return DSA_OK;
    }
    if (d->n_idx_heads == 4 && d->idx_dim == 32 && d->n_heads == 8 && d->qk_dim == 80 &&
        d->v_dim == 64) {
        *shape = Shape::Tiny;
        return DSA_OK;
    }
    return DSA_ERR_UNSUPPORTED;
}

dsa_status check_batch(const dsa_batch* b, Batch* out) {
    if (b == nullptr || b->n_seqs < 1 || b->cu_q_host == nullptr || b->cu_k_host == nullptr ||
        b->cu_q_dev == nullptr || b->cu_k_dev == nullptr)
        return DSA_ERR_INVALID_ARG;
    if (b->cu_q_host[0] != 0 || b->cu_k_host[0] != 0) return DSA_ERR_INVALID_ARG;
    Batch r;
    r.raw = b;
    r.B = b->n_seqs;
    r.decode = true;
    for (int i = 0; i < b->n_seqs; ++i) {
        const int64_t lq = (int64_t)b->cu_q_host[i + 1] - b->cu_q_host[i];
        const int64_t lk = (int64_t)b->cu_k_host[i + 1] - b->cu_k_host[i];
        if (lq < 0 || lk < 0 || lq > lk) return DSA_ERR_INVALID_ARG;
        if (lk > kMaxLenK) return DSA_ERR_UNSUPPORTED;
        if (lq > r.max_lq) r.max_lq = (int)lq;
        if (lk > r.max_lk) r.max_lk = (int)lk;
        if (lq != 1) r.decode = false;
    }
    r.T = b->cu_q_host[b->n_seqs];
    r.S = b->cu_k_host[b->n_seqs];
    if (b->page_table_dev != nullptr) {
        if (b->pages_per_seq < 1 || (int64_t)b->pages_per_seq * kPage < r.max_lk || b->pool_rows < 0)
            return DSA_ERR_INVALID_ARG;
        r.pages = b->page_table_dev;
        r.pages_per_seq = b->pages_per_seq;
        r.pool_rows = b->pool_rows;
    }
    *out = r;
    return DSA_OK;
}

// Split count of the sparse MQA for a batch of T rows: about one workgroup per CU (256,
// two workgroups of 64 heads per row) when there are few rows (decode), at least 128
// selected slots per split.  More splits would run in a second round of workgroups and
// write more partials.
int mqa_splits(int T, int topk) {
    if (T <= 0 || T >= 128) return 1;
    int n = (128 + T - 1) / T;
    const int cap = (topk + 127) / 128;
    if (n > cap) n = cap;
    if (n > 8) n = 8;
    return n < 1 ? 1 : n;
}

int64_t score_stride_for(const Batch& bt) { return ((int64_t)bt.max_lk + 3) & ~(int64_t)3; }

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

struct ForwardPlan {
    int64_t stride = 0;
    int chunk = 0;  // prefill rows per pass
    size_t scores_off = 0, idx_off = 0, hist_off = 0, tail_off = 0, topk_bytes = 0, total = 0;
};

// Workspace layout of dsa_forward: [scores | idx (when idx_out is NULL) | hist | tail].
// Prefill: hist holds the indexer's per-row score counts that the top-k starts from.
// Decode: the tail holds the per-row score counts, the top-k list sizes and lists, and,
// later on the same stream, the MQA split partials.
ForwardPlan plan_forward(const dsa_dims* d, Shape shape, const Batch& bt, int chunk) {
    ForwardPlan p;
    p.stride = score_stride_for(bt);
    p.chunk = bt.decode ? bt.T : chunk;
    p.scores_off = 0;
    p.idx_off = align_up((size_t)p.chunk * p.stride * sizeof(float));
    p.hist_off = p.idx_off + align_up((size_t)p.chunk * d->topk * sizeof(int32_t));
    const size_t hist_bytes = bt.decode ? 0 : (size_t)p.chunk * kHistBins * sizeof(uint32_t);
    p.tail_off = p.hist_off + align_up(hist_bytes);
    p.topk_bytes = bt.decode ? (size_t)p.chunk * kHistBins * sizeof(uint32_t) + topk_list_ws_bytes(p.chunk) : 0;
    size_t tail = p.topk_bytes;
    if (bt.decode) {
        const size_t mqa = mqa_split_bytes(shape, bt.T, mqa_splits(bt.T, d->topk));
        if (mqa > tail) tail = mqa;
    }
    p.total = p.tail_off + align_up(tail);
    return p;
}

int default_chunk(const Batch& bt) {
    int c = bt.max_lq < kDefaultChunkRows ? bt.max_lq : kDefaultChunkRows;
    return c < 1 ? 1 : c;
}

}  // namespace

// Flags that DSA_DEBUG_CHECKS=1 collects from every index row a gather reads (the OR of the
// checker's row flags), per device; read and cleared by dsa_debug_flags.
static __device__ uint32_t debug_flags;

// Workspace of dsa_forward_noalloc: one array per GPU that loads the library, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the device memory:
// the device address is taken with hipGetSymbolAddress, once per device, and only that
// pointer reaches kernels.
static __device__ __attribute__((aligned(256))) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
uint32_t* g_debug_dev[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call there).
dsa_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSA_ERR_HIP;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return DSA_OK;
}

// Device address of the current device's debug flag word.
dsa_status debug_word_of_current_device(uint32_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_debug_dev[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_flags)) != hipSuccess || p == nullptr) return DSA_ERR_HIP;
        g_debug_dev[dev] = (uint32_t*)p;
    }
    *out = g_debug_dev[dev];
    return DSA_OK;
}

// Read on every call, so that a process can switch the checks on and off.
bool debug_checks() {
    const char* e = getenv("DSA_DEBUG_CHECKS");
    return e != nullptr && e[0] == '1';
}

// With DSA_DEBUG_CHECKS=1: checks the index rows a gather is about to read and ORs their flags
// into the device's debug word (a no-op otherwise).
hipError_t debug_check(const int32_t* idx, int topk, const RowMap& map, int n_rows, hipStream_t st) {
    if (!debug_checks() || idx == nullptr) return hipSuccess;
    uint32_t* word = nullptr;
    if (debug_word_of_current_device(&word) != DSA_OK) return hipErrorInvalidValue;
    return launch_check_indices(idx, topk, map, n_rows, nullptr, word, st);
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
    // a caller may pass any integer; reading it as an int keeps values outside the enum defined
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: unsupported dims";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace too small";
        case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP launch failure";
    }
    return "unknown dsa_status";
}

dsa_status dsa_workspace_size(const dsa_dims* dims, const dsa_batch* batch, size_t* bytes) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if (bytes == nullptr) return DSA_ERR_INVALID_ARG;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    const ForwardPlan p = plan_forward(dims, shape, bt, default_chunk(bt));
    // dsa_sparse_mqa and dsa_dense_mqa on the whole batch split fewer than 128 rows over
    // several workgroups (by k, or by the longest row)
    const int slots = dims->topk > bt.max_lk ? dims->topk : bt.max_lk;
    const size_t mqa = align_up(mqa_split_bytes(shape, bt.T, mqa_splits(bt.T, slots)));
    *bytes = p.total > mqa ? p.total : mqa;
    return DSA_OK;
}

dsa_status dsa_workspace_min(const dsa_dims* dims, const dsa_batch* batch, size_t* bytes) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if (bytes == nullptr) return DSA_ERR_INVALID_ARG;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    const int c = bt.max_lq < kRowGranule ? (bt.max_lq < 1 ? 1 : bt.max_lq) : kRowGranule;
    const ForwardPlan p = plan_forward(dims, shape, bt, c);
    *bytes = p.total;
    return DSA_OK;
}

namespace {

dsa_status indexer_scores(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                          const float* w, const uint8_t* k8, const float* k_scale, float* scores,
                          int64_t score_stride, uint32_t* counts, hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!q8 || !q_scale || !w || !k8 || !k_scale || !scores) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q8) || !aligned16(q_scale) || !aligned16(w) || !aligned16(k8) ||
        !aligned16(k_scale) || !aligned16(scores))
        return DSA_ERR_INVALID_ARG;
    if (score_stride < bt.max_lk || (score_stride & 3) != 0) return DSA_ERR_INVALID_ARG;
    if (counts != nullptr && (!aligned16(counts))) return DSA_ERR_INVALID_ARG;
    IndexerArgs a{shape, q8, q_scale, w, k8, k_scale, scores, score_stride};
    if (bt.decode) {
        if (counts != nullptr) return DSA_ERR_UNSUPPORTED;  // counts come from the prefill kernel
        return hip_status(launch_indexer_decode(a, bt.B, bt.max_lk, batch->cu_q_dev, batch->cu_k_dev, bt.pages,
                                                bt.pages_per_seq, stream));
    }
    if (bt.pages != nullptr) return DSA_ERR_UNSUPPORTED;  // paged caches: decode batches only
    if (counts != nullptr && launch_zero_words(counts, (int64_t)bt.T * kHistBins, stream) != hipSuccess)
        return DSA_ERR_HIP;
    for (int b = 0; b < bt.B; ++b) {
        const int lq = bt.lq(b), lk = bt.lk(b);
        if (lq == 0) continue;
        const int row0 = batch->cu_q_host[b];
        hipError_t e = launch_indexer_prefill(a, row0, lq, lk - lq, batch->cu_k_host[b],
                                              scores + (int64_t)row0 * score_stride, stream,
                                              counts ? counts + (int64_t)row0 * kHistBins : nullptr);
        if (e != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

}  // namespace

dsa_status dsa_indexer_scores(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                              const float* q_scale, const float* w, const uint8_t* k8,
                              const float* k_scale, float* scores, int64_t score_stride,
                              hipStream_t stream) {
    return indexer_scores(dims, batch, q8, q_scale, w, k8, k_scale, scores, score_stride, nullptr, stream);
}

dsa_status dsa_indexer_scores_counted(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                                      const float* q_scale, const float* w, const uint8_t* k8,
                                      const float* k_scale, float* scores, int64_t score_stride,
                                      uint32_t* counts, hipStream_t stream) {
    if (counts == nullptr) return DSA_ERR_INVALID_ARG;
    return indexer_scores(dims, batch, q8, q_scale, w, k8, k_scale, scores, score_stride, counts, stream);
}

dsa_status dsa_topk_counted(const dsa_dims* dims, const dsa_batch* batch, const float* scores,
                            int64_t score_stride, const uint32_t* counts, int32_t* idx, hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!scores || !idx || !counts || !aligned16(scores) || !aligned16(idx) || !aligned16(counts))
        return DSA_ERR_INVALID_ARG;
    if (score_stride < bt.max_lk || (score_stride & 3) != 0) return DSA_ERR_INVALID_ARG;
    const RowMap map = bt.map();
    return hip_status(launch_topk_from_hist(scores, score_stride, counts, idx, dims->topk, map, bt.T, stream));
}

dsa_status dsa_topk_workspace_size(const dsa_dims* dims, const dsa_batch* batch, size_t* bytes) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if (bytes == nullptr) return DSA_ERR_INVALID_ARG;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    *bytes = topk_ws_bytes(bt.T, bt.max_lk, dims->topk);
    return DSA_OK;
}

dsa_status dsa_topk(const dsa_dims* dims, const dsa_batch* batch, const float* scores,
                    int64_t score_stride, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!scores || !idx || !aligned16(scores) || !aligned16(idx)) return DSA_ERR_INVALID_ARG;
    if (score_stride < bt.max_lk || (score_stride & 3) != 0) return DSA_ERR_INVALID_ARG;
    if (ws != nullptr && !aligned16(ws)) return DSA_ERR_WORKSPACE;
    const RowMap map = bt.map();
    return hip_status(launch_topk(scores, score_stride, idx, dims->topk, map, bt.T, bt.max_lk, ws,
                                  ws == nullptr ? 0 : ws_bytes, stream));
}

dsa_status dsa_sparse_mqa(const dsa_dims* dims, const dsa_batch* batch, const uint16_t* q,
                          const uint16_t* kv, const int32_t* idx, uint16_t* out, float* lse,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!q || !kv || !idx || !out) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(idx) || !aligned16(out) ||
        (lse != nullptr && !aligned16(lse)))
        return DSA_ERR_INVALID_ARG;
    const int n_split = mqa_splits(bt.T, dims->topk);
    const size_t need = mqa_split_bytes(shape, bt.T, n_split);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return DSA_ERR_WORKSPACE;
    MqaArgs a{shape, q, kv, idx, dims->topk, out, lse, dims->sm_scale};
    const RowMap map = bt.map();
    hipError_t e = debug_check(idx, dims->topk, map, bt.T, stream);
    if (e == hipSuccess) e = launch_sparse_mqa(a, map, bt.T, n_split, ws, stream);
    return hip_status(e);
}

dsa_status dsa_dense_mqa(const dsa_dims* dims, const dsa_batch* batch, const uint16_t* q,
                         const uint16_t* kv, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!q || !kv || !out) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (lse != nullptr && !aligned16(lse)))
        return DSA_ERR_INVALID_ARG;
    const int n_split = mqa_splits(bt.T, bt.max_lk);
    const size_t need = mqa_split_bytes(shape, bt.T, n_split);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return DSA_ERR_WORKSPACE;
    MqaArgs a{shape, q, kv, nullptr, dims->topk, out, lse, dims->sm_scale, IdxMode::Dense};
    const RowMap map = bt.map();
    return hip_status(launch_sparse_mqa(a, map, bt.T, n_split, ws, stream));
}

dsa_status dsa_forward(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                       const float* q_scale, const float* w, const uint8_t* k8,
                       const float* k_scale, const uint16_t* q, const uint16_t* kv,
                       uint16_t* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!q8 || !q_scale || !w || !k8 || !k_scale || !q || !kv || !out) return DSA_ERR_INVALID_ARG;
    const void* ptrs[] = {q8, q_scale, w, k8, k_scale, q, kv, out};
    for (const void* p : ptrs)
        if (!aligned16(p)) return DSA_ERR_INVALID_ARG;
    if ((lse != nullptr && !aligned16(lse)) || (idx_out != nullptr && !aligned16(idx_out)))
        return DSA_ERR_INVALID_ARG;
    if (ws == nullptr || !aligned16(ws)) return DSA_ERR_WORKSPACE;
    const int topk = dims->topk;
    uint8_t* wsb = (uint8_t*)ws;

    if (bt.decode) {
        const ForwardPlan p = plan_forward(dims, shape, bt, bt.T);
        if (ws_bytes < p.total) return DSA_ERR_WORKSPACE;
        float* sc = (float*)(wsb + p.scores_off);
        int32_t* ix = idx_out ? idx_out : (int32_t*)(wsb + p.idx_off);
        IndexerArgs ia{shape, q8, q_scale, w, k8, k_scale, sc, p.stride};
        const RowMap map = bt.map();
        const int n_split = mqa_splits(bt.T, topk);
        // the top-k rows hold their valid slots first: short rows read only p + 1 of them
        MqaArgs ma{shape, q, kv, ix, topk, out, lse, dims->sm_scale, IdxMode::Front};
        if (debug_log())
            fprintf(stderr, "[dsa] decode B=%d max_len_k=%d stride=%lld splits=%d\n", bt.B, bt.max_lk,
                    (long long)p.stride, n_split);
        // tail: [counts (T x kHistBins) | list sizes (T) | lists]; counts and sizes start at 0
        uint32_t* hs = (uint32_t*)(wsb + p.tail_off);
        hipError_t e = launch_zero_words(hs, (int64_t)bt.T * (kHistBins + 1), stream);
        if (e == hipSuccess)
            e = launch_indexer_decode(ia, bt.B, bt.max_lk, batch->cu_q_dev, batch->cu_k_dev, bt.pages,
                                      bt.pages_per_seq, stream, hs);
        if (e == hipSuccess)
            e = launch_topk_list(sc, p.stride, hs, ix, topk, map, bt.T, bt.max_lk, hs + (size_t)bt.T * kHistBins,
                                 stream);
        if (e == hipSuccess) e = debug_check(ix, topk, map, bt.T, stream);
        if (e == hipSuccess) e = launch_sparse_mqa(ma, map, bt.T, n_split, wsb + p.tail_off, stream);
        return hip_status(e);
    }

    // Prefill: passes of query rows per sequence.  A pass of R rows ending at row r1 takes
    // [scores R x stride(r1) | idx R x topk | counts R x kHistBins] from the start of the
    // workspace, stride(r1) the length of its last row (rounded up to 4), so early passes of a
    // long sequence, whose rows are short, hold more rows than late ones; every pass takes as
    // many rows as fit (a multiple of kRowGranule, or the rest of the sequence).  The rows'
    // results do not depend on the passes.
    if (bt.pages != nullptr) return DSA_ERR_UNSUPPORTED;  // paged caches: decode batches only
    auto pass_bytes = [&](int64_t rows, int64_t stride_p) {
        return align_up((size_t)(rows * stride_p) * sizeof(float)) + align_up((size_t)rows * topk * sizeof(int32_t)) +
               align_up((size_t)rows * kHistBins * sizeof(uint32_t));
    };
    auto stride_to = [](int64_t len) { return (len + 3) & ~(int64_t)3; };
    // the workspace must hold kRowGranule full-length rows (all rows of shorter sequences)
    {
        const int min_rows = bt.max_lq < kRowGranule ? bt.max_lq : kRowGranule;
        if (pass_bytes(min_rows, score_stride_for(bt)) > ws_bytes) return DSA_ERR_WORKSPACE;
    }
    for (int b = 0; b < bt.B; ++b) {
        const int lq = bt.lq(b), lk = bt.lk(b);
        const int qb = batch->cu_q_host[b], kb = batch->cu_k_host[b];
        const int pos0 = lk - lq;
        for (int r0 = 0; r0 < lq;) {
            auto fits = [&](int rows) { return pass_bytes(rows, stride_to((int64_t)pos0 + r0 + rows)) <= ws_bytes; };
            int rows = lq - r0;
            if (!fits(rows)) {  // largest count that fits: fits() is monotone in the row count
                int lo = 1, hi = rows - 1;
                while (lo < hi) {
                    const int mid = lo + (hi - lo + 1) / 2;
                    if (fits(mid)) lo = mid; else hi = mid - 1;
                }
                rows = lo > kRowGranule ? lo - lo % kRowGranule : lo;
                if (!fits(rows)) return DSA_ERR_WORKSPACE;
            }
            const int r1 = r0 + rows;
            const int64_t stride = stride_to((int64_t)pos0 + r1);
            float* sc = (float*)wsb;
            int32_t* ix_ws = (int32_t*)(wsb + align_up((size_t)((int64_t)rows * stride) * sizeof(float)));
            uint32_t* hs = (uint32_t*)((uint8_t*)ix_ws + align_up((size_t)rows * topk * sizeof(int32_t)));
            if (debug_log())
                fprintf(stderr, "[dsa] prefill seq %d rows %d..%d stride %lld\n", b, r0, r1, (long long)stride);
            const IndexerArgs ia{shape, q8, q_scale, w, k8, k_scale, sc, stride};
            // rows with p + 1 <= topk keep every earlier position: no scores needed
            int rsel = topk - pos0;
            if (rsel < r0) rsel = r0;
            hipError_t e = hipSuccess;
            // the indexer counts each row's scores for the top-k as it stores them
            uint32_t* hrows = hs + (int64_t)(rsel - r0) * kHistBins;
            if (rsel < r1) e = launch_zero_words(hrows, (int64_t)(r1 - rsel) * kHistBins, stream);
            if (e == hipSuccess && rsel < r1)
                e = launch_indexer_prefill(ia, qb + rsel, r1 - rsel, pos0 + rsel, kb,
                                           sc + (int64_t)(rsel - r0) * stride, stream, hrows);
            int32_t* ix = idx_out ? idx_out + (int64_t)(qb + r0) * topk : ix_ws;
            RowMap map{nullptr, nullptr, 1, qb + r0, pos0 + r0, kb};
            // every row of the pass keeps all earlier positions (p + 1 <= k): dense causal
            // attention, and the index rows only if the caller asked for them
            const bool dense = pos0 + r1 <= topk;
            if (e == hipSuccess && (!dense || idx_out != nullptr))
                e = launch_topk_from_hist(sc, stride, hs, ix, topk, map, r1 - r0, stream);
            MqaArgs ma{shape, q, kv, ix, topk, out, lse, dims->sm_scale, dense ? IdxMode::Dense : IdxMode::Front};
            if (e == hipSuccess && !dense) e = debug_check(ix, topk, map, r1 - r0, stream);
            if (e == hipSuccess) e = launch_sparse_mqa(ma, map, r1 - r0, 1, nullptr, stream);
            if (e != hipSuccess) return DSA_ERR_HIP;
            r0 = r1;
        }
    }
    return DSA_OK;
}

dsa_status dsa_forward_noalloc(const dsa_dims* dims, const dsa_batch* batch, const uint8_t* q8,
                               const float* q_scale, const float* w, const uint8_t* k8,
                               const float* k_scale, const uint16_t* q, const uint16_t* kv,
                               uint16_t* out, float* lse, int32_t* idx_out, hipStream_t stream) {
    size_t need = 0;
    dsa_status st = dsa_workspace_min(dims, batch, &need);
    if (st != DSA_OK) return st;
    if (need > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != DSA_OK) return st;
    // dsa_forward sizes its passes to the array and clears, with kernels, every part of the
    // workspace that must start at zero
    return dsa_forward(dims, batch, q8, q_scale, w, k8, k_scale, q, kv, out, lse, idx_out, ws,
                       DSA_NOALLOC_SCRATCH_BYTES, stream);
}

dsa_status dsa_check_indices(const dsa_dims* dims, const dsa_batch* batch, const int32_t* idx,
                             uint32_t* row_flags, hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!idx || !row_flags || !aligned16(idx) || !aligned16(row_flags)) return DSA_ERR_INVALID_ARG;
    return hip_status(launch_check_indices(idx, dims->topk, bt.map(), bt.T, row_flags, nullptr, stream));
}

dsa_status dsa_debug_flags(uint32_t* flags, int clear) {
    if (flags == nullptr) return DSA_ERR_INVALID_ARG;
    uint32_t* word = nullptr;
    dsa_status st = debug_word_of_current_device(&word);
    if (st != DSA_OK) return st;
    if (hipMemcpy(flags, word, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return DSA_ERR_HIP;
    if (clear && hipMemset(word, 0, sizeof(uint32_t)) != hipSuccess) return DSA_ERR_HIP;
    return DSA_OK;
}

dsa_status dsa_indexer_kl(const dsa_dims* dims, const dsa_batch* batch, const uint16_t* q,
                          const uint16_t* kv, const float* lse, const int32_t* idx, const float* scores,
                          int64_t score_stride, float* kl, float* kl_rev, hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!q || !kv || !lse || !scores || !kl) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(lse) || !aligned16(scores) || !aligned16(kl) ||
        (idx != nullptr && !aligned16(idx)) || (kl_rev != nullptr && !aligned16(kl_rev)))
        return DSA_ERR_INVALID_ARG;
    if (score_stride < bt.max_lk || (score_stride & 3) != 0) return DSA_ERR_INVALID_ARG;
    KlArgs a{shape, q, kv, lse, idx, dims->topk, idx ? IdxMode::General : IdxMode::Dense, scores, score_stride,
             kl, kl_rev, dims->sm_scale};
    const RowMap map = bt.map();
    hipError_t e = debug_check(idx, dims->topk, map, bt.T, stream);
    if (e == hipSuccess) e = launch_indexer_kl(a, map, bt.T, stream);
    return hip_status(e);
}

dsa_status dsa_cache_append(const dsa_dims* dims, const dsa_batch* batch, const float* q_idx,
                            const float* k_idx, const uint16_t* kv_new, const float* rope_cos,
                            const float* rope_sin, int32_t n_pos, uint8_t* q8, float* q_scale,
                            uint8_t* k8_cache, float* k_scale_cache, uint16_t* kv_cache,
                            hipStream_t stream) {
    Shape shape;
    Batch bt;
    dsa_status st;
    if ((st = check_dims(dims, &shape)) != DSA_OK) return st;
    if ((st = check_batch(batch, &bt)) != DSA_OK) return st;
    if (bt.T == 0) return DSA_OK;
    if (!q_idx || !k_idx || !rope_cos || !rope_sin || !q8 || !q_scale || !k8_cache || !k_scale_cache)
        return DSA_ERR_INVALID_ARG;
    if ((kv_new == nullptr) != (kv_cache == nullptr)) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(rope_cos) || !aligned16(rope_sin) ||
        !aligned16(q8) || !aligned16(q_scale) || !aligned16(k8_cache) || !aligned16(k_scale_cache) ||
        (kv_new != nullptr && (!aligned16(kv_new) || !aligned16(kv_cache))))
        return DSA_ERR_INVALID_ARG;
    if (n_pos < bt.max_lk) return DSA_ERR_INVALID_ARG;  // every new position has a table row
    const RowMap map = bt.map();
    CacheAppendArgs a{shape, q_idx, k_idx, kv_new, rope_cos, rope_sin, q8, q_scale, k8_cache, k_scale_cache, kv_cache};
    return hip_status(launch_cache_append(a, map, bt.T, stream));
}

}  // extern "C"
