// Host-side declarations shared between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

enum class Shape { Prod, Tiny };

struct IndexerArgs {
    Shape shape;
    const uint8_t* q8;
    const float* q_scale;
    const float* w;
    const uint8_t* k8;
    const float* k_scale;
    float* scores;
    int64_t score_stride;
};

// Prefill tiles for rows [row0, row0 + n_rows) of one sequence whose first row sits at
// position pos0 and whose key rows start at kbase.  Row i of the launch writes
// scores + i * score_stride.
// With hist != nullptr, row i also adds its stored non-negative scores to the kHistBins
// counts at hist + i * kHistBins (key bits 30..21 of score_key; the counts must start at 0).
constexpr int kHistBins = 1024;
hipError_t launch_indexer_prefill(const IndexerArgs& a, int row0, int n_rows, int pos0,
                                  int kbase, float* scores, hipStream_t st, uint32_t* hist = nullptr);
// Decode: one query row per sequence (cu_q[b+1] - cu_q[b] == 1); row cu_q[b] of the scores.
// Paged caches: pages != nullptr (see RowMap).
// With hist, also adds each row's counts of stored scores >= +0 by key bits 30..21 to
// hist + row * kHistBins (which must start at 0), like the prefill kernel.
hipError_t launch_indexer_decode(const IndexerArgs& a, int n_seqs, int max_keys,
                                 const int32_t* cu_q, const int32_t* cu_k, const int32_t* pages,
                                 int pages_per_seq, hipStream_t st, uint32_t* hist = nullptr);

// Top-k over n_rows score rows; row i reads scores + i * stride and writes idx + i * topk.
// With a workspace of topk_ws_bytes(n_rows, max_len, topk) bytes (max_len = the longest
// row) rows are split over several workgroups; without one (or for rows too long for the
// split) one workgroup selects each row.  Both give the same result.
size_t topk_ws_bytes(int n_rows, int max_len, int topk);
// Top-k of few long rows from the indexer's per-row counts (decode): segment workgroups
// append each row's candidates to a list in the workspace, then one workgroup per row selects
// from it; rows the list path does not apply to are selected from the scores.  The workspace
// holds topk_list_ws_bytes(n_rows) bytes: n_rows int list sizes, which must be 0 at the
// launch, then the lists.  The result equals launch_topk's.
size_t topk_list_ws_bytes(int n_rows);
hipError_t launch_topk_list(const float* scores, int64_t stride, const uint32_t* hist, int32_t* idx, int topk,
                            const RowMap& map, int n_rows, int max_len, void* ws, hipStream_t st);
// Top-k of rows whose non-negative scores the indexer counted into hist (kHistBins per row):
// one read of each row when it holds at least topk non-negative scores; the same result.
hipError_t launch_topk_from_hist(const float* scores, int64_t stride, const uint32_t* hist, int32_t* idx,
                                 int topk, const RowMap& map, int n_rows, hipStream_t st);
// p[0 .. n) = 0 (a kernel, so that the call can be captured in a graph).
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t st);
hipError_t launch_topk(const float* scores, int64_t stride, int32_t* idx, int topk,
                       const RowMap& map, int n_rows, int max_len, void* ws, size_t ws_bytes,
                       hipStream_t st);

// How the attention finds a row's key positions.
enum class IdxMode : int {
    General = 0,  // idx row of topk slots, -1 anywhere
    Front = 1,    // idx row whose valid slots come first (top-k output): only the first
                  // min(topk, p + 1) slots are read
    Dense = 2,    // no idx: slot j holds position j for j <= p (dense causal attention)
};

struct MqaArgs {
    Shape shape;
    const uint16_t* q;
    const uint16_t* kv;
    const int32_t* idx;  // row i of the launch at idx + i * topk (unused when Dense)
    int topk;
    uint16_t* out;       // indexed by packed query row
    float* lse;          // nullable, indexed by packed query row
    float sm_scale;
    IdxMode mode = IdxMode::General;
};

// Bytes of split partials for n_rows rows split n_split ways.
size_t mqa_split_bytes(Shape shape, int n_rows, int n_split);
// Sparse MQA for n_rows rows; n_split > 1 splits each row's slots over workgroups and
// merges the partials (ws must hold mqa_split_bytes).
hipError_t launch_sparse_mqa(const MqaArgs& a, const RowMap& map, int n_rows, int n_split,
                             void* ws, hipStream_t st);

struct CacheAppendArgs {
    Shape shape;
    const float* q_idx;      // [T, H_I, d_I] new tokens' indexer queries (before RoPE)
    const float* k_idx;      // [T, d_I] new tokens' indexer keys (before RoPE)
    const uint16_t* kv_new;  // [T, qk_dim] bf16 latent rows, or nullptr
    const float* rope_cos;   // [n_pos, d_I / 4]
    const float* rope_sin;
    uint8_t* q8;             // [T, H_I, d_I]
    float* q_scale;          // [T, H_I]
    uint8_t* k8_cache;       // rows of the caches (packed or paged, see RowMap)
    float* k_scale_cache;
    uint16_t* kv_cache;
};

// RoPE + FP8 codes of the new tokens' indexer query and key; key codes, scale and latent row
// written at each token's cache row.
hipError_t launch_cache_append(const CacheAppendArgs& a, const RowMap& map, int n_rows, hipStream_t st);

struct KlArgs {
    Shape shape;
    const uint16_t* q;      // [T, H, qk_dim] bf16
    const uint16_t* kv;     // latent cache rows (packed or paged, see RowMap)
    const float* lse;       // [T, H] natural-log LSE of the attention over the same slots
    const int32_t* idx;     // [T, topk] slot positions (unused when Dense)
    int topk;
    IdxMode mode;
    const float* scores;    // indexer scores, row i at scores + i * stride, index = position
    int64_t stride;
    float* kl;              // [T] KL(P || softmax(I))
    float* kl_rev;          // [T] KL(softmax(I) || P) or nullptr
    float sm_scale;
};

// Flags of an index row (the values of DSA_IDX_* in dsa.h).
constexpr uint32_t kIdxOutOfRange = 1u;  // an entry below -1 or past the sequence
constexpr uint32_t kIdxNotCausal = 2u;   // an entry past the query's own position
constexpr uint32_t kIdxNotSorted = 4u;   // valid entries not strictly ascending before the -1 pads
constexpr uint32_t kIdxBadPage = 8u;     // paged caches: an entry's page lies outside the pool
// Checks n_rows index rows (row i at idx + i * topk): row_flags[i] (if given) receives the OR
// of the row's flags, and every non-zero row ORs them into *any_flags (if given).
hipError_t launch_check_indices(const int32_t* idx, int topk, const RowMap& map, int n_rows, uint32_t* row_flags,
                                uint32_t* any_flags, hipStream_t st);

// KL divergences between the heads-summed attention distribution and the indexer's softmax
// over each row's slots (one workgroup per row).
hipError_t launch_indexer_kl(const KlArgs& a, const RowMap& map, int n_rows, hipStream_t st);

}  // namespace dsa
