// Shared device-side definitions for the gfx950 DSA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxTopk = 2048;

// Maps a query row to its sequence, absolute position and key-row base.
//  single-sequence mode (cu_q == nullptr): row i -> position pos0 + i, key base kbase,
//      query row row0 + i of the packed query arrays;
//  batch mode: row i is a global query row; its sequence b is found in cu_q.
struct RowMap {
    const int32_t* cu_q;
    const int32_t* cu_k;
    int n_seqs;
    int row0;
    int pos0;
    int kbase;
};

struct RowInfo {
    int qrow;   // packed query row
    int pos;    // absolute position p (keys 0..p)
    int kbase;  // packed key row of position 0
};

__device__ __forceinline__ RowInfo row_info(const RowMap& m, int i) {
    RowInfo r;
    if (m.cu_q == nullptr) {
        r.qrow = m.row0 + i;
        r.pos = m.pos0 + i;
        r.kbase = m.kbase;
        return r;
    }
    int lo = 0, hi = m.n_seqs - 1;  // last b with cu_q[b] <= i
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (m.cu_q[mid] <= i) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    int lq = m.cu_q[b + 1] - m.cu_q[b];
    int lk = m.cu_k[b + 1] - m.cu_k[b];
    r.qrow = i;
    r.pos = lk - lq + (i - m.cu_q[b]);
    r.kbase = m.cu_k[b];
    return r;
}

// Order-preserving map of a float score to an unsigned key: larger score -> larger key,
// -0 and +0 map to the same key, every NaN maps to 0 (below -inf, whose key is 0x007fffff).
__device__ __forceinline__ uint32_t score_key(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
    if (u == 0x80000000u) u = 0u;                      // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

}  // namespace dsa
