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
constexpr int kMaxTopk = 8192;  // largest k accepted (k = 2048 in the DeepSeek-V3.2-Exp shape)

// Maps a query row to its sequence, absolute position and key-row base.
//  single-sequence mode (cu_q == nullptr): row i -> position pos0 + i, key base kbase,
//      query row row0 + i of the packed query arrays;
//  batch mode: row i is a global query row; its sequence b is found in cu_q.
//  paged caches (pages != nullptr): position p of sequence s is cache row
//      pages[s * pages_per_seq + p / kPage] * kPage + p % kPage
//  of a pool of pool_rows rows (0: not given, page ids are then trusted).
//  one_row_per_seq (batch mode, set by the host only when every sequence has exactly one
//      query row, so cu_q[b] = b): row i is sequence i, found without searching cu_q.
struct RowMap {
    const int32_t* cu_q;
    const int32_t* cu_k;
    int n_seqs;
    int row0;
    int pos0;
    int kbase;
    const int32_t* pages = nullptr;
    int pages_per_seq = 0;
    int64_t pool_rows = 0;
    bool one_row_per_seq = false;
};

constexpr int kPage = 64;  // positions per cache page

struct RowInfo {
    int qrow;   // packed query row
    int pos;    // absolute position p (keys 0..p)
    int kbase;  // packed key row of position 0
    int seq;    // sequence of the row
    int lim;    // largest position an index slot may name: len_k - 1 of the row's sequence in
                // batch mode, p in single-sequence mode (whose index rows the top-k wrote)
};

// Cache row of position p of the row's sequence.
__device__ __forceinline__ int64_t cache_row(const RowMap& m, const RowInfo& r, int p) {
    if (m.pages == nullptr) return (int64_t)r.kbase + p;
    return (int64_t)m.pages[(int64_t)r.seq * m.pages_per_seq + p / kPage] * kPage + p % kPage;
}

__device__ __forceinline__ RowInfo row_info(const RowMap& m, int i) {
    RowInfo r;
    if (m.cu_q == nullptr) {
        r.qrow = m.row0 + i;
        r.pos = m.pos0 + i;
        r.kbase = m.kbase;
        r.seq = 0;
        r.lim = r.pos;
        return r;
    }
    int b, lq, q0;
    if (m.one_row_per_seq) {  // decode batches: no chain of dependent loads through cu_q
        b = i;
        lq = 1;
        q0 = i;
    } else {
        int lo = 0, hi = m.n_seqs - 1;  // last b with cu_q[b] <= i
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (m.cu_q[mid] <= i) lo = mid; else hi = mid - 1;
        }
        b = lo;
        q0 = m.cu_q[b];
        lq = m.cu_q[b + 1] - q0;
    }
    const int lk = m.cu_k[b + 1] - m.cu_k[b];
    r.qrow = i;
    r.pos = lk - lq + (i - q0);
    r.kbase = m.cu_k[b];
    r.seq = b;
    r.lim = lk - 1;
    return r;
}

// Cache row that index slot value id names for the row, or -1 when the slot is empty or its
// value cannot be loaded: -1 and every value outside [0, lim], and with paged caches of known
// pool size a page id outside the pool.  Gathers load only rows this returns, so an index row
// with out-of-range entries can never make them read outside the caches.
__device__ __forceinline__ int64_t slot_row(const RowMap& m, const RowInfo& r, int id) {
    if ((unsigned)id > (unsigned)r.lim) return -1;
    const int64_t row = cache_row(m, r, id);
    if (m.pages != nullptr && m.pool_rows > 0 && (row < 0 || row >= m.pool_rows)) return -1;
    return row;
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


// ---- LDS and direct global->LDS helpers ----

typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

typedef __attribute__((address_space(3))) v4i lds_v4i;

// LDS accesses by 32-bit LDS byte address (a uniform buffer base plus a per-lane offset, so a
// read costs one add and constant parts ride in the instruction's offset field).
__device__ __forceinline__ v4s ds_read_tr16(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(size_t)a);
}
__device__ __forceinline__ v4i lds_read16(uint32_t a) { return *(const lds_v4i*)(size_t)a; }
__device__ __forceinline__ void lds_write16(uint32_t a, v4i v) { *(lds_v4i*)(size_t)a = v; }

// Workgroup barrier that orders LDS accesses only: in-flight direct global->LDS loads into
// the other buffers are not waited for (the fence of a full __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves above the barrier
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}


// One direct global->LDS load of 16 bytes per lane from base + off: lane i's bytes land at
// lds_base + 16 * i.  Issued from asm so that the compiler's wait-count bookkeeping does not
// see it: as a FLAT access that touches LDS it would otherwise turn every later LDS wait into
// a full drain.  Completion is tracked by hand with wait_loads (the load counts on vmcnt only)
// and a barrier before any other wave reads the bytes.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; the clobber still orders it
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_base), "v"(off), "s"(base)
        : "memory", "m0");
}
// The same from a full 64-bit address per lane (no scalar base): for rows beyond 4 GiB of
// the base, e.g. in a large page pool.
__device__ __forceinline__ void dma16_at(const void* addr, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_base), "v"(addr)
        : "memory", "m0");
}
// The same with 4 bytes per lane: lane i's dword lands at lds_base + 4 * i.
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2"
        :
        : "s"(lds_base), "v"(off), "s"(base)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N vector memory operations of this wave are still in flight.  Loads
// complete in issue order, so waiting down to the number of loads issued after a given one
// guarantees that one has landed; stores also count here but may finish out of order, so a
// caller counts only younger loads (younger stores can only make the wait longer).
template <int N>
__device__ __forceinline__ void wait_loads() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace dsa
