// Per-query top-k selection on gfx950 (fine-grained token selection of DSA: keep the k
// positions with the largest index scores; DeepSeek-V3.2-Exp deep dive, section 2.2, and
// lightning-indexer walk-through, step 4).
//
// One workgroup of 512 threads selects one row.  Scores become order-preserving 32-bit keys
// (larger score -> larger key, -0 == +0, NaN lowest) and the k-th largest key is found by a
// radix select over three digits (11, 11 and 10 bits):
//   pass 1  streams the row once and builds a per-wave histogram of the top digit in LDS;
//           the threshold digit b1 and, per wave, the number of elements at or above it
//           follow from the histograms;
//   pass 2  streams the row again and compacts every element at or above b1 into an LDS
//           list, in position order (each wave owns a contiguous segment and knows its
//           output offset from pass 1);
//   the remaining two digits are resolved on that list inside LDS, and the list is emitted
//   in position order: keys above the threshold, plus the lowest-positioned ties at the
//   threshold until k are taken.
// Rows whose list would not fit in LDS (huge tie groups, e.g. constant rows) take a slower
// path that resolves the remaining digits with more passes over the row.  Both paths give
// the unique result, so the output is deterministic and bit-exact.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins1 = 2048;  // key bits 31..21
constexpr int kBins2 = 2048;  // key bits 20..10
constexpr int kBins3 = 1024;  // key bits 9..0
constexpr int kCap = 8192;    // list entries held in LDS
constexpr int kUnroll = 4;    // 256-element pieces per wave and loop iteration

struct Smem {
    union {
        uint32_t hist_w[kWaves][kBins1];
        struct {
            uint32_t key[kCap];
            int32_t pos[kCap];
        } cand;
        uint32_t hist3_w[kWaves][kBins3];
    } u;
    uint32_t hist[kBins2];
    int wsum[kWaves];
    int wcnt[kWaves];
    int wcnt2[kWaves];
    int sel_bin, sel_above;
};

__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int s = wsum[i];
        base += (i < w) ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + incl - v;
}

// Finds bin b of an LDS histogram with count(bins > b) < need <= count(bins >= b).
// Requires 1 <= need <= total count.  Result in sm.sel_bin / sm.sel_above.
__device__ void find_threshold(const uint32_t* hist, int nb, int need, Smem& sm) {
    if (threadIdx.x == 0) {  // defined result even if no bin qualifies (ordered by the scan's barrier)
        sm.sel_bin = 0;
        sm.sel_above = 0;
    }
    const int per = nb / kThreads;
    const int top = nb - 1 - threadIdx.x * per;
    int s = 0;
    for (int j = 0; j < per; ++j) s += (int)hist[top - j];
    int total;
    const int before = block_exclusive_scan(s, sm.wsum, total);
    if (before < need && need <= before + s) {
        int cum = before;
        for (int j = 0; j < per; ++j) {
            const int c = (int)hist[top - j];
            if (cum + c >= need) {
                sm.sel_bin = top - j;
                sm.sel_above = cum;
                break;
            }
            cum += c;
        }
    }
    __syncthreads();
}

// Loads elements e..e+3 of the row (e is a multiple of 4); entries at or past `end` are
// marked invalid and never read.
__device__ __forceinline__ void load4(const float* __restrict__ x, int e, int end, uint32_t k[4],
                                      bool ok[4]) {
    if (e + 3 < end) {
        const float4 v = *(const float4*)(x + e);
        k[0] = score_key(v.x);
        k[1] = score_key(v.y);
        k[2] = score_key(v.z);
        k[3] = score_key(v.w);
        ok[0] = ok[1] = ok[2] = ok[3] = true;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ok[c] = e + c < end;
            k[c] = ok[c] ? score_key(x[e + c]) : 0u;
        }
    }
}

// Ordered compaction inside one wave: lane l contributes the flagged entries among its four
// consecutive elements; returns this lane's first output slot and the wave total.
__device__ __forceinline__ int wave_slot(int f, int& total) {
    const int incl = wave_inclusive_scan(f);
    total = __shfl(incl, 63);
    return incl - f;
}

__global__ __launch_bounds__(kThreads, 2) void topk_kernel(const float* __restrict__ scores,
                                                           int64_t stride, int32_t* __restrict__ idx,
                                                           int topk, RowMap map, int n_rows) {
    __shared__ Smem sm;
    const int row = blockIdx.x;
    if (row >= n_rows) return;
    const RowInfo ri = row_info(map, row);
    const int n = ri.pos + 1;
    int32_t* out = idx + (int64_t)row * topk;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (n <= topk) {  // every candidate is selected
        for (int j = tid; j < topk; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const float* x = scores + (int64_t)row * stride;
    const int seg = ((n + kWaves - 1) / kWaves + 255) & ~255;
    const int sb = min(n, wv * seg), se = min(n, sb + seg);

    // ---- pass 1: per-wave histograms of the top digit ----
    for (int j = tid; j < kWaves * kBins1; j += kThreads) (&sm.u.hist_w[0][0])[j] = 0u;
    __syncthreads();
    uint32_t* hw = sm.u.hist_w[wv];
    // kUnroll pieces per lane are loaded before any is used, so each wave keeps kUnroll KiB
    // in flight (the row streams from HBM at the memory latency otherwise)
    for (int e0 = sb; e0 < se; e0 += 256 * kUnroll) {
        uint32_t k[kUnroll][4];
        bool ok[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) load4(x, e0 + 256 * u + 4 * lane, se, k[u], ok[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (ok[u][c]) atomicAdd(&hw[k[u][c] >> 21], 1u);
    }
    __syncthreads();
    for (int b = tid; b < kBins1; b += kThreads) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sm.u.hist_w[w][b];
        sm.hist[b] = s;
    }
    __syncthreads();
    find_threshold(sm.hist, kBins1, topk, sm);
    const int b1 = sm.sel_bin;
    const int above1 = sm.sel_above;
    const int nlist = above1 + (int)sm.hist[b1];
    {
        int c = 0;
        for (int b = b1 + lane; b < kBins1; b += 64) c += (int)hw[b];
        c = wave_sum_i(c);
        if (lane == 0) sm.wcnt[wv] = c;
    }
    __syncthreads();
    const int need = topk - above1;  // taken from digit b1, >= 1

    if (nlist <= kCap) {
        // ---- pass 2: compact everything at or above b1, in position order ----
        int run = 0;
        for (int w = 0; w < wv; ++w) run += sm.wcnt[w];
        for (int e00 = sb; e00 < se; e00 += 256 * kUnroll) {
            uint32_t kk4[kUnroll][4];
            bool ok4[kUnroll][4];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) load4(x, e00 + 256 * u + 4 * lane, se, kk4[u], ok4[u]);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {  // pieces in position order
                const uint32_t* k = kk4[u];
                const bool* ok = ok4[u];
                const int e = e00 + 256 * u + 4 * lane;
                int f = 0;
                bool q[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    q[c] = ok[c] && (int)(k[c] >> 21) >= b1;
                    f += q[c];
                }
                if (__ballot(f > 0) == 0ull) continue;
                int total;
                int j = run + wave_slot(f, total);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (q[c]) {
                        if (j < kCap) {
                            sm.u.cand.key[j] = k[c];
                            sm.u.cand.pos[j] = e + c;
                        }
                        ++j;
                    }
                run += total;
            }
        }
        for (int b = tid; b < kBins2; b += kThreads) sm.hist[b] = 0u;
        __syncthreads();
        // ---- digit 2 on the list ----
        for (int j = tid; j < nlist; j += kThreads) {
            const uint32_t kk = sm.u.cand.key[j];
            if ((int)(kk >> 21) == b1) atomicAdd(&sm.hist[(kk >> 10) & 2047u], 1u);
        }
        __syncthreads();
        find_threshold(sm.hist, kBins2, need, sm);
        const int b2 = sm.sel_bin;
        const int need2 = need - sm.sel_above;
        const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
        for (int b = tid; b < kBins3; b += kThreads) sm.hist[b] = 0u;
        __syncthreads();
        // ---- digit 3 on the list ----
        for (int j = tid; j < nlist; j += kThreads) {
            const uint32_t kk = sm.u.cand.key[j];
            if ((kk >> 10) == pre) atomicAdd(&sm.hist[kk & 1023u], 1u);
        }
        __syncthreads();
        find_threshold(sm.hist, kBins3, need2, sm);
        const uint32_t theta = (pre << 10) | (uint32_t)sm.sel_bin;
        const int need_eq = need2 - sm.sel_above;  // ties at theta, lowest positions first
        // ---- emission in position order ----
        const int E = (nlist + kThreads - 1) / kThreads;
        const int j0 = min(nlist, tid * E), j1 = min(nlist, j0 + E);
        int eq = 0;
        for (int j = j0; j < j1; ++j) eq += sm.u.cand.key[j] == theta;
        int total;
        const int eq_before = block_exclusive_scan(eq, sm.wsum, total);
        int sel = 0;
        {
            int r = eq_before;
            for (int j = j0; j < j1; ++j) {
                const uint32_t kk = sm.u.cand.key[j];
                sel += (kk > theta) || (kk == theta && r < need_eq);
                r += kk == theta;
            }
        }
        int o = block_exclusive_scan(sel, sm.wsum, total);
        int r = eq_before;
        for (int j = j0; j < j1; ++j) {
            const uint32_t kk = sm.u.cand.key[j];
            if ((kk > theta) || (kk == theta && r < need_eq)) {
                if (o < topk) out[o] = sm.u.cand.pos[j];
                ++o;
            }
            r += kk == theta;
        }
        return;
    }

    // ---- fallback: resolve digits 2 and 3 with more passes over the row ----
    for (int b = tid; b < kBins2; b += kThreads) sm.hist[b] = 0u;
    __syncthreads();
    for (int e0 = sb; e0 < se; e0 += 256) {
        uint32_t k[4];
        bool ok[4];
        load4(x, e0 + 4 * lane, se, k, ok);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (ok[c] && (int)(k[c] >> 21) == b1) atomicAdd(&sm.hist[(k[c] >> 10) & 2047u], 1u);
    }
    __syncthreads();
    find_threshold(sm.hist, kBins2, need, sm);
    const int b2 = sm.sel_bin;
    const int need2 = need - sm.sel_above;
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    for (int j = tid; j < kWaves * kBins3; j += kThreads) (&sm.u.hist3_w[0][0])[j] = 0u;
    __syncthreads();
    int gt = 0;
    uint32_t* h3 = sm.u.hist3_w[wv];
    for (int e0 = sb; e0 < se; e0 += 256) {
        uint32_t k[4];
        bool ok[4];
        load4(x, e0 + 4 * lane, se, k, ok);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (!ok[c]) continue;
            const uint32_t kp = k[c] >> 10;
            if (kp > pre) ++gt;
            else if (kp == pre) atomicAdd(&h3[k[c] & 1023u], 1u);
        }
    }
    gt = wave_sum_i(gt);
    if (lane == 0) sm.wcnt[wv] = gt;
    __syncthreads();
    for (int b = tid; b < kBins3; b += kThreads) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sm.u.hist3_w[w][b];
        sm.hist[b] = s;
    }
    __syncthreads();
    find_threshold(sm.hist, kBins3, need2, sm);
    const int b3 = sm.sel_bin;
    const uint32_t theta = (pre << 10) | (uint32_t)b3;
    const int need_eq = need2 - sm.sel_above;
    {
        int c = 0;
        for (int b = b3 + 1 + lane; b < kBins3; b += 64) c += (int)h3[b];
        c = wave_sum_i(c);
        if (lane == 0) {
            sm.wcnt[wv] += c;          // keys strictly above theta in this wave's segment
            sm.wcnt2[wv] = (int)h3[b3];  // keys equal to theta in this wave's segment
        }
    }
    __syncthreads();
    int base = 0, ties_before = 0;
    for (int w = 0; w < wv; ++w) {
        const int take = min(max(need_eq - ties_before, 0), sm.wcnt2[w]);
        base += sm.wcnt[w] + take;
        ties_before += sm.wcnt2[w];
    }
    const int take_me = min(max(need_eq - ties_before, 0), sm.wcnt2[wv]);
    int run = base, tie_run = 0;
    for (int e0 = sb; e0 < se; e0 += 256) {
        uint32_t k[4];
        bool ok[4];
        const int e = e0 + 4 * lane;
        load4(x, e, se, k, ok);
        int teq = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) teq += ok[c] && k[c] == theta;
        int ttot;
        int tr = tie_run + wave_slot(teq, ttot);
        bool q[4];
        int f = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool is_eq = ok[c] && k[c] == theta;
            q[c] = ok[c] && (k[c] > theta || (is_eq && tr < take_me));
            tr += is_eq;
            f += q[c];
        }
        tie_run += ttot;
        int total;
        int j = run + wave_slot(f, total);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (q[c]) {
                if (j < topk) out[j] = e + c;
                ++j;
            }
        run += total;
    }
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t stride, int32_t* idx, int topk,
                       const RowMap& map, int n_rows, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(n_rows), dim3(kThreads), 0, st, scores, stride, idx, topk,
                       map, n_rows);
    return hipGetLastError();
}

}  // namespace dsa
