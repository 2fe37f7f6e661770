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
template <class S>
__device__ void find_threshold(const uint32_t* hist, int nb, int need, S& sm) {
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

// Selects the top-k of the row x[0..n) (n > topk) into out, in position order.
__device__ void select_row(Smem& sm, const float* __restrict__ x, int n, int topk, int32_t* __restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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

__global__ __launch_bounds__(kThreads, 2) void topk_kernel(const float* __restrict__ scores,
                                                           int64_t stride, int32_t* __restrict__ idx,
                                                           int topk, RowMap map, int n_rows) {
    __shared__ Smem sm;
    const int row = blockIdx.x;
    if (row >= n_rows) return;
    const RowInfo ri = row_info(map, row);
    const int n = ri.pos + 1;
    int32_t* out = idx + (int64_t)row * topk;
    if (n <= topk) {  // every candidate is selected
        for (int j = threadIdx.x; j < topk; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    select_row(sm, scores + (int64_t)row * stride, n, topk, out);
}

// ---------------------------------------------------------------------------------------
// Segmented selection: several workgroups per row.
//
// Under the total order "larger key first, lower position first among equal keys" the
// selected set is the first k elements of the row.  An element among the first k of its
// row is also among the first k of any part of the row that holds it (fewer elements
// precede it there), so the selection equals the first k of the union of every segment's
// own first k.  The segment kernel keeps a segment of kSeg scores in LDS, reads it from
// memory once and writes its first k as (key, position) candidates in position order; the
// merge kernel selects the row's first k among at most kMaxSegs * k candidates.  Both give
// the same unique result as the single-workgroup kernel above.
constexpr int kSeg = 16384;   // scores per segment workgroup (64 KiB of keys in LDS)
constexpr int kMaxSegs = 8;   // segments per row the merge holds in LDS
// Fewer rows than this are split (one workgroup per row would leave most CUs idle); with
// more, one workgroup per row is faster, as it keeps no candidates in memory.
constexpr int kSplitRows = 128;
// Largest k of the segmented path (the merge holds kMaxSegs * k candidates in LDS).
constexpr int kSegMaxTopk = 2048;

struct SelSmem {
    uint32_t hist[kBins1];
    int wsum[kWaves];
    int wgt[kWaves], weq[kWaves];
    int sel_bin, sel_above;
    int wcnt[2];
};

// Among keys[0..m) in LDS, the kk-th largest key theta (1 <= kk <= m) and the number of
// keys above it.  Radix select over the keys' actual range [lo, hi]: each pass splits the
// current range into 2048 bins (11 bits of key - lo), so at most three passes reach a
// single key value.  keys must hold m rounded up to a multiple of 4 entries (16-byte reads).
// A caller that knows the range holding theta passes it as [lo_hint, lo_hint + lim_hint]:
// the first pass then histograms that range directly and counts the keys above it, with no
// pass for the keys' extent.  If some key lies below the range, or theta is not in it, the
// hint is dropped and the general search runs.
__device__ void lds_kth_key(const uint32_t* keys, int m, int kk, SelSmem& sm, uint32_t& theta,
                            int& above, uint32_t lo_hint = 0u, uint32_t lim_hint = 0xffffffffu) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint4* k4 = (const uint4*)keys;
    const int m4 = (m + 3) >> 2;
    uint32_t lo = 0xffffffffu, hi = 0u, lim = 0u;
    int need = kk, ab = 0;
    bool hinted = false;
    if (lim_hint != 0xffffffffu) {
        const int bits = 32 - __clz(lim_hint);
        const int sh = bits > 11 ? bits - 11 : 0;
        for (int j = tid; j < kBins1; j += kThreads) sm.hist[j] = 0u;
        __syncthreads();
        int ca = 0, cb = 0;  // keys above / below the range
        for (int i = tid; i < m4; i += kThreads) {
            const uint4 v = k4[i];
            const uint32_t k[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * i + c < m) {
                    if (k[c] < lo_hint) ++cb;
                    else if (k[c] - lo_hint > lim_hint) ++ca;
                    else atomicAdd(&sm.hist[(k[c] - lo_hint) >> sh], 1u);
                }
        }
        ca = wave_sum_i(ca);
        cb = wave_sum_i(cb);
        if (lane == 0) {
            sm.wgt[wv] = ca;
            sm.weq[wv] = cb;
        }
        __syncthreads();
        int ta = 0, tb = 0;
        for (int w = 0; w < kWaves; ++w) {
            ta += sm.wgt[w];
            tb += sm.weq[w];
        }
        if (tb == 0 && ta < kk && kk - ta <= m - ta) {
            find_threshold(sm.hist, kBins1, kk - ta, sm);  // its barriers also retire wgt / weq
            const uint32_t b = (uint32_t)sm.sel_bin;
            const int a = sm.sel_above;
            __syncthreads();
            ab = ta + a;
            need = kk - ta - a;
            lo = lo_hint + (b << sh);
            lim = min(lim_hint - (b << sh), (1u << sh) - 1u);
            hinted = true;
        } else {
            __syncthreads();  // wgt / weq are reused below
        }
    }
    if (!hinted) {
        for (int i = tid; i < m4; i += kThreads) {
            const uint4 v = k4[i];
            const uint32_t k[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * i + c < m) {
                    lo = min(lo, k[c]);
                    hi = max(hi, k[c]);
                }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
            hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
        }
        if (lane == 0) {
            sm.wgt[wv] = (int)lo;
            sm.weq[wv] = (int)hi;
        }
        __syncthreads();
        lo = 0xffffffffu;
        hi = 0u;
        for (int w = 0; w < kWaves; ++w) {
            lo = min(lo, (uint32_t)sm.wgt[w]);
            hi = max(hi, (uint32_t)sm.weq[w]);
        }
        __syncthreads();
        lim = hi - lo;
    }
    // the kk-th key lies in [lo, lo + lim]; `ab` keys lie above that range
    while (lim > 0) {
        const int bits = 32 - __clz(lim);
        const int sh = bits > 11 ? bits - 11 : 0;
        for (int j = tid; j < kBins1; j += kThreads) sm.hist[j] = 0u;
        __syncthreads();
        for (int i = tid; i < m4; i += kThreads) {
            const uint4 v = k4[i];
            const uint32_t k[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t d = k[c] - lo;
                if (4 * i + c < m && d <= lim) atomicAdd(&sm.hist[d >> sh], 1u);
            }
        }
        __syncthreads();
        find_threshold(sm.hist, kBins1, need, sm);
        const uint32_t b = (uint32_t)sm.sel_bin;
        const int a = sm.sel_above;
        __syncthreads();
        ab += a;
        need -= a;
        lo += b << sh;
        lim = min(lim - (b << sh), (1u << sh) - 1u);
    }
    theta = lo;
    above = ab;
}

// Number of set bits of ballot b in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t b) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// Emits, in position order, the keys[0..m) above theta and the first need_eq equal to it.
// Wave w owns a contiguous range of 256-element groups; lane l of a group holds its 4
// consecutive elements 4l .. 4l+3 (one 16-byte LDS read).  emit(j, key, slot) is called for
// the element j taking output slot `slot`.  keys must hold m rounded up to a multiple of 4.
template <class F>
__device__ void emit_ordered(const uint32_t* keys, int m, uint32_t theta, int need_eq, SelSmem& sm,
                             F&& emit) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint4* k4 = (const uint4*)keys;
    const int ngrp = (m + 255) >> 8;
    const int per = (ngrp + kWaves - 1) / kWaves;
    const int g0 = min(ngrp, wv * per), g1 = min(ngrp, g0 + per);
    auto load = [&](int g, uint32_t (&k)[4], bool (&in)[4]) {
        const int j = (g << 8) + 4 * lane;
        const uint4 v = j < m ? k4[j >> 2] : make_uint4(0u, 0u, 0u, 0u);
        k[0] = v.x;
        k[1] = v.y;
        k[2] = v.z;
        k[3] = v.w;
#pragma unroll
        for (int c = 0; c < 4; ++c) in[c] = j + c < m;
    };
    int gt = 0, eq = 0;
    for (int g = g0; g < g1; ++g) {
        uint32_t k[4];
        bool in[4];
        load(g, k, in);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            gt += __popcll(__ballot(in[c] && k[c] > theta));
            eq += __popcll(__ballot(in[c] && k[c] == theta));
        }
    }
    if (lane == 0) {
        sm.wgt[wv] = gt;
        sm.weq[wv] = eq;
    }
    __syncthreads();
    int eq_run = 0, out_run = 0;
    for (int w = 0; w < wv; ++w) {
        const int e = sm.weq[w];
        out_run += sm.wgt[w] + min(e, max(0, need_eq - eq_run));
        eq_run += e;
    }
    for (int g = g0; g < g1; ++g) {
        uint32_t k[4];
        bool in[4];
        load(g, k, in);
        bool e[4], sel[4];
        uint64_t be[4], bs[4];
        int r = eq_run;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            e[c] = in[c] && k[c] == theta;
            be[c] = __ballot(e[c]);
            r += lanes_below(be[c]);
        }
        int ne = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ne += __popcll(be[c]);
            sel[c] = in[c] && (k[c] > theta || (e[c] && r < need_eq));
            r += e[c] ? 1 : 0;
        }
        int slot = out_run, ns = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bs[c] = __ballot(sel[c]);
            slot += lanes_below(bs[c]);
            ns += __popcll(bs[c]);
        }
        const int j = (g << 8) + 4 * lane;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (sel[c]) emit(j + c, k[c], slot++);
        out_run += ns;
        eq_run += ne;
    }
}

// Candidates of row r, segment g: cand_key / cand_pos + (r * n_segs + g) * topk, min(topk,
// segment length) of them, in position order.
__global__ __launch_bounds__(kThreads, 2) void topk_segment_kernel(
    const float* __restrict__ scores, int64_t stride, int topk, RowMap map, int n_rows, int n_segs,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_pos) {
    __shared__ __attribute__((aligned(16))) uint32_t keys[kSeg];
    __shared__ SelSmem sm;
    const int g = blockIdx.x, row = blockIdx.y;
    if (row >= n_rows) return;
    const RowInfo ri = row_info(map, row);
    const int n = ri.pos + 1;
    const int s0 = g * kSeg;
    if (n <= topk || s0 >= n) return;  // the merge handles short rows
    const int m = min(kSeg, n - s0);
    const int tid = threadIdx.x;
    const float* x = scores + (int64_t)row * stride + s0;
    {
        // all of this thread's pieces are loaded before any is stored, so the whole segment
        // is in flight at once
        constexpr int NP = kSeg / (4 * kThreads);
        uint32_t k[NP][4];
        bool ok[NP][4];
#pragma unroll
        for (int u = 0; u < NP; ++u) load4(x, 4 * (tid + u * kThreads), m, k[u], ok[u]);
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int e = 4 * (tid + u * kThreads);
            if (ok[u][3]) *(uint4*)&keys[e] = make_uint4(k[u][0], k[u][1], k[u][2], k[u][3]);
            else
                for (int c = 0; c < 4; ++c)
                    if (ok[u][c]) keys[e + c] = k[u][c];
        }
    }
    __syncthreads();
    const int64_t base = ((int64_t)row * n_segs + g) * topk;
    uint32_t* ck = cand_key + base;
    int32_t* cp = cand_pos + base;
    if (m <= topk) {  // the whole segment is a candidate set
        for (int j = tid; j < m; j += kThreads) {
            ck[j] = keys[j];
            cp[j] = s0 + j;
        }
        return;
    }
    uint32_t theta;
    int above;
    lds_kth_key(keys, m, topk, sm, theta, above);
    emit_ordered(keys, m, theta, topk - above, sm, [&](int j, uint32_t key, int slot) {
        ck[slot] = key;
        cp[slot] = s0 + j;
    });
}

__global__ __launch_bounds__(kThreads, 1) void topk_merge_kernel(
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos, int32_t* __restrict__ idx,
    int topk, RowMap map, int n_rows, int n_segs) {
    __shared__ __attribute__((aligned(16))) uint32_t keys[kMaxSegs * kSegMaxTopk];
    __shared__ __attribute__((aligned(16))) int32_t pos[kMaxSegs * kSegMaxTopk];
    __shared__ SelSmem sm;
    const int row = blockIdx.x;
    if (row >= n_rows) return;
    const RowInfo ri = row_info(map, row);
    const int n = ri.pos + 1;
    int32_t* out = idx + (int64_t)row * topk;
    const int tid = threadIdx.x;
    if (n <= topk) {  // every candidate is selected
        for (int j = tid; j < topk; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    // every segment but the last holds exactly topk candidates (kSeg >= topk), so the row's
    // candidates are one contiguous run
    const int nseg = (n + kSeg - 1) / kSeg;
    const int total = (nseg - 1) * topk + min(topk, n - (nseg - 1) * kSeg);
    const uint32_t* ck = cand_key + (int64_t)row * n_segs * topk;
    const int32_t* cp = cand_pos + (int64_t)row * n_segs * topk;
    constexpr int U = 8;
    for (int e0 = tid; e0 < total; e0 += U * kThreads) {
        uint32_t kv[U];
        int32_t pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * kThreads;
            kv[u] = e < total ? ck[e] : 0u;
            pv[u] = e < total ? cp[e] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * kThreads;
            if (e < total) {
                keys[e] = kv[u];
                pos[e] = pv[u];
            }
        }
    }
    __syncthreads();
    uint32_t theta;
    int above;
    lds_kth_key(keys, total, topk, sm, theta, above);
    emit_ordered(keys, total, theta, topk - above, sm, [&](int j, uint32_t, int slot) { out[slot] = pos[j]; });
}

// ---------------------------------------------------------------------------------------
// Selection from an indexer-built histogram (fused indexer -> top-k).
//
// The prefill indexer counts, per query row, the scores whose key has the top bit set (the
// non-negative scores) in 1024 bins of key bits 30..21, which are exactly bins 1024..2047 of
// the first digit above.  When the row has at least k such scores, the threshold digit b1
// and the list size follow from these counts alone, so the row is read once: every element
// of digit >= b1 goes to the LDS list (in any order), digits 2 and 3 are resolved on the
// list, and the selection is put back in position order through two position bitmaps (keys
// above the threshold; ties at it, of which the lowest-positioned are taken).  Rows with
// fewer than k non-negative scores, lists beyond LDS or rows longer than the bitmaps take
// select_row.  The result is the same unique selection.
constexpr int kBitmapWords = kCap / 2;     // each bitmap takes half of the list's key array
constexpr int kFusedMaxLen = kBitmapWords * 32;

struct FusedSmem {
    uint32_t key[kCap];  // list keys; later the two position bitmaps
    int32_t pos[kCap];   // list positions; class bits 30..31 after the threshold is known
    SelSmem sel;
    int count;
};

union TopkSmem {
    Smem full;
    FusedSmem fused;
};

// The selection from a list of every candidate that can be selected (sm.key / sm.pos hold
// nlist >= topk entries in any order, every key at or above the first digit b1; n is the row
// length, at most kFusedMaxLen): digits 2 and 3 on the list give theta and the ties taken,
// then two position bitmaps give position order.
__device__ void finish_from_list(FusedSmem& sm, int nlist, int topk, int n, int b1, int32_t* __restrict__ out) {
    const int tid = threadIdx.x;
    // ---- digits 2 and 3 on the list: theta, and how many ties at theta are taken; theta has
    // first digit b1 (keys 1 << 31 | (b1 - kHistBins) << 21 and the 2^21 - 1 after it) ----
    uint32_t theta;
    int above;
    lds_kth_key(sm.key, nlist, topk, sm.sel, theta, above, 0x80000000u | ((uint32_t)(b1 - kHistBins) << 21),
                (1u << 21) - 1u);
    const int need_eq = topk - above;
    // classes: 1 = above theta, 2 = tie at theta, 0 = not selected
    for (int j = tid; j < nlist; j += kThreads) {
        const uint32_t kk = sm.key[j];
        const int cls = kk > theta ? 1 : kk == theta ? 2 : 0;
        sm.pos[j] |= cls << 30;
    }
    __syncthreads();  // the keys are dead: their array becomes the two bitmaps
    const int W = (n + 31) >> 5;
    uint32_t* bm_gt = sm.key;
    uint32_t* bm_eq = sm.key + kBitmapWords;
    for (int w = tid; w < W; w += kThreads) {
        bm_gt[w] = 0u;
        bm_eq[w] = 0u;
    }
    __syncthreads();
    for (int j = tid; j < nlist; j += kThreads) {
        const int v = sm.pos[j];
        const int cls = (int)((uint32_t)v >> 30), p = v & 0x3fffffff;
        if (cls == 1) atomicOr(&bm_gt[p >> 5], 1u << (p & 31));
        else if (cls == 2) atomicOr(&bm_eq[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    // ---- emission in position order: thread t owns bitmap words [t*per, (t+1)*per) ----
    const int per = (W + kThreads - 1) / kThreads;
    const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
    int n_gt = 0, n_eq = 0;
    for (int w = w0; w < w1; ++w) {
        n_gt += __popc(bm_gt[w]);
        n_eq += __popc(bm_eq[w]);
    }
    int t_gt, t_eq;
    int r_gt = block_exclusive_scan(n_gt, sm.sel.wsum, t_gt);
    int r_eq = block_exclusive_scan(n_eq, sm.sel.wsum, t_eq);
    for (int w = w0; w < w1; ++w) {
        const uint32_t g = bm_gt[w];
        uint32_t e = bm_eq[w];
        // keep the ties of rank < need_eq: the first (need_eq - r_eq) set bits of e
        const int keep = need_eq - r_eq;
        const int ne = __popc(e);
        if (keep <= 0) {
            e = 0u;
        } else if (keep < ne) {
            uint32_t m = e, kept = 0u;
            for (int i = 0; i < keep; ++i) {
                const uint32_t low = m & (~m + 1u);
                kept |= low;
                m ^= low;
            }
            e = kept;
        }
        r_eq += ne;
        uint32_t sel = g | e;
        int o = r_gt + min(r_eq - ne, need_eq);  // selected elements before this word
        r_gt += __popc(g);
        while (sel != 0u) {
            const int b = __builtin_ctz(sel);
            sel &= sel - 1u;
            if (o < topk) out[o] = (w << 5) + b;
            ++o;
        }
    }
}

// The first digit from a row's counts: the threshold digit b1 and the number of elements of
// digit >= b1; false when the list path does not apply (fewer than topk counted scores, more
// than kCap candidates, or a row longer than the bitmaps).  One wave does the search (lane l
// holds bins 16l .. 16l+15, suffix sums over the lanes from the top), so the only barrier is
// the one that hands the result to the other waves.  Ends with a barrier.
__device__ bool threshold_from_counts(SelSmem& sel, const uint32_t* __restrict__ h, int n, int topk, int& b1,
                                      int& nlist) {
    static_assert(kHistBins == 16 * kWave, "16 count bins per lane");
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        uint32_t c[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = *(const uint4*)(h + 16 * lane + 4 * q);
            c[4 * q] = v.x;
            c[4 * q + 1] = v.y;
            c[4 * q + 2] = v.z;
            c[4 * q + 3] = v.w;
        }
        int own = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) own += (int)c[j];
        int suf = own;  // counts of this lane's bins and of every higher lane's
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int t = __shfl_down(suf, o);
            if (lane + o < kWave) suf += t;
        }
        const int total = __shfl(suf, 0);
        // the lane whose bins hold the topk-th largest counted score (none if total < topk)
        if (lane == 0) {
            sel.sel_bin = 0;
            sel.sel_above = 0;
            sel.wcnt[0] = 0;
            sel.wcnt[1] = total;
        }
        int cum = suf - own;
        if (cum < topk && topk <= suf) {
            int bin = 16 * lane, above = cum, through = suf;
            bool found = false;
#pragma unroll
            for (int j = 15; j >= 0; --j) {
                if (!found && cum + (int)c[j] >= topk) {
                    found = true;
                    bin = 16 * lane + j;
                    above = cum;
                    through = cum + (int)c[j];
                }
                cum += (int)c[j];
            }
            sel.sel_bin = bin;
            sel.sel_above = above;
            sel.wcnt[0] = through;
        }
    }
    __syncthreads();
    const int total = sel.wcnt[1];
    bool fused = total >= topk && n <= kFusedMaxLen;
    b1 = 0;
    nlist = 0;
    if (fused) {
        b1 = kHistBins + sel.sel_bin;
        nlist = sel.wcnt[0];
        fused = nlist <= kCap;
    }
    __syncthreads();  // every thread has read the threshold before the shared memory is reused
    return fused;
}

// The float whose bits are (b1 - kHistBins) << 21: for a threshold digit b1 among the scores
// >= +0 (b1 >= kHistBins, at most +inf's digit), an element's key digit is >= b1 exactly when
// the element compares >= this float (see topk_hist_kernel).
__device__ __forceinline__ float list_threshold(int b1) { return __uint_as_float((uint32_t)(b1 - kHistBins) << 21); }

__global__ __launch_bounds__(kThreads, 2) void topk_hist_kernel(const float* __restrict__ scores, int64_t stride,
                                                                const uint32_t* __restrict__ hist,
                                                                int32_t* __restrict__ idx, int topk, RowMap map,
                                                                int n_rows) {
    __shared__ __attribute__((aligned(16))) TopkSmem smu;  // 16-byte key reads
    FusedSmem& sm = smu.fused;
    const int row = blockIdx.x;
    if (row >= n_rows) return;
    const RowInfo ri = row_info(map, row);
    const int n = ri.pos + 1;
    int32_t* out = idx + (int64_t)row * topk;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (n <= topk) {
        for (int j = tid; j < topk; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const float* x = scores + (int64_t)row * stride;
    int b1, nlist;
    const bool fused = threshold_from_counts(sm.sel, hist + (int64_t)row * kHistBins, n, topk, b1, nlist);
    if (!fused) {
        select_row(smu.full, x, n, topk, out);
        return;
    }
    // ---- one pass: every element of digit >= b1 into the list ----
    // Here b1 >= kHistBins (the threshold lies among the scores >= +0, below +inf's digit), and
    // for such digits key >> 21 >= b1 holds exactly when x >= thr, the float whose bits are
    // (b1 - kHistBins) << 21: non-negative floats order like their bits, -0 passes only when
    // thr = +0 (its key digit is kHistBins), negative scores and NaN never pass.  So the scan
    // is one float compare per element; the keys are formed for the few that pass, which are
    // placed by wave ballots (the list order is free).
    const float thr = list_threshold(b1);
    if (tid == 0) sm.count = 0;
    __syncthreads();
    const int seg = ((n + kWaves - 1) / kWaves + 255) & ~255;
    const int sb = min(n, wv * seg), se = min(n, sb + seg);
    constexpr int kStep = 256 * kUnroll;
    // loads of one step: whole steps need no bounds checks
    auto load_step = [&](int e0, bool whole, float (&v)[kUnroll][4]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = e0 + 256 * u + 4 * lane;
            if (whole || e + 3 < se) {
                const float4 t = *(const float4*)(x + e);
                v[u][0] = t.x;
                v[u][1] = t.y;
                v[u][2] = t.z;
                v[u][3] = t.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) v[u][c] = e + c < se ? x[e + c] : -INFINITY;
            }
        }
    };
    auto append_step = [&](int e0, const float (&v)[kUnroll][4]) {
        uint64_t m[kUnroll][4];
        int tot = 0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                m[u][c] = __ballot(v[u][c] >= thr);
                tot += __popcll(m[u][c]);
            }
        if (tot == 0) return;
        int base = 0;
        if (lane == 0) base = atomicAdd(&sm.count, tot);
        base = __builtin_amdgcn_readfirstlane(__shfl(base, 0));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint64_t mk = m[u][c];
                if (mk == 0) continue;
                if ((mk >> lane) & 1) {
                    const int j = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
                    if (j < kCap) {
                        sm.key[j] = score_key(v[u][c]);
                        sm.pos[j] = e0 + 256 * u + 4 * lane + c;
                    }
                }
                base += __popcll(mk);
            }
    };
    // Whole steps alternate between two register sets, the next step's loads in flight while
    // this one is appended (loads are unconditional, the last step re-read if needed, so the
    // wait before each append is for the older set only); then the tail.
    const int nsteps = (se - sb) / kStep;
    int e0 = sb + nsteps * kStep;
    if (nsteps > 0) {
        float va[kUnroll][4], vb[kUnroll][4];
        load_step(sb, true, va);
        for (int i = 0; i < nsteps; i += 2) {
            load_step(sb + min(i + 1, nsteps - 1) * kStep, true, vb);
            append_step(sb + i * kStep, va);
            if (i + 1 >= nsteps) break;
            load_step(sb + min(i + 2, nsteps - 1) * kStep, true, va);
            append_step(sb + (i + 1) * kStep, vb);
        }
    }
    if (e0 < se) {
        float v[kUnroll][4];
        load_step(e0, false, v);
        append_step(e0, v);
    }
    __syncthreads();
    finish_from_list(sm, nlist, topk, n, b1, out);
}

// Few long rows (decode): the list path split over segment workgroups.  Every workgroup of a
// row finds the row's threshold digit from the counts and appends the elements of its kSeg
// scores that reach it to the row's list in global memory (in any order, one global atomic
// per workgroup); topk_list_finish_kernel then selects from the list with one workgroup
// per row.  A row the list path does not apply to is left to the finish kernel's select_row.
__global__ __launch_bounds__(kThreads, 2) void topk_list_append_kernel(const float* __restrict__ scores,
                                                                       int64_t stride,
                                                                       const uint32_t* __restrict__ hist,
                                                                       int topk, RowMap map, int n_rows,
                                                                       uint32_t* __restrict__ lkey,
                                                                       int32_t* __restrict__ lpos,
                                                                       int* __restrict__ lcount) {
    __shared__ SelSmem sel;
    const int row = blockIdx.y;
    if (row >= n_rows) return;
    const int n = row_info(map, row).pos + 1;
    const int s0 = blockIdx.x * kSeg;
    if (n <= topk || s0 >= n) return;
    const float* x = scores + (int64_t)row * stride;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    constexpr int kPerWave = kSeg / kWaves;  // whole steps of 256 * kUnroll elements
    constexpr int kSteps = kPerWave / (256 * kUnroll);
    static_assert(kPerWave % (256 * kUnroll) == 0, "whole steps per wave");
    const int sb = min(n, s0 + wv * kPerWave), se = min(n, sb + kPerWave);
    // the wave's scores stay in registers: they are counted first, so that the workgroup
    // reserves its list space with one atomic (atomics of many waves on one row's counter
    // serialize), then placed.  They are loaded before the threshold is known, so the row's
    // count read and the score reads are in flight together.
    float v[kSteps][kUnroll][4];
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = sb + 256 * (kUnroll * st + u) + 4 * lane;
            if (e + 3 < se) {
                const float4 t = *(const float4*)(x + e);
                v[st][u][0] = t.x;
                v[st][u][1] = t.y;
                v[st][u][2] = t.z;
                v[st][u][3] = t.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) v[st][u][c] = e + c < se ? x[e + c] : -INFINITY;
            }
        }
    int b1, nlist;
    if (!threshold_from_counts(sel, hist + (int64_t)row * kHistBins, n, topk, b1, nlist)) return;
    const float thr = list_threshold(b1);
    int cnt = 0;
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) cnt += __popcll(__ballot(v[st][u][c] >= thr));
    __shared__ int wave_cnt[kWaves];
    __shared__ int wg_base;
    if (lane == 0) wave_cnt[wv] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        int tot = 0;
        for (int w = 0; w < kWaves; ++w) tot += wave_cnt[w];
        wg_base = tot > 0 ? atomicAdd(&lcount[row], tot) : 0;
    }
    __syncthreads();
    if (cnt == 0) return;
    int base = wg_base;
    for (int w = 0; w < wv; ++w) base += wave_cnt[w];
    base = __builtin_amdgcn_readfirstlane(base);
    uint32_t* rkey = lkey + (int64_t)row * kCap;
    int32_t* rpos = lpos + (int64_t)row * kCap;
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool pass = v[st][u][c] >= thr;
                const uint64_t mk = __ballot(pass);
                if (mk == 0) continue;
                if (pass) {
                    const int j = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
                    if (j < kCap) {  // the counts bound the list by nlist <= kCap
                        rkey[j] = score_key(v[st][u][c]);
                        rpos[j] = sb + 256 * (kUnroll * st + u) + 4 * lane + c;
                    }
                }
                base += __popcll(mk);
            }
}

__global__ __launch_bounds__(kThreads, 2) void topk_list_finish_kernel(const float* __restrict__ scores,
                                                                       int64_t stride,
                                                                       const uint32_t* __restrict__ hist,
                                                                       int32_t* __restrict__ idx, int topk,
                                                                       RowMap map, int n_rows,
                                                                       const uint32_t* __restrict__ lkey,
                                                                       const int32_t* __restrict__ lpos) {
    __shared__ __attribute__((aligned(16))) TopkSmem smu;
    FusedSmem& sm = smu.fused;
    const int row = blockIdx.x;
    if (row >= n_rows) return;
    const int n = row_info(map, row).pos + 1;
    int32_t* out = idx + (int64_t)row * topk;
    const int tid = threadIdx.x;
    if (n <= topk) {
        for (int j = tid; j < topk; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const float* x = scores + (int64_t)row * stride;
    int b1, nlist;
    if (!threshold_from_counts(sm.sel, hist + (int64_t)row * kHistBins, n, topk, b1, nlist)) {
        select_row(smu.full, x, n, topk, out);
        return;
    }
    // every load of the list is issued before the first is used (a plain loop would wait for
    // each round trip in turn)
    constexpr int kPer = kCap / kThreads;
    uint32_t kk[kPer];
    int32_t pp[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = tid + i * kThreads;
        if (j < nlist) {
            kk[i] = lkey[(int64_t)row * kCap + j];
            pp[i] = lpos[(int64_t)row * kCap + j];
        }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = tid + i * kThreads;
        if (j < nlist) {
            sm.key[j] = kk[i];
            sm.pos[j] = pp[i];
        }
    }
    __syncthreads();
    finish_from_list(sm, nlist, topk, n, b1, out);
}

}  // namespace

// [list sizes (n_rows ints, padded to 16 bytes) | keys (n_rows x kCap) | positions (n_rows x kCap)]
static size_t list_sizes_bytes(int n_rows) { return ((size_t)n_rows * sizeof(int) + 15) & ~(size_t)15; }

size_t topk_list_ws_bytes(int n_rows) {
    return n_rows <= 0 ? 0
                       : list_sizes_bytes(n_rows) + (size_t)n_rows * kCap * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_topk_list(const float* scores, int64_t stride, const uint32_t* hist, int32_t* idx, int topk,
                            const RowMap& map, int n_rows, int max_len, void* ws, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    int* lcount = (int*)ws;
    uint32_t* lkey = (uint32_t*)((uint8_t*)ws + list_sizes_bytes(n_rows));
    int32_t* lpos = (int32_t*)(lkey + (size_t)n_rows * kCap);
    hipLaunchKernelGGL(topk_list_append_kernel, dim3((max_len + kSeg - 1) / kSeg, n_rows), dim3(kThreads), 0, st,
                       scores, stride, hist, topk, map, n_rows, lkey, lpos, lcount);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_list_finish_kernel, dim3(n_rows), dim3(kThreads), 0, st, scores, stride, hist, idx,
                       topk, map, n_rows, lkey, lpos);
    return hipGetLastError();
}

int topk_segments(int max_len) { return (max_len + kSeg - 1) / kSeg; }

size_t topk_ws_bytes(int n_rows, int max_len, int topk) {
    const int ns = topk_segments(max_len);
    if (ns > kMaxSegs || n_rows <= 0 || n_rows >= kSplitRows || topk > kSegMaxTopk) return 0;
    return (size_t)n_rows * ns * topk * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_topk_from_hist(const float* scores, int64_t stride, const uint32_t* hist, int32_t* idx,
                                 int topk, const RowMap& map, int n_rows, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_hist_kernel, dim3(n_rows), dim3(kThreads), 0, st, scores, stride, hist, idx, topk, map,
                       n_rows);
    return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t stride, int32_t* idx, int topk,
                       const RowMap& map, int n_rows, int max_len, void* ws, size_t ws_bytes,
                       hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    const size_t need = topk_ws_bytes(n_rows, max_len, topk);
    if (need == 0 || ws == nullptr || ws_bytes < need) {
        hipLaunchKernelGGL(topk_kernel, dim3(n_rows), dim3(kThreads), 0, st, scores, stride, idx, topk,
                           map, n_rows);
        return hipGetLastError();
    }
    const int ns = topk_segments(max_len);
    uint32_t* ck = (uint32_t*)ws;
    int32_t* cp = (int32_t*)(ck + (size_t)n_rows * ns * topk);
    hipLaunchKernelGGL(topk_segment_kernel, dim3(ns, n_rows), dim3(kThreads), 0, st, scores, stride, topk,
                       map, n_rows, ns, ck, cp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(n_rows), dim3(kThreads), 0, st, ck, cp, idx, topk, map,
                       n_rows, ns);
    return hipGetLastError();
}

}  // namespace dsa
