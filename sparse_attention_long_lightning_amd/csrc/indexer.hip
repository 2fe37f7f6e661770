// Lightning indexer on gfx950: FP8 e4m3 MFMA contraction with the ReLU / head-weight /
// head-sum epilogue fused in registers.
//
// Score of query row t against key s (DeepSeek-V3.2-Exp overview, indexer formula; lightning
// indexer walk-through, steps 2 and 3):
//     I[t,s] = ks[s] * sum_j w'[t,j] * ReLU(D_j),   D_j = q8[t,j,:] . k8[s,:],   w' = w * qs
// The two FP8 scales are positive, so they factor out of the ReLU exactly.
//
// MFMA mapping (v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales, OCP e4m3 operands):
//   M = 16 indexer heads of one query token, N = 16 keys, K = 128 = the whole head dim, so one
//   instruction yields D_j for 16 heads x 16 keys.  Lane l holds key l%16 and heads
//   4*(l/16)+r (r = 0..3) of the tile, so the weighted ReLU sum over heads runs inside the
//   lane and needs only two cross-lane additions at the end.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b) {
    v4f zero = {0.f, 0.f, 0.f, 0.f};
    // cbsz = blgp = 0 selects e4m3 for both operands; scale 127 is 2^0 in E8M0.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

// Sum over the four 16-lane groups; every lane ends with the total of its column.
__device__ __forceinline__ float sum_over_groups(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

constexpr int kPrefillTokens = 8;    // query tokens per workgroup (2 per wave)
constexpr int kPrefillKeys = 512;    // keys per workgroup tile
constexpr int kPrefillThreads = 256;

// One workgroup scores kPrefillTokens consecutive query rows of one sequence against one
// span of kPrefillKeys keys.  The key span is staged in LDS once; each wave keeps the FP8
// query fragments of its two tokens in registers and sweeps the span 16 keys at a time.
template <int H, int D>
__global__ __launch_bounds__(kPrefillThreads, 2) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, float* __restrict__ scores,
    int64_t stride, int row0, int n_rows, int pos0, int kbase) {
    constexpr int NMT = (H + 15) / 16;  // 16-head M tiles per token
    constexpr int KGRP = D / 32;        // 32-byte K groups that carry data (D = 32 or 128)
    constexpr int KPITCH = D + 16;      // LDS bytes per key row (padding spreads banks)
    static_assert(D % 32 == 0 && D <= 128, "indexer head dim must be 32..128 in steps of 32");
    __shared__ __attribute__((aligned(16))) uint8_t lk[kPrefillKeys * KPITCH];
    __shared__ float lks[kPrefillKeys];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;

    const int i_first = blockIdx.x * kPrefillTokens;
    if (i_first >= n_rows) return;
    const int i_last = min(n_rows, i_first + kPrefillTokens) - 1;
    const int k0 = blockIdx.y * kPrefillKeys;
    const int pmax = pos0 + i_last;
    if (k0 > pmax) return;  // tile entirely above the causal diagonal
    const int kend = min(k0 + kPrefillKeys, pmax + 1);
    const int nk = kend - k0;
    const int nk16 = (nk + 15) & ~15;

    // Stage the key span: 16-byte pieces, zero rows past the causal end of the tile.
    constexpr int PIECES = D / 16;
    for (int e = tid; e < nk16 * PIECES; e += kPrefillThreads) {
        const int r = e / PIECES, c = e % PIECES;
        v4i val = {0, 0, 0, 0};
        if (r < nk) val = *(const v4i*)(k8 + (int64_t)(kbase + k0 + r) * D + c * 16);
        *(v4i*)(lk + r * KPITCH + c * 16) = val;
    }
    for (int r = tid; r < nk16; r += kPrefillThreads) lks[r] = r < nk ? ks[kbase + k0 + r] : 0.f;

    // Query fragments and folded head weights of this wave's two tokens.
    v8i qa[2][NMT];
    float wt[2][NMT][4];
    int tpos[2];
    int trow[2];
#pragma unroll
    for (int tok = 0; tok < 2; ++tok) {
        const int i = i_first + 2 * wv + tok;
        const bool ok = i < n_rows;
        tpos[tok] = ok ? pos0 + i : -1;
        trow[tok] = i;
        const int64_t qrow = (int64_t)(row0 + (ok ? i : 0));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const int h = mt * 16 + col;
            v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
            if (ok && h < H && grp < KGRP) {
                const uint8_t* src = q8 + (qrow * H + h) * D + grp * 32;
                const v4i lo = *(const v4i*)src;
                const v4i hi = *(const v4i*)(src + 16);
                a = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
            qa[tok][mt] = a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = mt * 16 + grp * 4 + r;
                wt[tok][mt][r] = (ok && hh < H) ? w[qrow * H + hh] * qs[qrow * H + hh] : 0.f;
            }
        }
    }
    __syncthreads();

    const int tmax = max(tpos[0], tpos[1]);
    if (tmax < k0) return;
    const int ngroups = (min(kend, tmax + 1) - k0 + 15) >> 4;
    for (int g = 0; g < ngroups; ++g) {
        // k-groups past the head dim carry zeros in A and must carry zeros in B as well:
        // 0 * (a stray NaN code) would poison the whole column.
        v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
        if (grp < KGRP) {
            const uint8_t* bp = lk + (16 * g + col) * KPITCH + grp * 32;
            const v4i blo = *(const v4i*)bp;
            const v4i bhi = *(const v4i*)(bp + 16);
            b = (v8i){blo.x, blo.y, blo.z, blo.w, bhi.x, bhi.y, bhi.z, bhi.w};
        }
        v4f acc[2][NMT];
#pragma unroll
        for (int tok = 0; tok < 2; ++tok)
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) acc[tok][mt] = mfma_fp8_16x16x128(qa[tok][mt], b);
        const int s = k0 + 16 * g + col;
        const float kscale = lks[16 * g + col];
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) part += wt[tok][mt][r] * fmaxf(acc[tok][mt][r], 0.f);
            part = sum_over_groups(part);
            if (grp == 0 && s <= tpos[tok]) scores[(int64_t)trow[tok] * stride + s] = part * kscale;
        }
    }
}

constexpr int kDecodeThreads = 256;
constexpr int kDecodeKeysPerWave = 512;
constexpr int kDecodeKeys = kDecodeKeysPerWave * (kDecodeThreads / kWave);
constexpr int kDecodeUnroll = 4;

// Decode: one query row per sequence against its whole key cache.  The work is a stream of
// 132 bytes per cached key, so each wave reads its key fragments straight from memory into
// MFMA operand registers, several 16-key groups ahead.
template <int H, int D>
__global__ __launch_bounds__(kDecodeThreads) void indexer_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, float* __restrict__ scores,
    int64_t stride, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k) {
    constexpr int NMT = (H + 15) / 16;
    constexpr int KGRP = D / 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int b = blockIdx.y;
    const int kbase = cu_k[b];
    const int nkeys = cu_k[b + 1] - kbase;
    const int qrow = cu_q[b];  // decode: exactly one query row, at position nkeys - 1
    const int s_begin = blockIdx.x * kDecodeKeys + wv * kDecodeKeysPerWave;
    if (s_begin >= nkeys) return;
    const int s_end = min(s_begin + kDecodeKeysPerWave, nkeys);

    v8i qa[NMT];
    float wt[NMT][4];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int h = mt * 16 + col;
        v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
        if (h < H && grp < KGRP) {
            const uint8_t* src = q8 + ((int64_t)qrow * H + h) * D + grp * 32;
            const v4i lo = *(const v4i*)src;
            const v4i hi = *(const v4i*)(src + 16);
            a = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
        qa[mt] = a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = mt * 16 + grp * 4 + r;
            wt[mt][r] = hh < H ? w[(int64_t)qrow * H + hh] * qs[(int64_t)qrow * H + hh] : 0.f;
        }
    }
    float* srow = scores + (int64_t)qrow * stride;
    for (int s0 = s_begin; s0 < s_end; s0 += 16 * kDecodeUnroll) {
        v8i bf[kDecodeUnroll];
        float kscale[kDecodeUnroll];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int s = s0 + 16 * u + col;
            v8i bv = {0, 0, 0, 0, 0, 0, 0, 0};
            float sc = 0.f;
            if (s < s_end) {
                if (grp < KGRP) {
                    const uint8_t* src = k8 + (int64_t)(kbase + s) * D + grp * 32;
                    const v4i lo = *(const v4i*)src;
                    const v4i hi = *(const v4i*)(src + 16);
                    bv = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
                sc = ks[kbase + s];
            }
            bf[u] = bv;
            kscale[u] = sc;
        }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const v4f acc = mfma_fp8_16x16x128(qa[mt], bf[u]);
#pragma unroll
                for (int r = 0; r < 4; ++r) part += wt[mt][r] * fmaxf(acc[r], 0.f);
            }
            part = sum_over_groups(part);
            const int s = s0 + 16 * u + col;
            if (grp == 0 && s < s_end) srow[s] = part * kscale[u];
        }
    }
}

template <int H, int D>
hipError_t launch_prefill_t(const IndexerArgs& a, int row0, int n_rows, int pos0, int kbase,
                            float* scores, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    const int pmax = pos0 + n_rows - 1;
    dim3 grid((n_rows + kPrefillTokens - 1) / kPrefillTokens, pmax / kPrefillKeys + 1);
    hipLaunchKernelGGL((indexer_prefill_kernel<H, D>), grid, dim3(kPrefillThreads), 0, st, a.q8,
                       a.q_scale, a.w, a.k8, a.k_scale, scores, a.score_stride, row0, n_rows,
                       pos0, kbase);
    return hipGetLastError();
}

template <int H, int D>
hipError_t launch_decode_t(const IndexerArgs& a, int n_seqs, int max_keys, const int32_t* cu_q,
                           const int32_t* cu_k, hipStream_t st) {
    dim3 grid((max_keys + kDecodeKeys - 1) / kDecodeKeys, n_seqs);
    hipLaunchKernelGGL((indexer_decode_kernel<H, D>), grid, dim3(kDecodeThreads), 0, st, a.q8,
                       a.q_scale, a.w, a.k8, a.k_scale, a.scores, a.score_stride, cu_q, cu_k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_prefill(const IndexerArgs& a, int row0, int n_rows, int pos0,
                                  int kbase, float* scores, hipStream_t st) {
    if (a.shape == Shape::Prod) return launch_prefill_t<64, 128>(a, row0, n_rows, pos0, kbase, scores, st);
    return launch_prefill_t<4, 32>(a, row0, n_rows, pos0, kbase, scores, st);
}

hipError_t launch_indexer_decode(const IndexerArgs& a, int n_seqs, int max_keys,
                                 const int32_t* cu_q, const int32_t* cu_k, hipStream_t st) {
    if (a.shape == Shape::Prod) return launch_decode_t<64, 128>(a, n_seqs, max_keys, cu_q, cu_k, st);
    return launch_decode_t<4, 32>(a, n_seqs, max_keys, cu_q, cu_k, st);
}

}  // namespace dsa
