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
//
// Linear part on the matrix cores (prefill): with ReLU(x) = (x + |x|) / 2,
//     sum_j w'_j ReLU(D_j) = sum_j (w'_j/2) |D_j| + k8[s,:] . u,   u = sum_j (w'_j/2) q8[t,j,:]
// The second term is linear in the key, so it is one more dot product per (t, s) instead of
// one more FMA per head.  u (fp32, per token) is written as a sum of kLinTerms FP8 vectors
// u = sum_i 2^(E-7-4i) c_i (E = exponent of max|u|; each term takes the rounding residual of
// the ones before, |u - sum| <= 2^-4*kLinTerms * max|u|), and one extra MFMA per 16-key group,
// whose A rows are the terms of the wave's two tokens, gives k8 . c_i for all of them.  The
// epilogue is then one FMA per head instead of two.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b) {
    v4f zero = {0.f, 0.f, 0.f, 0.f};
    // cbsz = blgp = 0 selects e4m3 for both operands; scale 127 is 2^0 in E8M0.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

// Forces a loaded value to be present in registers at this point of the program.
__device__ __forceinline__ void materialize(const v8i& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void materialize(float x) { asm volatile("" ::"v"(x)); }

// The decode epilogue takes p + w * ReLU(x) as two FMAs, w/2 * x and w/2 * |x|, using
// ReLU(x) = (x + |x|) / 2 with the 1/2 folded into w: max-based forms cost an extra
// instruction to quiet the MFMA output first.  The two terms cancel to within fp32 rounding
// of |w x| for x < 0, far below the FP8 products' own error.  (Prefill moves the x terms onto
// the matrix cores, see above.)

// x from the lane that DPP control CTRL names (row_mirror, row_half_mirror, quad_perm).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within each row of 16
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each half row
constexpr int kDppQuadReverse = 0x1B;     // quad_perm [3,2,1,0]: i <-> i ^ 3
constexpr int kDppQuadSwap = 0xB1;        // quad_perm [1,0,3,2]: i <-> i ^ 1

// One reduce-scatter step over lane pairs (partners differ in the bit `upper`): each lane keeps
// half of its 2N values (the upper half if `upper`) and adds the partner's copy of that half.
template <int N, int CTRL>
__device__ __forceinline__ void reduce_half(float* v, bool upper) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float keep = upper ? v[i + N] : v[i];
        const float send = upper ? v[i] : v[i + N];
        v[i] = keep + dpp_f<CTRL>(send);
    }
}

constexpr int kLinTerms = 6;  // FP8 terms of the linear-part query (at most 8 rows per token)

// Sum over the four 16-lane groups; every lane ends with the total of its column.
__device__ __forceinline__ float sum_over_groups(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

constexpr int kIxTokens = 24;    // query tokens per workgroup (2 per wave)
constexpr int kIxThreads = 768;  // 12 waves: three per SIMD, so one wave's epilogue runs under
                                 // the other's MFMAs
constexpr int kIxWaves = kIxThreads / kWave;
constexpr int kIxTile = 256;     // keys per LDS tile
constexpr int kIxSeg = 8192;     // keys per workgroup: a run of tiles through a 3-deep ring
constexpr int kIxBufs = 3;
static_assert(kIxSeg % kIxTile == 0 && kIxSeg < 65536, "whole tiles; a segment's counts fit 16-bit bins");

// LDS image of one key tile: kIxTile rows of D FP8 bytes, 16-byte chunks XOR-swizzled per row
// (the direct loads write 1 KiB contiguous pieces, so the swizzle is applied to which global
// chunk each lane fetches), followed by the tile's kIxTile key scales.
template <int D>
struct IxTile {
    static constexpr int CH = D / 16;                    // chunks per key row
    static constexpr int ROWS_PER_INSTR = 64 / CH;
    static constexpr int KEY_INSTRS = kIxTile * D / 1024;
    static constexpr int KEY_BYTES = kIxTile * D;
    static constexpr int BYTES = KEY_BYTES + kIxTile * 4;
    static constexpr int SCALE_INSTRS = kIxTile / 64;    // 4-byte loads of the key scales
    static constexpr int INSTRS = KEY_INSTRS + SCALE_INSTRS;
    static constexpr int PER_WAVE = (INSTRS + kIxWaves - 1) / kIxWaves;
    // 8 consecutive rows read at one logical chunk fall in distinct 16-byte bank groups (a
    // 128-byte row spans all of them, so row r's chunks rotate by r mod 8).  Rotating pairs of
    // rows instead, which keeps 16 rows apart in 64-bank terms, measured 1% slower.
    __device__ static __forceinline__ int swz(int r) { return r & (CH - 1); }
    __device__ static __forceinline__ int chunk(int r, int c) { return r * D + 16 * (c ^ swz(r)); }
};

// One workgroup scores kIxTokens consecutive query rows of one sequence against one segment
// of kIxSeg keys.  The segment streams through LDS one kIxTile-key tile at a time with direct
// global->LDS loads two tiles ahead; each wave keeps the FP8 query fragments of its two tokens
// in registers and sweeps each tile 16 keys at a time.
template <int H, int D>
__global__ __launch_bounds__(kIxThreads, 1) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, float* __restrict__ scores,
    int64_t stride, int row0, int n_rows, int pos0, int kbase, uint32_t* __restrict__ hist) {
    using T = IxTile<D>;
    constexpr int NMT = (H + 15) / 16;  // 16-head M tiles per token
    constexpr int KGRP = D / 32;        // 32-byte K groups that carry data (D = 32 or 128)
    static_assert(D % 32 == 0 && D <= 128, "indexer head dim must be 32..128 in steps of 32");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kIxBufs * T::BYTES];
    // per token of the workgroup, counts of the stored non-negative scores by key bits 30..21
    // (top-k's first digit, upper half), two 16-bit bins per word; at most kIxSeg per bin
    __shared__ uint32_t hcount[kIxTokens][kHistBins / 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int grp = lane >> 4;

    const int i_first = blockIdx.x * kIxTokens;
    if (i_first >= n_rows) return;
    const int i_last = min(n_rows, i_first + kIxTokens) - 1;
    const int seg0 = blockIdx.y * kIxSeg;
    const int pmax = pos0 + i_last;
    if (seg0 > pmax) return;  // segment entirely above the causal diagonal
    const int seg_end = min(seg0 + kIxSeg, pmax + 1);
    const int ntiles = (seg_end - seg0 + kIxTile - 1) / kIxTile;
    if (hist != nullptr) {  // each wave clears the counts of its own two tokens
        uint32_t* hc = &hcount[2 * wv][0];
        for (int j = lane; j < kHistBins; j += kWave) hc[j] = 0u;
    }

    // Query fragments and folded head weights of this wave's two tokens.  Every load is
    // issued unconditionally from a clamped (valid) address and masked afterwards, so they
    // all fly together instead of one branch-guarded round trip at a time.
    v8i qa[2][NMT];
    float wt[2][NMT][4];
    float wa[2][NMT];  // w'/2 of the head of lane's A row (head mt*16 + col)
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
            const bool qv = ok && h < H && grp < KGRP;
            const uint8_t* src = q8 + (qrow * H + min(h, H - 1)) * D + min(grp, KGRP - 1) * 32;
            const v4i lo = *(const v4i*)src;
            const v4i hi = *(const v4i*)(src + 16);
            const v8i a = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            qa[tok][mt] = qv ? a : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
            {
                const int64_t e = qrow * H + min(h, H - 1);
                const float v = 0.5f * w[e] * qs[e];
                wa[tok][mt] = (ok && h < H) ? v : 0.f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = mt * 16 + grp * 4 + r;
                const int64_t e = qrow * H + min(hh, H - 1);
                const float v = 0.5f * w[e] * qs[e];  // halved: ReLU(x) = (x + |x|) / 2
                wt[tok][mt][r] = (ok && hh < H) ? v : 0.f;
            }
        }
    }
    const int tmax = max(tpos[0], tpos[1]);
    // The query loads complete here, before any direct load is issued: a wait for them placed
    // by the compiler inside the tile loop would also drain the direct loads in flight.
#pragma unroll
    for (int tok = 0; tok < 2; ++tok)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            materialize(qa[tok][mt]);
            materialize(wa[tok][mt]);
#pragma unroll
            for (int r = 0; r < 4; ++r) materialize(wt[tok][mt][r]);
        }

    // Direct loads of tile t into its ring buffer: instruction I < KEY_INSTRS moves rows
    // I*ROWS_PER_INSTR.., the others 64 key scales each.  Rows past the causal end of the
    // segment read the last valid key instead (their scores are never stored).
    const uint8_t* kseq = k8 + (int64_t)kbase * D;
    const float* sseq = ks + kbase;
    const uint32_t lds0 = lds_addr(lds);
    auto buf_of = [&](int t) {
        return (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(t % kIxBufs) * T::BYTES);
    };
    auto issue_tile = [&](int t) {
        const uint32_t buf = buf_of(t);
        const int key0 = seg0 + t * kIxTile;
        // the per-lane offsets are recomputed for each tile (a few VALU) rather than kept
        // live across the loop, where they would compete with the MFMA operands for registers
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int k = 0; k < T::PER_WAVE; ++k) {
            const int I = wv + kIxWaves * k;
            if (I < T::KEY_INSTRS) {
                const int r = I * T::ROWS_PER_INSTR + ln / T::CH;
                const int p = ln % T::CH;
                const int key = min(key0 + r, pmax);
                dma16(kseq, (uint32_t)key * D + 16 * (p ^ T::swz(r)), buf + I * 1024);
            } else if (I < T::INSTRS) {
                const int j = I - T::KEY_INSTRS;
                const int key = min(key0 + 64 * j + ln, pmax);
                dma4(sseq, (uint32_t)key * 4, buf + T::KEY_BYTES + 256 * j);
            }
        }
    };
    // Loads this wave issues per tile (the same for every tile), for the waits.
    const int my_loads = (T::INSTRS - wv + kIxWaves - 1) / kIxWaves;

    auto load_b = [&](uint32_t buf, int g) {
        v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
        if (grp < KGRP) {
            const int r = 16 * g + col;
            const v4i blo = lds_read16(buf + T::chunk(r, 2 * grp));
            const v4i bhi = lds_read16(buf + T::chunk(r, 2 * grp + 1));
            b = (v8i){blo.x, blo.y, blo.z, blo.w, bhi.x, bhi.y, bhi.z, bhi.w};
        }
        return b;
    };
    // Scores of a tile are held in registers and stored at the start of the next tile, after
    // its wait: stores issued between the direct loads would otherwise lengthen the waits
    // (they count on the same counter).  Slot s holds key groups 2s and 2s+1: lane group r
    // keeps group 2s + (r & 1) of token r >> 1, so each store instruction writes 64 scores.
    // (Stores spread over the next tile's MFMA stream, one slot per group, measured slower.)
    float held[8];
    int held_key0 = 0, held_groups = 0;
    // Counts a stored score if it is >= +0 (the top bit of its order-preserving key is set):
    // for such scores key bits 30..21 are the float's own bits 30..21 (-0 counts as +0 in
    // bin 0; NaN and negative scores fail the comparison).
    auto count = [&](float v, int tok) {
        const uint32_t b = (__float_as_uint(v) >> 21) & (kHistBins - 1);
        if (v >= 0.f) atomicAdd(&hcount[2 * wv + tok][b >> 1], 1u << ((b & 1) << 4));
    };
    auto flush_slot = [&](int slot) {
        const int g_odd = grp & 1, tok = grp >> 1;
        const int my_pos = tok ? tpos[1] : tpos[0];
        const int64_t my_row = tok ? trow[1] : trow[0];
        const int g = 2 * slot + g_odd;
        const int s = held_key0 + 16 * g + col;
        if (g < held_groups && s <= my_pos) {
            scores[my_row * stride + s] = held[slot];
            if (hist != nullptr) count(held[slot], tok);
        }
    };
    auto flush = [&]() {
        if (held_groups == kIxTile / 16 && held_key0 + kIxTile - 1 <= min(tpos[0], tpos[1])) {
            // the whole held tile lies below both tokens' positions: no per-slot tests
            const int tok = grp >> 1;
            float* rp = scores + (int64_t)(tok ? trow[1] : trow[0]) * stride + held_key0 + 16 * (grp & 1) + col;
#pragma unroll
            for (int slot = 0; slot < 8; ++slot) {
                rp[32 * slot] = held[slot];
                if (hist != nullptr) count(held[slot], tok);
            }
        } else {
#pragma unroll
            for (int slot = 0; slot < 8; ++slot) flush_slot(slot);
        }
        held_groups = 0;
    };
    // Sums the partials of groups 2s (pe) and 2s+1 (po) over the four lane groups with two
    // lane-swap rounds, leaving lane group r with group 2s + (r & 1) of token r >> 1 (the
    // layout flush expects), then applies that key's scale (read a group ahead: a read here
    // would make the MFMAs wait for every LDS read in flight, operand prefetch included).
    auto reduce_pair = [&](const float (&pe)[2], const float (&po)[2], float kscale, int slot) {
        auto sw32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pe[0]), __float_as_uint(pe[1]), false, false);
        auto sw32o = __builtin_amdgcn_permlane32_swap(__float_as_uint(po[0]), __float_as_uint(po[1]), false, false);
        const float x = __uint_as_float(sw32[0]) + __uint_as_float(sw32[1]);
        const float y = __uint_as_float(sw32o[0]) + __uint_as_float(sw32o[1]);
        auto sw16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        const float z = __uint_as_float(sw16[0]) + __uint_as_float(sw16[1]);
        held[slot] = z * kscale;
    };
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);

    // Linear-part query of each token, while the first tiles load.  u = sum_j (w'_j/2) q_j is
    // folded in the A layout (lane: head mt*16 + col, dims 32*grp + e), summed over the 16 lanes
    // of a row by a reduce-scatter that leaves dims 32*grp + 2*col + {0,1} in each lane, and
    // split into FP8 terms there.  The codes go through LDS (ring buffer 2, not loaded before
    // the first barrier of the tile loop) into the A fragment of the linear MFMA: row
    // rho = col holds term rho & 7 of token rho >> 3 (terms >= kLinTerms are zero).
    constexpr int kLinBytes = 2 * 8 * KGRP * 32;  // per wave: [token][term][K group][32 bytes]
    static_assert(kIxBufs >= 3 && kIxWaves * kLinBytes <= T::BYTES, "linear codes fit ring buffer 2");
    uint8_t* lin_lds = lds + 2 * T::BYTES + wv * kLinBytes;
    v8i ql;
    float lin_scale[2];  // multiplier of this lane's linear row sum for token 0 / 1
    {
        int ex[2];
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {
            float v[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) v[e] = 0.f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int x = qa[tok][mt][i];
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
                    v[4 * i + 0] = fmaf(wa[tok][mt], lo[0], v[4 * i + 0]);
                    v[4 * i + 1] = fmaf(wa[tok][mt], lo[1], v[4 * i + 1]);
                    v[4 * i + 2] = fmaf(wa[tok][mt], hi[0], v[4 * i + 2]);
                    v[4 * i + 3] = fmaf(wa[tok][mt], hi[1], v[4 * i + 3]);
                }
            }
            // partners of the four steps differ in lane bits 3, 2, 1, 0 of col (the masks
            // 15, 7, 3, 1 generate every xor of the row, so all 16 lanes are summed)
            reduce_half<16, kDppRowMirror>(v, col & 8);
            reduce_half<8, kDppRowHalfMirror>(v, col & 4);
            reduce_half<4, kDppQuadReverse>(v, col & 2);
            reduce_half<2, kDppQuadSwap>(v, col & 1);
            float m = fmaxf(fabsf(v[0]), fabsf(v[1]));
            m = fmaxf(m, dpp_f<kDppRowMirror>(m));
            m = fmaxf(m, dpp_f<kDppRowHalfMirror>(m));
            m = fmaxf(m, dpp_f<kDppQuadReverse>(m));
            m = fmaxf(m, dpp_f<kDppQuadSwap>(m));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            // E = exponent of max|u| (at least -100, so every scale below is a normal float or
            // an exact subnormal); |u| < 2^(E+1) puts the first term below 256, and each
            // residual is at most half an FP8 step of the term before, below 128 in the next
            // term's units, so no term saturates.
            const int e = max((int)((__float_as_uint(m) >> 23) & 0xff) - 127, -100);
            ex[tok] = __builtin_amdgcn_readfirstlane(e);
#pragma unroll
            for (int j = 0; j < kLinTerms; ++j) {
                const float up = ldexpf(1.f, 7 + 4 * j - ex[tok]);
                const float dn = ldexpf(1.f, ex[tok] - 7 - 4 * j);
                const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * up, v[1] * up, 0, false);
                const auto back = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
                v[0] = fmaf(-back[0], dn, v[0]);  // exact: the rounding residual
                v[1] = fmaf(-back[1], dn, v[1]);
                if (grp < KGRP)
                    *(uint16_t*)(lin_lds + ((tok * 8 + j) * KGRP + grp) * 32 + 2 * col) = (uint16_t)pk;
            }
        }
        const int rt = col >> 3, rj = col & 7;
        const uint8_t* src = lin_lds + ((rt * 8 + min(rj, kLinTerms - 1)) * KGRP + min(grp, KGRP - 1)) * 32;
        const v4i lo = *(const v4i*)src;
        const v4i hi = *(const v4i*)(src + 16);
        ql = (rj < kLinTerms && grp < KGRP) ? (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}
                                            : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
        materialize(ql);  // the reads complete before the buffer is reused
        // C layout of the linear MFMA: lane group grp holds rows 4*grp + r, i.e. terms
        // 4*(grp & 1) + r of token grp >> 1, whose sum is 2^(E-7-16*(grp&1)) * (C0 + C1/16 +
        // C2/256 + C3/4096)
#pragma unroll
        for (int tok = 0; tok < 2; ++tok)
            lin_scale[tok] = (grp >> 1) == tok ? ldexpf(1.f, ex[tok] - 7 - 16 * (grp & 1)) : 0.f;
    }

    for (int t = 0; t < ntiles; ++t) {
        // Tile t has landed for this wave (the younger loads of tile t+1 may still fly; the
        // stores issued since are older than nothing we wait for), then for every wave; the
        // barrier also retires tile t-1, whose buffer tile t+2 takes over.
        if (t + 1 < ntiles) {
            if (my_loads == 5) wait_loads<5>();
            else if (my_loads == 4) wait_loads<4>();
            else if (my_loads == 3) wait_loads<3>();
            else if (my_loads == 2) wait_loads<2>();
            else if (my_loads == 1) wait_loads<1>();
            else wait_loads<0>();
        } else {
            wait_loads<0>();
        }
        lds_barrier();
        flush();  // scores of tile t-1, before the loads of tile t+2
        if (t + 2 < ntiles) issue_tile(t + 2);
        const int key0 = seg0 + t * kIxTile;
        if (key0 > tmax) continue;  // this wave's tokens are all before the tile
        const uint32_t buf = buf_of(t);
        const int ngroups = min(kIxTile / 16, (tmax - key0) / 16 + 1);

        // The MFMAs of a group (k = 0: the linear part of both tokens; then token-major,
        // k = 1 + NMT*tok + mt) each run with the epilogue of the MFMA issued DEP = 2 before
        // them, so the matrix pipe stays busy while the VALU works on a result that has landed
        // (three accumulator tiles rotate; at distance 1 the epilogue would wait on the MFMA's
        // latency); the last DEP MFMAs of a group are taken up under the first DEP of the next.
        // Operand reads fly two groups ahead.  Every group of the tile is computed (rows past
        // the causal end hold valid clamped keys; their scores are not stored), so the fully
        // unrolled sequence has no branches and the held slots, accumulators and operand
        // registers stay static.
        constexpr int NG = kIxTile / 16;
        constexpr int NK = 2 * NMT + 1;
        constexpr int DEP = 2;
        v8i bq[2];
        v4f acc[2][NMT];
        v4f accl;
        float part[2][2];  // [group parity][token]
        bq[0] = load_b(buf, 0);
        bq[1] = load_b(buf, 1);
        // Epilogue of MFMA k of group gg.  The linear MFMA's row sum starts each token's chain
        // of |x| terms (dependent VALU instructions issue back to back at the wave's cadence).
        float linv[2][2], ev[2][2];  // [group parity][token]
        float kscale = 0.f;  // scale of this lane's key in the next slot to be reduced
        auto epi_k = [&](int gg, int k) {
            if (k == 0) {
                float hs = fmaf(accl[3], 0.0625f, accl[2]);
                hs = fmaf(hs, 0.0625f, accl[1]);
                hs = fmaf(hs, 0.0625f, accl[0]);
                float l0 = hs * lin_scale[0], l1 = hs * lin_scale[1];
                asm volatile("" : "+v"(l0), "+v"(l1));
                linv[gg & 1][0] = l0;
                linv[gg & 1][1] = l1;
                return;
            }
            const int tok = (k - 1) / NMT, mt = (k - 1) % NMT;
            float a = mt == 0 ? linv[gg & 1][tok] : ev[gg & 1][tok];
#pragma unroll
            for (int r = 0; r < 4; ++r) a = fmaf(wt[tok][mt][r], fabsf(acc[tok][mt][r]), a);
            asm volatile("" : "+v"(a));  // keep these FMAs in this step
            ev[gg & 1][tok] = a;
            if (mt == NMT - 1) part[gg & 1][tok] = a;
        };
#pragma unroll
        for (int g = 0; g < NG; ++g) {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                // MFMA k overwrites its accumulator, whose previous contents were consumed a
                // step ago
                if (k == 0) {
                    if (g & 1) {  // slot (g-1)/2 holds groups g-1 and g; lane group r keeps g-1+(r&1)
                        int ln = lane;  // recomputed, not held in a register per group
                        asm volatile("" : "+v"(ln));
                        kscale = *(const __attribute__((address_space(3))) float*)(size_t)(
                            buf + T::KEY_BYTES + 4 * (16 * (g - 1 + ((ln >> 4) & 1)) + (ln & 15)));
                    }
                    accl = mfma_fp8_16x16x128(ql, bq[g & 1]);
                } else {
                    const int tok = (k - 1) / NMT, mt = (k - 1) % NMT;
                    acc[tok][mt] = mfma_fp8_16x16x128(qa[tok][mt], bq[g & 1]);
                }
                if (k >= DEP) {
                    epi_k(g, k - DEP);
                } else if (g > 0) {
                    epi_k(g - 1, NK - DEP + k);  // the previous group's last DEP
                    if (k == DEP - 1 && !(g & 1)) reduce_pair(part[0], part[1], kscale, (g - 1) >> 1);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // the MFMA first,
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // then the FMAs
                __builtin_amdgcn_sched_barrier(0);
            }
            if (g + 2 < NG) bq[g & 1] = load_b(buf, g + 2);
        }
#pragma unroll
        for (int d = DEP; d >= 1; --d) epi_k(NG - 1, NK - d);
        reduce_pair(part[0], part[1], kscale, (NG - 1) >> 1);
        held_key0 = key0;
        held_groups = ngroups;
    }
    flush();
    if (hist != nullptr) {  // add this segment's counts to the rows' histograms
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {
            if (tpos[tok] < 0) continue;
            uint32_t* hrow = hist + (int64_t)trow[tok] * kHistBins;
            const uint32_t* hc = &hcount[2 * wv + tok][0];
            for (int j = lane; j < kHistBins / 2; j += kWave) {
                const uint32_t v = hc[j];
                if (v & 0xffffu) atomicAdd(&hrow[2 * j], v & 0xffffu);
                if (v >> 16) atomicAdd(&hrow[2 * j + 1], v >> 16);
            }
        }
    }
}

constexpr int kDecodeThreads = 256;
constexpr int kDecodeKeysPerWave = 256;
constexpr int kDecodeKeys = kDecodeKeysPerWave * (kDecodeThreads / kWave);
constexpr int kDecodeUnroll = 4;  // 16-key groups per step (two steps in flight)
static_assert(kDecodeUnroll % 4 == 0, "each lane group stores every fourth group");

// Decode: one query row per sequence against its whole key cache.  The work is a stream of
// 132 bytes per cached key, so each wave reads its key fragments straight from memory into
// MFMA operand registers, several 16-key groups ahead.
template <int H, int D>
__global__ __launch_bounds__(kDecodeThreads) void indexer_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, float* __restrict__ scores,
    int64_t stride, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ pages, int pages_per_seq, uint32_t* __restrict__ hist) {
    constexpr int NMT = (H + 15) / 16;
    constexpr int KGRP = D / 32;
    // counts of this workgroup's stored scores >= +0 by key bits 30..21 (when hist is given)
    __shared__ uint32_t hcount[kHistBins];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int b = blockIdx.y;
    const int kbase = cu_k[b];
    const int nkeys = cu_k[b + 1] - kbase;
    const int qrow = cu_q[b];  // decode: exactly one query row, at position nkeys - 1
    if (blockIdx.x * kDecodeKeys >= nkeys) return;  // the whole workgroup
    if (hist != nullptr) {
        for (int j = tid; j < kHistBins; j += kDecodeThreads) hcount[j] = 0u;
        __syncthreads();
    }
    const int s_begin = blockIdx.x * kDecodeKeys + wv * kDecodeKeysPerWave;
    // a wave past the keys takes part in the barriers only
    const int s_end = max(s_begin, min(s_begin + kDecodeKeysPerWave, nkeys));
    if (s_begin < s_end) {

    v8i qa[NMT];
    float wt[NMT][4];  // half the folded weight: w * ReLU(x) = wt * x + wt * |x|
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
            wt[mt][r] = hh < H ? 0.5f * w[(int64_t)qrow * H + hh] * qs[(int64_t)qrow * H + hh] : 0.f;
        }
    }
    float* srow = scores + (int64_t)qrow * stride;
    // Key fragments of kDecodeUnroll 16-key groups per step, loaded one step ahead: the loads
    // of step i+1 go out before the scores of step i are stored, so waiting for them never
    // waits for those stores (stores and loads share one counter, which drains in order).
    // Addresses are clamped to the wave's range (stores of clamped keys are masked), so the
    // loads carry no branches.
    struct Frag {
        v8i b[kDecodeUnroll];
        float ks[kDecodeUnroll];
    };
    // Cache row of the step's first key: a step of 64 keys is one page of a paged cache
    // (steps start at multiples of 64).
    static_assert(16 * kDecodeUnroll == kPage && kDecodeKeysPerWave % kPage == 0, "one page per step");
    auto step_row = [&](int s0) -> int64_t {
        if (pages == nullptr) return (int64_t)kbase + s0;
        return (int64_t)pages[(int64_t)b * pages_per_seq + s0 / kPage] * kPage;
    };
    auto load = [&](int s0, Frag& f) {
        const int64_t r0 = step_row(s0);
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int ds = min(s0 + 16 * u + col, s_end - 1) - s0;
            const uint8_t* src = k8 + (r0 + ds) * D + (grp < KGRP ? grp : 0) * 32;
            const v4i lo = *(const v4i*)src;
            const v4i hi = *(const v4i*)(src + 16);
            f.b[u] = grp < KGRP ? (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}
                                : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
            f.ks[u] = ks[r0 + ds];
        }
    };
    constexpr int STEP = 16 * kDecodeUnroll;
    constexpr int NSTEP = kDecodeKeysPerWave / STEP;
    static_assert(kDecodeKeysPerWave % STEP == 0 && kDecodeUnroll == 4, "one score per lane and step");
    // the wave's scores are held (one per lane and step) and stored after the loop, so no
    // store is in flight while the key loads stream
    float held[NSTEP];
    Frag cur, nxt;
    load(s_begin, nxt);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
        const int s0 = s_begin + st * STEP;
        cur = nxt;
        if (st + 1 < NSTEP && s0 + STEP < s_end) load(s0 + STEP, nxt);
        float sc[kDecodeUnroll];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const v4f acc = mfma_fp8_16x16x128(qa[mt], cur.b[u]);
#pragma unroll
                for (int r = 0; r < 4; ++r) part = fmaf(wt[mt][r], fabsf(acc[r]), fmaf(wt[mt][r], acc[r], part));
            }
            sc[u] = sum_over_groups(part) * cur.ks[u];  // every lane group holds the sum
        }
        // lane group g keeps group u = g: 64 consecutive keys per step over all lanes
        held[st] = grp == 0 ? sc[0] : grp == 1 ? sc[1] : grp == 2 ? sc[2] : sc[3];
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
        const int s = s_begin + st * STEP + 16 * grp + col;
        if (s < s_end) {
            srow[s] = held[st];
            // a score >= +0 has key bits 30..21 equal to its own bits 30..21 (-0 in bin 0)
            const uint32_t bin = (__float_as_uint(held[st]) >> 21) & (kHistBins - 1);
            if (hist != nullptr && held[st] >= 0.f) atomicAdd(&hcount[bin], 1u);
        }
    }
    }  // s_begin < s_end
    if (hist != nullptr) {
        __syncthreads();
        uint32_t* hrow = hist + (int64_t)qrow * kHistBins;
        for (int j = tid; j < kHistBins; j += kDecodeThreads) {
            const uint32_t c = hcount[j];
            if (c != 0u) atomicAdd(&hrow[j], c);
        }
    }
}

template <int H, int D>
hipError_t launch_prefill_t(const IndexerArgs& a, int row0, int n_rows, int pos0, int kbase,
                            float* scores, uint32_t* hist, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    const int pmax = pos0 + n_rows - 1;
    dim3 grid((n_rows + kIxTokens - 1) / kIxTokens, pmax / kIxSeg + 1);
    hipLaunchKernelGGL((indexer_prefill_kernel<H, D>), grid, dim3(kIxThreads), 0, st, a.q8,
                       a.q_scale, a.w, a.k8, a.k_scale, scores, a.score_stride, row0, n_rows,
                       pos0, kbase, hist);
    return hipGetLastError();
}

template <int H, int D>
hipError_t launch_decode_t(const IndexerArgs& a, int n_seqs, int max_keys, const int32_t* cu_q,
                           const int32_t* cu_k, const int32_t* pages, int pages_per_seq, uint32_t* hist,
                           hipStream_t st) {
    dim3 grid((max_keys + kDecodeKeys - 1) / kDecodeKeys, n_seqs);
    hipLaunchKernelGGL((indexer_decode_kernel<H, D>), grid, dim3(kDecodeThreads), 0, st, a.q8,
                       a.q_scale, a.w, a.k8, a.k_scale, a.scores, a.score_stride, cu_q, cu_k, pages,
                       pages_per_seq, hist);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_prefill(const IndexerArgs& a, int row0, int n_rows, int pos0,
                                  int kbase, float* scores, hipStream_t st, uint32_t* hist) {
    if (a.shape == Shape::Prod) return launch_prefill_t<64, 128>(a, row0, n_rows, pos0, kbase, scores, hist, st);
    return launch_prefill_t<4, 32>(a, row0, n_rows, pos0, kbase, scores, hist, st);
}

hipError_t launch_indexer_decode(const IndexerArgs& a, int n_seqs, int max_keys,
                                 const int32_t* cu_q, const int32_t* cu_k, const int32_t* pages,
                                 int pages_per_seq, hipStream_t st, uint32_t* hist) {
    if (a.shape == Shape::Prod)
        return launch_decode_t<64, 128>(a, n_seqs, max_keys, cu_q, cu_k, pages, pages_per_seq, hist, st);
    return launch_decode_t<4, 32>(a, n_seqs, max_keys, cu_q, cu_k, pages, pages_per_seq, hist, st);
}

}  // namespace dsa
