// Indexer training target, forward only, on gfx950 (DeepSeek-V3.2-Exp overview, "训练";
// 解析 §二; DSA deep dive §3): for query row t over its slot positions S_t (every s <= p in the
// dense warm-up, the top-k set in the sparse stage)
//     P_t[s] = sum_h exp(z[t,h,s] - lse[t,h]),  z = sm_scale * q[t,h,:] . kv[s,:]
// (the main attention probabilities summed over heads), L1-normalised over S_t, compared with
// Q_t = softmax over S_t of the indexer scores I[t,s]:
//     KL(P||Q) = A/Z - ln Z - B/Z + LSE(I)      with Z = sum P, A = sum P ln P, B = sum P I
//     KL(Q||P) = (R1 - R2)/l - LSE(I) + ln Z    with l = sum e^(I-m), R1 = sum e^(I-m) I,
//                                                    R2 = sum e^(I-m) ln P,  LSE = m + ln l
// so one pass over the slots accumulates every term.
//
// One workgroup of 4 waves per query row; wave w owns heads 32w .. 32w+31 and keeps their
// query in registers as the A operand of v_mfma_f32_32x32x16_bf16 (M = heads, K = dims); a
// block of 32 slots is gathered into LDS by direct global->LDS loads, chunk-major ([16-byte
// column chunk][slot]), so that the B operand of k-slice i (N = slots, lane l: slot l % 32,
// chunk 2i + l / 32) is one contiguous 1 KiB read and one load instruction fills it.  Each
// accumulator lane then holds one slot and 16 heads, so the head sum is in-lane plus one
// exchange with lane l ^ 32; the four waves' sums meet in LDS.  Bound: bf16 MFMA (147,456
// FLOP per slot) against the LDS reads of the block (each wave reads all of it).
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kKlThreads = 256;
constexpr int kKlSlots = 32;  // slots per block

__device__ __forceinline__ v16f mfma32(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int H, int DQK>
struct KlCfg {
    static constexpr int KS = DQK / 16;                 // k-slices = load instructions per block
    static constexpr int ROWB = DQK * 2;                // bytes of a latent row
    static constexpr int NWA = (H + 31) / 32;           // waves holding heads
    static constexpr int NW = kKlThreads / kWave;
    static constexpr int PER_W = (KS + NW - 1) / NW;    // load instructions per wave and block
    static constexpr int BUF = KS * 1024;               // [2 KS chunks][32 slots][16 B]
    static_assert(DQK % 16 == 0 && NWA <= NW, "at most 128 heads");
};

// Running sums of one lane over the slots it owns (plain data: it also lives in LDS).
struct KlAcc {
    double z, a, b;     // sum P, sum P ln P, sum P I
    float m;            // running max of I
    double l, r1, r2;   // sum e^(I-m), sum e^(I-m) I, sum e^(I-m) ln P
    int pzero;          // some slot has P = 0 (KL(Q||P) is then infinite)
    __device__ void init() {
        z = a = b = l = r1 = r2 = 0.0;
        m = -INFINITY;
        pzero = 0;
    }
    __device__ void add(float p, float I) {
        z += p;
        const float lp = p > 0.f ? __logf(p) : 0.f;
        if (p > 0.f) {
            a += (double)(p * lp);
            b += (double)p * (double)I;
        } else {
            pzero = 1;
        }
        if (I > m) {
            const double s = m == -INFINITY ? 0.0 : (double)__expf(m - I);
            l *= s;
            r1 *= s;
            r2 *= s;
            m = I;
        }
        const double w = (double)__expf(I - m);
        l += w;
        r1 += w * (double)I;
        r2 += w * (double)lp;
    }
    // Merge with another lane's sums.
    __device__ void merge(const KlAcc& o) {
        z += o.z;
        a += o.a;
        b += o.b;
        pzero = pzero | o.pzero;
        if (o.m == -INFINITY) return;
        if (m == -INFINITY) {
            m = o.m;
            l = o.l;
            r1 = o.r1;
            r2 = o.r2;
            return;
        }
        const float M = fmaxf(m, o.m);
        const double s0 = (double)__expf(m - M), s1 = (double)__expf(o.m - M);
        l = l * s0 + o.l * s1;
        r1 = r1 * s0 + o.r1 * s1;
        r2 = r2 * s0 + o.r2 * s1;
        m = M;
    }
    __device__ void shfl_merge(int o) {
        KlAcc t;
        t.z = __shfl_xor(z, o);
        t.a = __shfl_xor(a, o);
        t.b = __shfl_xor(b, o);
        t.m = __shfl_xor(m, o);
        t.l = __shfl_xor(l, o);
        t.r1 = __shfl_xor(r1, o);
        t.r2 = __shfl_xor(r2, o);
        t.pzero = __shfl_xor(pzero, o);
        merge(t);
    }
};

template <int H, int DQK>
__global__ __launch_bounds__(kKlThreads, 2) void indexer_kl_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ lse,
    const int32_t* __restrict__ idx, int topk, int mode, const float* __restrict__ scores, int64_t stride,
    float* __restrict__ kl, float* __restrict__ kl_rev, RowMap map, int n_rows, float sm_log2) {
    using C = KlCfg<H, DQK>;
    __shared__ __attribute__((aligned(1024))) uint8_t buf[2][C::BUF];
    __shared__ float psum[C::NWA][kKlSlots];
    __shared__ int ids[2][kKlSlots];
    __shared__ KlAcc fin[C::NWA];

    const int row = blockIdx.x;
    if (row >= n_rows) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const RowInfo ri = row_info(map, row);
    const bool dense = mode == (int)IdxMode::Dense;
    const int jn = dense ? ri.pos + 1 : mode == (int)IdxMode::Front ? min(topk, ri.pos + 1) : topk;
    const int nblk = (jn + kKlSlots - 1) / kKlSlots;
    const int32_t* irow = dense ? nullptr : idx + (int64_t)row * topk;
    const float* srow = scores + (int64_t)row * stride;
    const bool paged = map.pages != nullptr;
    const uint8_t* kvb = (const uint8_t*)(paged ? kv : kv + (int64_t)ri.kbase * DQK);

    // a slot's position, or -1 when it is empty or names no loadable row (values outside the
    // sequence, page ids outside a pool of known size): such slots take no part, so no load or
    // score read ever leaves the caches
    auto slot_id = [&](int b, int s) {
        const int j = b * kKlSlots + s;
        if (j >= jn) return -1;
        const int id = dense ? j : irow[j];
        return slot_row(map, ri, id) >= 0 ? id : -1;
    };
    auto kv_row = [&](int id) -> int64_t { return paged ? cache_row(map, ri, id) : (int64_t)id; };

    // query fragments (A operand): lane l holds head 32 wv + l % 32, dims 16 i + 8 (l / 32) ..
    const int hq = 32 * wv + (lane & 31);
    const bool has_heads = wv < C::NWA;
    v8bf qf[C::KS];
    {
        const uint16_t* qp = q + ((int64_t)ri.qrow * H + (hq < H ? hq : 0)) * DQK + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < C::KS; ++i) {
            const v4i v = has_heads && hq < H ? *(const v4i*)(qp + 16 * i) : (v4i){0, 0, 0, 0};
            qf[i] = __builtin_bit_cast(v8bf, v);
        }
    }
    // base-2 log-sum-exp of the 16 heads of each accumulator lane (+inf: no such head)
    float lse2[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int h = 32 * wv + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        const float v = has_heads && h < H ? lse[(int64_t)ri.qrow * H + h] : -INFINITY;
        lse2[r] = v == -INFINITY ? INFINITY : v * 1.4426950408889634f;
    }

    // gather of block b: load instruction i (k-slice i) moves chunk 2i + l / 32 of slot l % 32
    // to buf + i * 1024 + 16 l; wave w issues instructions w, w + 4, ...  An empty slot loads
    // row 0 (its column of the product is never used).  Packed caches load at 32-bit offsets
    // from the sequence's first row (a sequence is shorter than 2^32 / 1152 positions, checked
    // on the host); paged caches at 64-bit addresses, so a page pool may exceed 4 GiB.
    auto load_block = [&](int b) {
        const int id = ids[b & 1][lane & 31];
        const uint32_t dst = lds_addr(buf[b & 1]);
        if (paged) {
            const uint8_t* src = kvb + (id >= 0 ? (uint64_t)kv_row(id) * C::ROWB : 0) + 16u * (lane >> 5);
#pragma unroll
            for (int u = 0; u < C::PER_W; ++u) {
                const int i = wv + C::NW * u;
                if (i < C::KS) dma16_at(src + 32u * i, dst + 1024u * i);
            }
            return;
        }
        const uint32_t roff = id >= 0 ? (uint32_t)id * (uint32_t)C::ROWB : 0u;
#pragma unroll
        for (int u = 0; u < C::PER_W; ++u) {
            const int i = wv + C::NW * u;
            if (i < C::KS) dma16(kvb, roff + 32u * i + 16u * (lane >> 5), dst + 1024u * i);
        }
    };
    // block b is accumulated by wave b % NWA, which fetches its ids and scores one block
    // early into register slot b & 1 (with one wave holding heads, it owns consecutive blocks)
    KlAcc acc;
    acc.init();
    int my_id[2] = {-1, -1};
    float my_sc[2] = {0.f, 0.f};
    auto fetch_owned = [&](int b) {
        if (b < nblk && wv == b % C::NWA && lane < kKlSlots) {
            const int id = ids[b & 1][lane];
            const float sc = id >= 0 ? srow[id] : 0.f;
            if (b & 1) {
                my_id[1] = id;
                my_sc[1] = sc;
            } else {
                my_id[0] = id;
                my_sc[0] = sc;
            }
        }
    };

    if (nblk > 0) {
        if (wv == 0 && lane < kKlSlots) {
            ids[0][lane] = slot_id(0, lane);
            ids[1][lane] = slot_id(1, lane);
        }
        __syncthreads();
        load_block(0);
        fetch_owned(0);
        wait_loads<0>();
        __syncthreads();
    }
    for (int b = 0; b < nblk; ++b) {
        const bool more = b + 1 < nblk;
        if (more) {
            load_block(b + 1);
            fetch_owned(b + 1);
        }
        if (has_heads) {
            const uint32_t cb = lds_addr(buf[b & 1]) + 16u * lane;
            v16f s = {};
#pragma unroll
            for (int i = 0; i < C::KS; ++i) s = mfma32(qf[i], __builtin_bit_cast(v8bf, lds_read16(cb + 1024u * i)), s);
            float e = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) e += __builtin_amdgcn_exp2f(fmaf(s[r], sm_log2, -lse2[r]));
            e += __shfl_xor(e, 32);
            if (lane < kKlSlots) psum[wv][lane] = e;
        }
        lds_barrier();  // head sums of block b visible; block b's buffer is no longer read
        const int cid = (b & 1) ? my_id[1] : my_id[0];
        if (wv == b % C::NWA && lane < kKlSlots && cid >= 0) {
            float p = 0.f;
#pragma unroll
            for (int w = 0; w < C::NWA; ++w) p += psum[w][lane];
            acc.add(p, (b & 1) ? my_sc[1] : my_sc[0]);
        }
        if (wv == 0 && lane < kKlSlots && b + 2 < nblk) ids[b & 1][lane] = slot_id(b + 2, lane);
        wait_loads<0>();  // this wave's loads of block b+1 (and its score fetch) have landed
        lds_barrier();    // block b+1 and the ids of block b+2 visible
    }

    // lanes 32..63 hold nothing: merge over the 32 slot lanes, then over the waves
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) acc.shfl_merge(o);
    if (wv < C::NWA && lane == 0) fin[wv] = acc;
    __syncthreads();
    if (tid != 0) return;
    KlAcc t = fin[0];
    for (int w = 1; w < C::NWA; ++w) t.merge(fin[w]);
    float f = 0.f, r = 0.f;
    if (t.z > 0.0) {
        const double lnz = log(t.z);
        const double lse_i = (double)t.m + log(t.l);
        f = (float)(t.a / t.z - lnz - t.b / t.z + lse_i);
        r = t.pzero ? INFINITY : (float)((t.r1 - t.r2) / t.l - lse_i + lnz);
    }
    kl[ri.qrow] = f;
    if (kl_rev != nullptr) kl_rev[ri.qrow] = r;
}

}  // namespace

hipError_t launch_indexer_kl(const KlArgs& a, const RowMap& map, int n_rows, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    const float sm_log2 = a.sm_scale * 1.4426950408889634f;
    if (a.shape == Shape::Prod)
        hipLaunchKernelGGL((indexer_kl_kernel<128, 576>), dim3(n_rows), dim3(kKlThreads), 0, st, a.q, a.kv, a.lse,
                           a.idx, a.topk, (int)a.mode, a.scores, a.stride, a.kl, a.kl_rev, map, n_rows, sm_log2);
    else
        hipLaunchKernelGGL((indexer_kl_kernel<8, 80>), dim3(n_rows), dim3(kKlThreads), 0, st, a.q, a.kv, a.lse,
                           a.idx, a.topk, (int)a.mode, a.scores, a.stride, a.kl, a.kl_rev, map, n_rows, sm_log2);
    return hipGetLastError();
}

}  // namespace dsa
