// Sparse MQA over the MLA latent cache on gfx950 (core attention of DSA on the top-k rows;
// DeepSeek-V3.2 explained, sections 二.1 and 二.4; DeepSeek-V3.2-Exp overview, module table).
//
// For query row t and head h, over the selected latent rows c_s (576 = 512 latent + 64
// rope; every head shares the row):
//     z_s = sm * <q[t,h,:], c_s>,  out[t,h,:] = sum_s softmax(z)_s c_s[:512],  lse = ln sum e^z
//
// Work decomposition: one workgroup = one query row x 64 heads (two workgroups per row of 128
// heads, issued 8 ids apart so both run on the same XCD and the second gather of each latent
// row hits its L2).  Its 4 waves are 2 head groups (32 heads) x 2 halves; a half owns half of
// the 576 logit dims (query fragments stay in registers) and half of the 512 value dims
// (fp32 accumulators).  Per block of 32 selected rows:
//   gather   direct global->LDS loads (no staging registers) in a three-deep ring, so the
//            loads of the next two blocks fly while this one computes;
//   S^T      = C Q^T with v_mfma_f32_32x32x16_bf16 (A = latent rows from LDS, M = rows;
//            B = query heads, N = heads) over the wave's dims; the halves' partial tiles are
//            summed through LDS (both waves form S0 + S1 in the same order);
//   softmax  online, in base 2; lane l owns head l%32, so running max and sum are per lane
//            (one exchange with lane l^32); O is rescaled only when a block max exceeds the
//            running max by more than 16 (2^16 of headroom in fp32 and bf16 P);
//   O^T      += V^T P^T with A = value columns read by ds_read_b64_tr_b16 straight from the
//            row-major block and B = P^T taken from the S^T accumulators (the S^T row order
//            puts 8 consecutive block rows in each lane per 16-row k-slice).
// LDS rows are XOR-swizzled in 16-byte chunks so that the 16 rows read together by an A
// operand, and the 4 consecutive rows of a transpose read, fall in distinct bank groups.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kBlk = 32;            // selected rows per LDS block
constexpr float kRescaleGap = 16.f;  // base-2 headroom before O is rescaled

// One region (value part or rope part) of the LDS image of a block: kBlk rows of NC 16-byte
// chunks, written 1 KiB (64 chunks) per direct-load instruction.
template <int NC>
struct Region {
    static_assert(NC == 64 || NC == 8 || NC == 2, "unsupported region width");
    static constexpr int NCH = NC;
    static constexpr int SWZ_BITS = NC == 64 ? 4 : (NC == 8 ? 3 : 1);  // bits swz(r) can set
    static constexpr int ROWS_PER_INSTR = 64 / NC;
    static constexpr int PITCH = NC * 16;
    static constexpr int BYTES = kBlk * PITCH;
    static constexpr int INSTRS = kBlk / ROWS_PER_INSTR;
    // 64-chunk rows: any 16 consecutive rows and any 4 consecutive rows (x 4 chunks) map to
    // distinct 16-byte bank groups; narrow rows: pairs of rows share a 256-byte line.
    __device__ static __forceinline__ int swz(int r) {
        if constexpr (NC == 64) return ((r & 3) << 2) | ((r >> 2) & 3);
        else return (r >> 1) & (NC - 1);
    }
    __device__ static __forceinline__ int chunk(int r, int c) { return r * PITCH + 16 * (c ^ swz(r)); }
};

template <int H, int DQK, int DV>
struct MqaCfg {
    static constexpr int THREADS = 512;        // 4 logit waves + 4 value waves (2 groups x 2 halves)
    static constexpr int NW = 4;
    static constexpr int NHH = (H + 63) / 64;  // workgroups per query row, 64 heads each
    static constexpr int KS = DQK / 16;        // k-slices of the logit product
    static constexpr int KSV = DV / 16;        // k-slices that fall in the value region
    static constexpr int KSV2 = KSV / 2;       // value slices per half
    static constexpr int R = KS - KSV;         // rope slices
    static constexpr int RH = (R + 1) / 2;     // rope slices of half 0 (half 1 takes the rest)
    static constexpr int KS0 = KSV2 + RH;      // slices of half 0 (the larger half)
    static constexpr int VT = DV / 32;         // 32-wide value tiles
    static constexpr int VT0 = VT / 2;         // value tiles per half
    using RV = Region<DV * 2 / 16>;
    using RR = Region<(DQK - DV) * 2 / 16>;
    static constexpr int BUF = RV::BYTES + RR::BYTES;
    static constexpr int INSTRS = RV::INSTRS + RR::INSTRS;
    static constexpr int ROW_BYTES = DQK * 2;           // bytes of one latent row in memory
    static constexpr int VBYTES = DV * 2;               // bytes of its value part
    static constexpr int LOADS_PER_WAVE = INSTRS / NW;  // direct loads per wave and block (min)
    static constexpr bool EVEN = R % 2 == 0;            // both halves have KS0 slices
    static constexpr int QK_AHEAD = KS0 < 9 ? KS0 : 9;  // logit operand loads kept in flight
    // Per-lane LDS offsets are kept for TLQ logit slices and TLV value tiles only: the rest
    // differ by a multiple of the swizzle period and reach the reads as immediate offsets.
    static constexpr int W = RV::SWZ_BITS;
    static constexpr int TLQ = (KSV % (1 << W) == 0 && KSV2 % (1 << (W - 1)) == 0) ? (1 << (W - 1)) : KSV2;
    static constexpr int TLV = ((4 * VT0) % (1 << W) == 0 && VT0 % (1 << (W - 2)) == 0) ? (1 << (W - 2)) : VT0;
    static_assert(DQK % 16 == 0 && DV % 64 == 0, "unsupported latent widths");
    static_assert(NHH <= 2, "at most 128 heads");
};

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keeps an MFMA accumulator tile in AGPRs across a join of control flow, so that the register
// allocator does not route the loop-carried tile through VGPRs on every iteration.
__device__ __forceinline__ void pin_agpr(v16f& x) { asm volatile("" : "+a"(x)); }

// Keeps a query fragment (an MFMA B operand, read as is from AGPRs) out of the VGPRs.
__device__ __forceinline__ void pin_agpr(v8bf& x) { asm volatile("" : "+a"(x)); }

// x *= alpha on a tile held in AGPRs, element by element through one VGPR (VALU instructions
// cannot read AGPRs), so the tile never has to live in VGPRs.
__device__ __forceinline__ void scale_agpr(v16f& x, float alpha) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float e = x[r], t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n"
            "v_mul_f32 %1, %2, %1\n"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(e), "=&v"(t)
            : "v"(alpha));
        x[r] = e;
    }
}


__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// Row and LDS byte offset of the 16-byte piece that lane `lane` moves in direct-load
// instruction I of a block (the hardware adds 16 * lane to the instruction's LDS base), and
// the byte column of the latent row it fetches.
template <class C>
__device__ __forceinline__ void piece_of(int I, int lane, int& r, int& col, int& base) {
    using RV = typename C::RV;
    using RR = typename C::RR;
    const bool rope = I >= RV::INSTRS;
    const int Ir = rope ? I - RV::INSTRS : I;
    const int rows = rope ? RR::ROWS_PER_INSTR : RV::ROWS_PER_INSTR;
    const int ncol = 64 / rows;  // chunks per row in this region
    r = Ir * rows + lane / ncol;
    const int p = lane % ncol;
    const int c = rope ? (p ^ RR::swz(r)) : (p ^ RV::swz(r));
    col = (rope ? C::VBYTES : 0) + 16 * c;
    base = rope ? RV::BYTES + Ir * 1024 : Ir * 1024;
}


// Issues the direct global->LDS loads of one block of kBlk latent rows into the buffer at
// LDS address `buf`; `offs` points at the block's kBlk row byte offsets in LDS (empty slots
// hold 0, i.e. row 0 of the sequence, and are zeroed by zero_empty_rows once landed).  The
// wave's instruction slots are fixed at compile time (I = wv + NW*k), so the sequence is
// fully unrolled: all offset reads first, then the loads.  Every wave issues the same number
// of instructions for every block, so the wait can count them.
template <class C>
__device__ __forceinline__ void issue_block(uint32_t buf, const uint8_t* kvb, const uint32_t* offs,
                                            int wv, int lane) {
    constexpr int MAXK = (C::INSTRS + C::NW - 1) / C::NW;
    constexpr bool FULL = C::INSTRS % C::NW == 0;  // every wave has MAXK slots
    uint32_t o[MAXK];
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
        const int I = wv + C::NW * k;
        int r, col, base;
        piece_of<C>(I, lane, r, col, base);
        o[k] = (FULL || I < C::INSTRS) ? offs[r] + col : 0u;
    }
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
        const int I = wv + C::NW * k;
        if (FULL || I < C::INSTRS) {
            int r, col, base;
            piece_of<C>(I, lane, r, col, base);
            dma16(kvb, o[k], buf + base);
        }
    }
}

// Zeroes the pieces of empty rows that this wave loaded itself (so the direct load has
// landed before the store, in this wave's program order).  Empty rows then contribute exact
// zeros to both products.
template <class C>
__device__ __forceinline__ void zero_empty_rows(uint32_t buf, uint32_t vmask, int wv, int lane) {
    constexpr int MAXK = (C::INSTRS + C::NW - 1) / C::NW;
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
        const int I = wv + C::NW * k;
        if (I < C::INSTRS) {
            int r, col, base;
            piece_of<C>(I, lane, r, col, base);
            if (!((vmask >> r) & 1u)) lds_write16(buf + base + 16 * lane, (v4i){0, 0, 0, 0});
        }
    }
}


template <int H, int DQK, int DV, bool SPLIT>
__global__ __launch_bounds__(512, 1) void sparse_mqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int topk, uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, RowMap map, int n_rows, int n_split, float sm_log2) {
    using C = MqaCfg<H, DQK, DV>;
    using RV = typename C::RV;
    using RR = typename C::RR;
    __shared__ __attribute__((aligned(16))) uint8_t lds[3 * C::BUF];
    __shared__ uint32_t lofs[kMaxTopk];            // byte offset of each selected row (0 if empty)
    __shared__ uint32_t lmask[kMaxTopk / kBlk];    // per block: bit j = slot j holds a row
    // partial S^T tiles: [block parity][group][half][r/4][lane][r%4]
    __shared__ __attribute__((aligned(16))) float sx[2][2][2][4][kWave][4];

    // Work item.  With two workgroups per row (64 heads each) the pair is issued 8 ids
    // apart, i.e. onto the same XCD, so the second gather of each latent row hits its L2.
    int row, hh;
    if (C::NHH == 1) {
        row = blockIdx.x;
        hh = 0;
    } else {
        const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
        row = (slot >> 1) * 8 + x;
        hh = slot & 1;
    }
    if (row >= n_rows) return;
    const int split = SPLIT ? blockIdx.y : 0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const bool logit_wave = wv < 4;  // waves 0-3: logits and softmax; 4-7: value product
    const int w4 = wv & 3;
    const int hg = w4 & 1;  // head group: 32 heads
    const int dp = w4 >> 1;  // half: of the logit dims (logit waves) or value tiles (value waves)
    const RowInfo ri = row_info(map, row);
    const int per = SPLIT ? (((topk + n_split - 1) / n_split + kBlk - 1) / kBlk) * kBlk : topk;
    const int j0 = split * per;
    const int j1 = min(topk, j0 + per);
    const int nblk = j1 > j0 ? (j1 - j0 + kBlk - 1) / kBlk : 0;
    const int32_t* irow = idx + (int64_t)row * topk;
    const uint8_t* kvb = (const uint8_t*)(kv + (int64_t)ri.kbase * DQK);
    const int head = hh * 64 + hg * 32 + (lane & 31);
    const int half = lane >> 5;
    const int mi = lane & 31;
    const int j16 = lane & 15;
    const uint32_t lds0 = lds_addr(lds);

    // Selected rows of the work item, staged in LDS once: byte offsets (row 0 for an empty
    // slot) and per-block occupancy masks.  A row's offset must fit in 31 bits.
    for (int j = tid; j < nblk * kBlk; j += C::THREADS) {
        const int id = j0 + j < j1 ? irow[j0 + j] : -1;
        lofs[j] = id >= 0 ? (uint32_t)id * (uint32_t)C::ROW_BYTES : 0u;
        const uint64_t m = __ballot(id >= 0);
        if (lane == 0) lmask[j >> 5] = (uint32_t)m;
        if (lane == 32) lmask[j >> 5] = (uint32_t)(m >> 32);
    }
    __syncthreads();

    // LDS address of block blk's buffer.  Passed through readfirstlane so that it stays one
    // opaque scalar per step: otherwise the compiler strength-reduces it into per-lane
    // induction variables and loses the immediate offsets of the reads.
    auto buf_of = [&](int blk) {
        return (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(blk % 3) * C::BUF);
    };
    // Per-lane addresses base + off, made opaque so that constant parts added afterwards go
    // into the instructions' offset field instead of into one add per read.
    auto opaque = [](uint32_t x) {
        asm volatile("" : "+v"(x));
        return x;
    };

    // Pipeline over the blocks (three LDS buffers for the gathered rows, two for the partial
    // logits), one barrier per step.  Step b:
    //   logit waves:  partial logits of block b+1 over their half of the dims (direct loads of
    //                 block b+2 between the MFMAs), published to LDS; then wait for block b+2
    //   value waves:  logits of block b from both published partials, online softmax, and
    //                 the value MFMAs of block b
    //   barrier: block b+1's partials and block b+2's rows are visible; block b's buffer is free
    // A logit wave and a value wave share each SIMD, so the softmax VALU work of one runs under
    // the other's MFMAs.
    if (logit_wave) {
        // ---------------- partial logits ----------------
        // Logit k-slices of this wave's half: value slices dp*KSV2 + i (i < KSV2), then rope
        // slices KSV + dp*RH + j.  Lane l holds head 64*hh + 32*hg + l%32, dims 8*(l/32) .. +7
        // of each slice.  Loaded unconditionally from clamped addresses and masked afterwards,
        // so all the loads fly together; then moved to AGPRs (MFMA B operands are read from
        // there).
        const int nrope = min(C::RH, C::R - dp * C::RH);
        const int nks = C::KSV2 + nrope;
        v8bf qf[C::KS0];
        {
            const uint16_t* qp = q + ((int64_t)ri.qrow * H + (head < H ? head : 0)) * DQK + 8 * half;
            v4i v[C::KS0];
#pragma unroll
            for (int i = 0; i < C::KS0; ++i) {
                const int ks = i < C::KSV2 ? dp * C::KSV2 + i : C::KSV + dp * C::RH + (i - C::KSV2);
                v[i] = *(const v4i*)(qp + 16 * min(ks, C::KS - 1));
            }
#pragma unroll
            for (int i = 0; i < C::KS0; ++i) {
                const bool ok = head < H && i < nks;
                qf[i] = __builtin_bit_cast(v8bf, ok ? v[i] : (v4i){0, 0, 0, 0});
                pin_agpr(qf[i]);
            }
        }
        // Block row held by MFMA row i = l%32 of the logit product: lanes of each 32-lane half
        // must own 8 consecutive block rows per 16-row k-slice of the value product.
        const int srow = 16 * (mi >> 4) + 8 * ((mi >> 2) & 1) + 4 * ((mi >> 3) & 1) + (mi & 3);
        // Per-lane LDS offsets within a block buffer: logit operand of value slice i at
        // qoff[i % TLQ] + 32*TLQ*(i / TLQ), of rope slice j at roff[j].
        uint32_t qoff[C::TLQ], roff[C::RH];
#pragma unroll
        for (int i = 0; i < C::TLQ; ++i) qoff[i] = RV::chunk(srow, dp * C::KSV + 2 * i + half);
#pragma unroll
        for (int j = 0; j < C::RH; ++j) roff[j] = RV::BYTES + RR::chunk(srow, 2 * (dp * C::RH + j) + half);
        const uint32_t sx_own0 = lds_addr(&sx[0][hg][dp][0][lane][0]);
        constexpr uint32_t SX_PAR = 2 * 2 * 4 * kWave * 4 * 4;  // bytes per parity

        auto land = [&](int blk) {  // block blk's loads have landed for this wave: zero its empty rows
            const uint32_t vm = lmask[blk];
            if (vm != 0xffffffffu) zero_empty_rows<C>(buf_of(blk), vm, w4, lane);
        };
        auto qk_read = [&](const uint32_t (&qa)[C::TLQ], const uint32_t (&ra)[C::RH], int i) {
            if (i < C::KSV2) return lds_read16(qa[i % C::TLQ] + 32 * C::TLQ * (i / C::TLQ));
            return lds_read16(ra[i - C::KSV2]);
        };
        // Partial S^T of block `nb` over this wave's dims, published for the value waves; the
        // direct loads of block `db` (when DMA) go out between the MFMAs.
        constexpr int MAXK = (C::INSTRS + C::NW - 1) / C::NW;
        constexpr int AHEAD = C::KS0 < 6 ? C::KS0 : 6;
        auto logits = [&](int nblk_idx, int db, auto DMA) {
            constexpr bool do_dma = decltype(DMA)::value;
            const uint32_t nb = buf_of(nblk_idx);
            uint32_t o[MAXK];
            uint32_t dbuf = 0;
            if constexpr (do_dma) {
                dbuf = buf_of(db);
#pragma unroll
                for (int k = 0; k < MAXK; ++k) {
                    const int I = w4 + C::NW * k;
                    int r, col, base;
                    piece_of<C>(I, lane, r, col, base);
                    o[k] = (C::INSTRS % C::NW == 0 || I < C::INSTRS) ? lofs[db * kBlk + r] + col : 0u;
                }
            }
            auto dma_k = [&](int k) {
                const int I = w4 + C::NW * k;
                if (C::INSTRS % C::NW == 0 || I < C::INSTRS) {
                    int r, col, base;
                    piece_of<C>(I, lane, r, col, base);
                    dma16(kvb, o[k], dbuf + base);
                }
            };
            uint32_t qa[C::TLQ], ra[C::RH];
#pragma unroll
            for (int i = 0; i < C::TLQ; ++i) qa[i] = opaque(nb + qoff[i]);
#pragma unroll
            for (int j = 0; j < C::RH; ++j) ra[j] = opaque(nb + roff[j]);
            v4i av[C::KS0];
#pragma unroll
            for (int i = 0; i < AHEAD; ++i) av[i] = qk_read(qa, ra, i);
            v16f sacc = (v16f){};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < C::KS0; ++i) {
                if (i + AHEAD < C::KS0) av[i + AHEAD] = qk_read(qa, ra, i + AHEAD);
                if (C::EVEN || i < nks) sacc = mfma_bf16(__builtin_bit_cast(v8bf, av[i]), qf[i], sacc);
                if constexpr (do_dma)
                    if (i < MAXK) dma_k(i);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (do_dma) {
#pragma unroll
                for (int k = C::KS0; k < MAXK; ++k) dma_k(k);
            }
            const uint32_t so = sx_own0 + (uint32_t)(nblk_idx & 1) * SX_PAR;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                lds_write16(so + 1024 * r4,
                            __builtin_bit_cast(v4i, (v4f){sacc[4 * r4], sacc[4 * r4 + 1], sacc[4 * r4 + 2],
                                                          sacc[4 * r4 + 3]}));
        };

        if (nblk > 0) {
            issue_block<C>(buf_of(0), kvb, lofs, w4, lane);
            if (nblk > 1) issue_block<C>(buf_of(1), kvb, lofs + kBlk, w4, lane);
            if (nblk > 1) wait_loads<C::LOADS_PER_WAVE>();
            else wait_loads<0>();
            land(0);
            lds_barrier();  // block 0 visible
            logits(0, 0, std::false_type{});
            if (nblk > 1) {
                wait_loads<0>();
                land(1);
            }
            lds_barrier();  // block 0's partials and block 1's rows visible
            for (int blk = 0; blk < nblk; ++blk) {
                if (blk + 1 < nblk) {
                    if (blk + 2 < nblk) logits(blk + 1, blk + 2, std::true_type{});
                    else logits(blk + 1, 0, std::false_type{});
                }
                if (blk + 2 < nblk) {
                    wait_loads<0>();
                    land(blk + 2);
                }
                lds_barrier();  // end of step blk
            }
        }
        return;
    }

    // ---------------- softmax and value product ----------------
    v16f oacc[C::VT0];
#pragma unroll
    for (int vt = 0; vt < C::VT0; ++vt) oacc[vt] = (v16f){};
    float m_run = -INFINITY;  // running max of the base-2 logits of this lane's head
    float l_run = 0.f;        // running sum over this lane's half of the block rows
    // value operand (tr16 read) of 16-row slice u, row quad h, tile t at
    // voff[u][h][t % TLV] + 64*TLV*(t / TLV); tr16 source lane j of each 16-lane group points
    // at block row 16u + 8*half + j/4 (+4 for h = 1) and value columns cl*8 + sub/2 .. +3
    uint32_t voff[2][2][C::TLV];
    {
        const int vsub = 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
        const int cl = vsub >> 3, sub = (vsub & 7) * 2;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int t = 0; t < C::TLV; ++t)
                    voff[u][h][t] = RV::chunk(16 * u + 8 * half + (j16 >> 2) + 4 * h,
                                              4 * (dp * C::VT0 + t) + cl) + sub;
    }
    const uint32_t sx0 = lds_addr(&sx[0][hg][0][0][lane][0]);
    const uint32_t sx1 = lds_addr(&sx[0][hg][1][0][lane][0]);
    constexpr uint32_t SX_PAR = 2 * 2 * 4 * kWave * 4 * 4;  // bytes per parity

    // Logits of block blk from the two published partials (the same sum in the same order in
    // both value waves of a group, so both hold identical softmax state), masked rows, running
    // max with lazy rescale of O, then P^T as the two bf16 B operands (slices u = 0, 1).
    auto softmax = [&](int blk, v8bf (&pf)[2]) {
        const uint32_t po = (uint32_t)(blk & 1) * SX_PAR;
        float z[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const v4f a = __builtin_bit_cast(v4f, lds_read16(sx0 + po + 1024 * r4));
            const v4f b = __builtin_bit_cast(v4f, lds_read16(sx1 + po + 1024 * r4));
#pragma unroll
            for (int e = 0; e < 4; ++e) z[4 * r4 + e] = a[e] + b[e];
        }
        const uint32_t vmask = lmask[blk];
        if (vmask != 0xffffffffu) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int slot = 16 * (r >> 3) + 8 * half + (r & 7);
                if (!((vmask >> slot) & 1u)) z[r] = -INFINITY;
            }
        }
        // max as a tree (med3(a, b, +inf) = max(a, b) for the non-NaN logits here; unlike
        // fmaxf it needs no quieting of its inputs first), then across the lane halves with a
        // lane swap instead of an LDS permute
        auto mx = [](float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); };
        float m8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) m8[r] = mx(z[2 * r], z[2 * r + 1]);
        float mb = mx(mx(mx(m8[0], m8[1]), mx(m8[2], m8[3])), mx(mx(m8[4], m8[5]), mx(m8[6], m8[7])));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
        mb = mx(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sm_log2;
        const bool bump = mb > m_run + kRescaleGap;
        if (__ballot(bump) != 0ull) {
            const bool fresh = m_run == -INFINITY;
            const float m_new = bump ? mb : m_run;
            const float alpha = fresh ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            if (__ballot(!fresh) != 0ull) {
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // MFMA results settle
#pragma unroll
                for (int vt = 0; vt < C::VT0; ++vt) scale_agpr(oacc[vt], alpha);
                asm volatile("s_nop 4" ::: "memory");  // before the next MFMA reads them
            }
        }
        // p = 2^(sm_log2 * z - m_run); masked rows give exact zeros, also while no row has been
        // seen (m_run = -inf is then replaced by 0)
        const float mref = m_run == -INFINITY ? 0.f : m_run;
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(z[8 * u + e], sm_log2, -mref));
                ls += pv;
                pf[u][e] = (__bf16)pv;
            }
        l_run += ls;
    };
    // O^T += V^T P^T over this wave's value tiles.
    auto values = [&](int blk, const v8bf (&pf)[2]) {
        const uint32_t cb = buf_of(blk);
        uint32_t va_[2][2][C::TLV];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int t = 0; t < C::TLV; ++t) va_[u][h][t] = opaque(cb + voff[u][h][t]);
        auto vread = [&](int u, int t) {
            const uint32_t imm = 64 * C::TLV * (t / C::TLV);
            const v4s lo = ds_read_tr16(va_[u][0][t % C::TLV] + imm);
            const v4s hi = ds_read_tr16(va_[u][1][t % C::TLV] + imm);
            const v2i l2 = __builtin_bit_cast(v2i, lo), h2 = __builtin_bit_cast(v2i, hi);
            return __builtin_bit_cast(v8bf, (v4i){l2.x, l2.y, h2.x, h2.y});
        };
        v8bf va[2][C::VT0];
#pragma unroll
        for (int t = 0; t < C::VT0; ++t) va[0][t] = vread(0, t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < C::VT0; ++t) {
            va[1][t] = vread(1, t);
            oacc[t] = mfma_bf16(va[0][t], pf[0], oacc[t]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < C::VT0; ++t) oacc[t] = mfma_bf16(va[1][t], pf[1], oacc[t]);
#pragma unroll
        for (int vt = 0; vt < C::VT0; ++vt) pin_agpr(oacc[vt]);
    };
    if (nblk > 0) {
        lds_barrier();  // block 0 visible
        lds_barrier();  // block 0's partials and block 1's rows visible
        for (int blk = 0; blk < nblk; ++blk) {
            v8bf pf[2];
            softmax(blk, pf);
            values(blk, pf);
            lds_barrier();  // end of step blk
        }
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32);

    // ---- epilogue ----
    if (head >= H) return;
    if (!SPLIT) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* op = out + ((int64_t)ri.qrow * H + head) * DV;
#pragma unroll
        for (int t = 0; t < C::VT0; ++t)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int v = 32 * (dp * C::VT0 + t) + 8 * rb + 4 * half;
                const uint32_t w0 = (uint32_t)f2bf(oacc[t][4 * rb + 0] * inv) |
                                    ((uint32_t)f2bf(oacc[t][4 * rb + 1] * inv) << 16);
                const uint32_t w1 = (uint32_t)f2bf(oacc[t][4 * rb + 2] * inv) |
                                    ((uint32_t)f2bf(oacc[t][4 * rb + 3] * inv) << 16);
                *(v2i*)(op + v) = (v2i){(int)w0, (int)w1};
            }
        if (lse != nullptr && half == 0 && dp == 0)
            lse[(int64_t)ri.qrow * H + head] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t item = (int64_t)row * n_split + split;
        float* op = part_o + (item * H + head) * DV;
#pragma unroll
        for (int t = 0; t < C::VT0; ++t)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int v = 32 * (dp * C::VT0 + t) + 8 * rb + 4 * half;
                *(v4f*)(op + v) = (v4f){oacc[t][4 * rb + 0], oacc[t][4 * rb + 1],
                                        oacc[t][4 * rb + 2], oacc[t][4 * rb + 3]};
            }
        if (half == 0 && dp == 0) part_ml[item * H + head] = make_float2(m_run, l_tot);
    }
}

// Merges the split partials of each (row, head): weights 2^(m_j - M) on the unnormalised
// partial outputs and sums.
template <int H, int DV>
__global__ __launch_bounds__(256) void mqa_combine_kernel(const float* __restrict__ part_o,
                                                          const float2* __restrict__ part_ml,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse, RowMap map,
                                                          int n_rows, int n_split) {
    const int row = blockIdx.x;
    const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (row >= n_rows || head >= H) return;
    const int lane = threadIdx.x & 63;
    const RowInfo ri = row_info(map, row);
    float M = -INFINITY;
    for (int j = 0; j < n_split; ++j) M = fmaxf(M, part_ml[((int64_t)row * n_split + j) * H + head].x);
    float L = 0.f;
    float acc[DV / 64];
#pragma unroll
    for (int i = 0; i < DV / 64; ++i) acc[i] = 0.f;
    if (M != -INFINITY) {
        for (int j = 0; j < n_split; ++j) {
            const int64_t item = (int64_t)row * n_split + j;
            const float2 ml = part_ml[item * H + head];
            if (ml.x == -INFINITY) continue;
            const float wgt = exp2f(ml.x - M);
            L += ml.y * wgt;
            const float* op = part_o + (item * H + head) * DV;
#pragma unroll
            for (int i = 0; i < DV / 64; ++i) acc[i] += wgt * op[lane + 64 * i];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* o = out + ((int64_t)ri.qrow * H + head) * DV;
#pragma unroll
    for (int i = 0; i < DV / 64; ++i) o[lane + 64 * i] = f2bf(acc[i] * inv);
    if (lse != nullptr && lane == 0)
        lse[(int64_t)ri.qrow * H + head] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Grid width: one workgroup per (row, 64-head half); rows are padded to a multiple of 8 when
// a row has two halves so the XCD-pairing map stays in range (padding ids exit at once).
template <class C>
int grid_x(int n_rows) {
    return C::NHH == 1 ? n_rows : ((n_rows + 7) / 8) * 8 * C::NHH;
}

template <int H, int DQK, int DV>
hipError_t launch_t(const MqaArgs& a, const RowMap& map, int n_rows, int n_split, void* ws,
                    hipStream_t st) {
    using C = MqaCfg<H, DQK, DV>;
    const float sm_log2 = a.sm_scale * 1.4426950408889634f;
    if (n_split <= 1) {
        hipLaunchKernelGGL((sparse_mqa_kernel<H, DQK, DV, false>), dim3(grid_x<C>(n_rows)), dim3(C::THREADS), 0,
                           st, a.q, a.kv, a.idx, a.topk, a.out, a.lse, nullptr, nullptr, map, n_rows,
                           1, sm_log2);
        return hipGetLastError();
    }
    float* part_o = (float*)ws;
    float2* part_ml = (float2*)(part_o + (size_t)n_rows * n_split * H * DV);
    hipLaunchKernelGGL((sparse_mqa_kernel<H, DQK, DV, true>), dim3(grid_x<C>(n_rows), n_split), dim3(C::THREADS),
                       0, st, a.q, a.kv, a.idx, a.topk, a.out, a.lse, part_o, part_ml, map, n_rows,
                       n_split, sm_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mqa_combine_kernel<H, DV>), dim3(n_rows, (H + 3) / 4), dim3(256), 0, st,
                       part_o, part_ml, a.out, a.lse, map, n_rows, n_split);
    return hipGetLastError();
}

}  // namespace

size_t mqa_split_bytes(Shape shape, int n_rows, int n_split) {
    if (n_split <= 1) return 0;
    const size_t H = shape == Shape::Prod ? 128 : 8;
    const size_t DV = shape == Shape::Prod ? 512 : 64;
    return (size_t)n_rows * n_split * H * (DV * sizeof(float) + sizeof(float2));
}

hipError_t launch_sparse_mqa(const MqaArgs& a, const RowMap& map, int n_rows, int n_split,
                             void* ws, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    if (a.shape == Shape::Prod) return launch_t<128, 576, 512>(a, map, n_rows, n_split, ws, st);
    return launch_t<8, 80, 64>(a, map, n_rows, n_split, ws, st);
}

}  // namespace dsa
