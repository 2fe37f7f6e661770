// Sparse MQA over the MLA latent cache on gfx950 (core attention of DSA on the top-k rows;
// DeepSeek-V3.2 explained, sections 二.1 and 二.4; DeepSeek-V3.2-Exp overview, module table).
//
// For query row t and head h, over the selected latent rows c_s (576 = 512 latent + 64
// rope; every head shares the row):
//     z_s = sm * <q[t,h,:], c_s>,  out[t,h,:] = sum_s softmax(z)_s c_s[:512],  lse = ln sum e^z
//
// Slots: a row's key positions come from its index row (any slot may be -1), from the first
// min(k, p + 1) slots of an index row whose valid slots come first (the top-k output), or,
// for dense causal attention (the short-sequence masked-MHA mode of the DeepSeek-V3.2-Exp
// deep dive, section 4), from the positions 0 .. p themselves.
//
// Work decomposition: one workgroup = one query row x 64 heads (two workgroups per row of 128
// heads, issued 8 ids apart so both run on the same XCD and the second gather of each latent
// row hits its L2); with few rows, each row's slots are also split over workgroups whose
// (m, l, O) partials a combine kernel merges.  Per block of 32 slots the 8 waves (wave w
// shares its SIMD with wave w + 4) work in three roles:
//   waves 0, 1  logits S^T = C Q^T (v_mfma_f32_32x32x16_bf16; A = latent rows from LDS,
//               B = the query heads of one 32-head group, kept in registers) over the first
//               half of the 576 dims; then the sum with the other half, masking, the base-2
//               online softmax (lane l owns head l % 32; O is rescaled only when a block max
//               exceeds the running max by more than 64) and P^T published to LDS;
//   waves 4, 5  the other half of the same group's logits, handed over through LDS and
//               computed one block ahead, so their MFMAs run beside the softmax of waves 0, 1
//               on the same SIMD; they also issue the direct global->LDS loads of the block
//               three steps ahead into a four-block ring;
//   waves 2, 3, 6, 7  O^T += V^T P^T for all 64 heads over a quarter of the 512 value dims,
//               A = value columns read by ds_read_b64_tr_b16 straight from the row-major block.
// LDS rows are XOR-swizzled in 16-byte chunks so that the 16 rows read together by an A
// operand, and the 4 consecutive rows of a transpose read, fall in distinct bank groups.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kBlk = 32;            // selected rows per LDS block
// Base-2 headroom of the lazy running max before O is rescaled.  A rescale costs the value
// waves ~2,000 cycles (their 128 accumulator AGPRs pass through VGPRs), and each one is taken
// for a whole wave of 64 heads, so a small gap rescales at almost every block once the heads
// meet their large logits in different blocks.  With the running max at most 64 below the
// true max, p <= 2^64, l <= n * 2^64 and |O| <= n * 2^64 * max|v| stay finite in fp32 for
// n <= 2^17 slots and |v| < 2^47; terms the lag pushes below fp32's range are below 2^-126 of
// the largest p, which is at least 1.
constexpr float kRescaleGap = 64.f;

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
    // 8 waves in three roles; wave w shares its SIMD with wave w + 4.
    //   waves 0, 1        logits over the first half of the dims for head group 0 / 1
    //                     (32 heads each), then the online softmax of the group
    //   waves 4, 5        logits over the second half of the dims of the same group,
    //                     handed to wave w - 4 through LDS, and most of the direct
    //                     global->LDS loads of the gathered rows
    //   waves 2, 3, 6, 7  value product (64 heads x a quarter of the DV dims each); waves
    //                     3, 6, 7 also issue the rest of the direct loads
    // Splitting each group's logits over two waves of one SIMD halves the LDS operand bytes
    // each wave must read per block (a single wave's LDS read rate is the limit otherwise).
    static constexpr int THREADS = 512;
    static constexpr int NDW = 2;              // helper waves issuing direct loads
    static constexpr int NBUF = 4;             // gathered blocks resident in LDS
    static constexpr int RING = 4;             // blocks of row offsets staged in LDS
    static constexpr int NHH = (H + 63) / 64;  // workgroups per query row, 64 heads each
    static constexpr int KS = DQK / 16;        // k-slices of the logit product
    static constexpr int KH = (KS + 1) / 2;    // slices of the first half (waves 0, 1)
    static constexpr int KSV = DV / 16;        // k-slices that fall in the value region
    static constexpr int VT = DV / 32;         // 32-wide value tiles
    static constexpr int NVW = VT < 4 ? VT : 4;  // value waves with product work
    static constexpr int VTW = VT / NVW;         // value tiles per value wave
    using RV = Region<DV * 2 / 16>;
    using RR = Region<(DQK - DV) * 2 / 16>;
    static constexpr int BUF = RV::BYTES + RR::BYTES;
    static constexpr int INSTRS = RV::INSTRS + RR::INSTRS;
    static constexpr int ROW_BYTES = DQK * 2;              // bytes of one latent row in memory
    static constexpr int VBYTES = DV * 2;                  // bytes of its value part
    // Direct-load instructions of a block: waves 4, 5 issue the first HLOAD of them, value
    // waves 3, 6, 7 the last VLOAD (blocks of the production shape only: small test shapes
    // leave every load to waves 4, 5)
    static constexpr int NVL = 3;                                    // value waves that load
    static constexpr int VLOAD = (INSTRS >= 24 && NVW == 4) ? 6 : 0;
    static constexpr int HLOAD = INSTRS - VLOAD;
    static constexpr int MAXK = (HLOAD + NDW - 1) / NDW;  // direct loads per helper wave and block
    static constexpr int LOADS_PER_WAVE = HLOAD / NDW;    // fewest of a helper wave per block
    static constexpr int VMAXK = VLOAD > 0 ? VLOAD / NVL : 1;  // per loading value wave and block
    static constexpr int QK_AHEAD = KH < 9 ? KH : 9;       // logit operand reads kept in flight
    // Per-lane LDS offsets are kept for TLQ logit slices and TLV value tiles only: the rest
    // differ by a multiple of the swizzle period and reach the reads as immediate offsets.
    static constexpr int W = RV::SWZ_BITS;
    static constexpr int TLQ = KSV % (1 << (W - 1)) == 0 ? (1 << (W - 1)) : KSV;
    static constexpr int TLV = ((4 * VTW) % (1 << W) == 0 && VTW % (1 << (W - 2)) == 0) ? (1 << (W - 2)) : VTW;
    static_assert(DQK % 16 == 0 && DV % 64 == 0 && VT % NVW == 0, "unsupported latent widths");
    static_assert(NHH <= 2, "at most 128 heads");
    static_assert(3 * MAXK <= 63, "direct loads of three blocks must fit the load counter");
    static_assert(VLOAD % NVL == 0, "loading value waves issue equal shares");
};

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keeps an MFMA accumulator tile in AGPRs across a join of control flow, so that the register
// allocator does not route the loop-carried tile through VGPRs on every iteration.
__device__ __forceinline__ void pin_agpr(v16f& x) { asm volatile("" : "+a"(x)); }

// Keeps a query fragment (an MFMA B operand, read as is from AGPRs) out of the VGPRs.
__device__ __forceinline__ void pin_agpr(v8bf& x) { asm volatile("" : "+a"(x)); }

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// max(a, b, c) for non-NaN inputs, as one instruction.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

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


// Issues direct global->LDS loads of one block of kBlk latent rows into the buffer at LDS
// address `buf`; `offs` points at the block's kBlk staged rows in LDS (empty slots hold row
// 0, and are zeroed by zero_pieces once landed).  Packed caches stage byte offsets from the
// sequence's first row (32 bits: a sequence is shorter than 2^32 / 1152 positions, checked on
// the host) and load from the scalar base kvb; paged caches stage pool rows and load from
// 64-bit per-lane addresses, so a page pool may exceed 4 GiB.  The calling wave owns
// instructions I = first + STEP*k (k < N) below lim, a pattern fixed at compile time per wave
// kind, so the sequence is fully unrolled: all offset reads first, then the loads.  FULL:
// every one of the N instructions is below lim.
template <class C, bool PAGED, int N, int STEP, bool FULL>
__device__ __forceinline__ void issue_pieces(uint32_t buf, const uint8_t* kvb, const uint32_t* offs,
                                             int first, int lim, int lane) {
    using Off = typename std::conditional<PAGED, const uint8_t*, uint32_t>::type;
    Off o[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int I = first + STEP * k;
        int r, col, base;
        piece_of<C>(I, lane, r, col, base);
        const bool live = FULL || I < lim;
        if constexpr (PAGED)
            o[k] = kvb + (live ? (uint64_t)offs[r] * C::ROW_BYTES + col : 0);
        else
            o[k] = live ? offs[r] + col : 0u;
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int I = first + STEP * k;
        if (FULL || I < lim) {
            int r, col, base;
            piece_of<C>(I, lane, r, col, base);
            if constexpr (PAGED)
                dma16_at(o[k], buf + base);
            else
                dma16(kvb, o[k], buf + base);
        }
    }
}

// Zeroes the pieces of empty rows that this wave loaded itself with issue_pieces (so the
// direct load has landed before the store, in this wave's program order).  Empty rows then
// contribute exact zeros to both products whatever row 0 of the sequence holds.
template <class C, int N, int STEP>
__device__ __forceinline__ void zero_pieces(uint32_t buf, uint32_t vmask, int first, int lim, int lane) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int I = first + STEP * k;
        if (I < lim) {
            int r, col, base;
            piece_of<C>(I, lane, r, col, base);
            if (!((vmask >> r) & 1u)) lds_write16(buf + base + 16 * lane, (v4i){0, 0, 0, 0});
        }
    }
}

// Waits until at most nb blocks' worth of direct loads (PER per block) of this wave are
// outstanding, nb chosen at run time among the counts the pipeline uses.
template <int PER>
__device__ __forceinline__ void wait_blocks_left(int nb) {
    if (nb >= 2) wait_loads<2 * PER>();
    else if (nb == 1) wait_loads<PER>();
    else wait_loads<0>();
}

template <int H, int DQK, int DV, bool SPLIT, bool PAGED>
__global__ __launch_bounds__(512, 1) void sparse_mqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int topk, uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, RowMap map, int n_rows, int n_split, float sm_log2, int mode) {
    using C = MqaCfg<H, DQK, DV>;
    using RV = typename C::RV;
    using RR = typename C::RR;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::NBUF * C::BUF];
    // P^T operands of the value product: [head group][16-row slice][lane] x 8 bf16
    __shared__ __attribute__((aligned(16))) v4i pl[2][2][kWave];
    // second-half logit tiles handed from waves 4, 5 to waves 0, 1: [group][r/4][lane][r%4]
    __shared__ __attribute__((aligned(16))) v4f sx[2][4][kWave];
    __shared__ float al[2][32];                // per-head rescale factor of O for the block
    __shared__ uint32_t rofs[C::RING][kBlk];   // row byte offsets of staged blocks
    __shared__ uint32_t rmask[C::RING];        // per staged block: bit j = slot j holds a row
    __shared__ float fin_l[2][32];             // softmax denominators at the end
    __shared__ int32_t rid[C::RING][kWave];    // index slots of blocks fetched ahead for staging

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
    const RowInfo ri = row_info(map, row);
    // slots of the row: all topk index slots, the first min(topk, p + 1) of a row whose
    // valid slots come first, or the p + 1 positions of dense causal attention
    const bool dense = mode == (int)IdxMode::Dense;
    const int jn = dense ? ri.pos + 1 : mode == (int)IdxMode::Front ? min(topk, ri.pos + 1) : topk;
    const int per = SPLIT ? (((jn + n_split - 1) / n_split + kBlk - 1) / kBlk) * kBlk : jn;
    const int j0 = split * per;
    const int j1 = min(jn, j0 + per);
    const int nblk = j1 > j0 ? (j1 - j0 + kBlk - 1) / kBlk : 0;
    const int32_t* irow = dense ? nullptr : idx + (int64_t)row * topk;
    // latent rows are addressed from the sequence's first row (packed caches) or from the
    // start of the page pool (paged caches)
    const uint8_t* kvb = (const uint8_t*)(PAGED ? kv : kv + (int64_t)ri.kbase * DQK);
    const int half = lane >> 5;
    const int mi = lane & 31;
    const int j16 = lane & 15;
    const uint32_t lds0 = lds_addr(lds);

    // Row offsets (packed: byte offset from the sequence's first row; paged: pool row) and
    // occupancy of block b, staged in ring slot b % RING: the first RING blocks here, the rest
    // by value wave 2 at the end of the step before the loads need them.  Slots that slot_row
    // rejects (-1, values
    // outside the sequence, page ids outside a pool of known size) are empty: row 0 is loaded
    // in their place and zeroed, so no load ever leaves the caches.
    auto stage = [&](int b, int id) {  // lanes 0..31 hold the ids of the block's slots
        const int64_t row = slot_row(map, ri, id);
        const bool ok = row >= 0;
        const uint32_t r = !ok ? 0u : PAGED ? (uint32_t)row : (uint32_t)id * (uint32_t)C::ROW_BYTES;
        if (lane < kBlk) rofs[b % C::RING][lane] = r;
        const uint64_t m = __ballot(ok);
        if (lane == 0) rmask[b % C::RING] = (uint32_t)m;
    };
    auto load_ids = [&](int b) {
        const int j = j0 + b * kBlk + lane;
        if (lane >= kBlk || j >= j1) return -1;
        return dense ? j : irow[j];
    };
    if (wv < C::RING && wv < nblk) stage(wv, load_ids(wv));
    __syncthreads();

    // LDS address of block blk's buffer.  Passed through readfirstlane so that it stays one
    // opaque scalar per step: otherwise the compiler strength-reduces it into per-lane
    // induction variables and loses the immediate offsets of the reads.
    auto buf_of = [&](int blk) {
        return (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(blk % C::NBUF) * C::BUF);
    };
    // Per-lane addresses base + off, made opaque so that constant parts added afterwards go
    // into the instructions' offset field instead of into one add per read.
    auto opaque = [](uint32_t x) {
        asm volatile("" : "+v"(x));
        return x;
    };

    // Pipeline over the blocks: a prologue step (-1) and steps 0 .. nblk-1, each with a
    // mid-step and an end barrier.  Step b:
    //   waves 0, 1:   first half of block b+1's logits; after the mid-step barrier, add the
    //                 second half, run the online softmax and publish block b+1's P^T and
    //                 rescale factors
    //   waves 4, 5:   hand over the second half of block b+1 (computed in step b-1); issue
    //                 their direct loads of block b+3 into the buffer block b-1 used and wait
    //                 for their loads of block b+2; after the mid-step barrier, the second
    //                 half of block b+2, so that these MFMAs run beside the softmax of waves
    //                 0, 1 on the same SIMD
    //   value waves:  read block b's P^T (published in step b-1); rescale O if needed and
    //                 O^T += V^T P^T for block b, half on each side of the mid-step barrier;
    //                 waves 3, 6, 7 wait for their loads of block b+2 before the mid-step
    //                 barrier and issue those of block b+3 after their second half
    //   end barrier:  block b+1's P^T is visible; block b's buffer is free
    if (wv != 2 && wv != 3 && wv != 6 && wv != 7) {
        // ---------------- logits (and softmax on waves 0, 1) ----------------
        const bool main = wv < 2;
        const int hg = wv & 1;
        const int head = hh * 64 + hg * 32 + mi;
        const int i0 = main ? 0 : C::KH;              // first logit slice of this wave
        const int nks = main ? C::KH : C::KS - C::KH;  // slices of this wave
        // Query fragments: lane l holds head 64*hh + 32*hg + l%32, dims 16 i + 8*(l/32) .. +7
        // of slice i = i0 + j.  Loaded unconditionally from clamped addresses and masked
        // afterwards, so all the loads fly together; then kept in AGPRs (MFMA B operands are
        // read from there).
        v8bf qf[C::KH];
        {
            const uint16_t* qp = q + ((int64_t)ri.qrow * H + (head < H ? head : 0)) * DQK + 8 * half;
            v4i v[C::KH];
#pragma unroll
            for (int j = 0; j < C::KH; ++j) v[j] = *(const v4i*)(qp + 16 * min(i0 + j, C::KS - 1));
#pragma unroll
            for (int j = 0; j < C::KH; ++j) {
                qf[j] = __builtin_bit_cast(v8bf, head < H && j < nks ? v[j] : (v4i){0, 0, 0, 0});
                pin_agpr(qf[j]);
            }
        }
        // Block row held by MFMA row i = l%32 of the logit product: lanes of each 32-lane half
        // must own 8 consecutive block rows per 16-row k-slice of the value product.
        const int srow = 16 * (mi >> 4) + 8 * ((mi >> 2) & 1) + 4 * ((mi >> 3) & 1) + (mi & 3);
        // LDS offsets of the logit operands within a block buffer, rebuilt for every read from
        // two lane constants per region (fewer live registers): value slice i sits at chunk
        // (2i + half) ^ swz(srow) = 2i ^ (half ^ swz(srow)) of row srow, plus 32*TLQ*(i / TLQ)
        // bytes for the slices past the swizzle period; rope slice j likewise in the rope region.
        const uint32_t qrow = srow * RV::PITCH, qx16 = 16 * (half ^ RV::swz(srow));
        const uint32_t rrow = RV::BYTES + srow * RR::PITCH, rx16 = 16 * (half ^ RR::swz(srow));
        auto qk_read = [&](uint32_t qb, uint32_t rb, int i) {
            if (i < C::KSV) {
                const int ii = i % C::TLQ;
                return lds_read16(((uint32_t)(32 * ii) ^ qx16) + qb + 32 * C::TLQ * (i / C::TLQ));
            }
            return lds_read16(((uint32_t)(32 * (i - C::KSV)) ^ rx16) + rb);
        };
        // This wave's half of the logit tile S^T of block blk (fp32, 16 values per lane).
        // The slice index is compile-time per wave kind, so the two kinds get separate code.
        auto half_logits = [&](int blk, auto MAIN) {
            constexpr bool M = decltype(MAIN)::value;
            constexpr int I0 = M ? 0 : C::KH;
            constexpr int N = M ? C::KH : C::KS - C::KH;
            constexpr int AH = C::QK_AHEAD < N ? C::QK_AHEAD : N;
            const uint32_t nb = buf_of(blk);
            const uint32_t qb = opaque(nb + qrow), rb = opaque(nb + rrow);
            v4i av[C::KH];
#pragma unroll
            for (int j = 0; j < AH; ++j) av[j] = qk_read(qb, rb, I0 + j);
            v16f sacc = (v16f){};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < N; ++j) {
                if (j + AH < N) av[j + AH] = qk_read(qb, rb, I0 + j + AH);
                sacc = mfma_bf16(__builtin_bit_cast(v8bf, av[j]), qf[j], sacc);
                __builtin_amdgcn_sched_barrier(0);
            }
            return sacc;
        };

        if (!main) {
            // -------- second half of the logits, handed over; direct loads --------
            const uint32_t sx_own = lds_addr(&sx[hg][0][lane]);
            auto publish = [&](const v16f& sp) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    lds_write16(sx_own + r4 * (kWave * 16),
                                __builtin_bit_cast(v4i, (v4f){sp[4 * r4], sp[4 * r4 + 1], sp[4 * r4 + 2],
                                                              sp[4 * r4 + 3]}));
            };
            // direct loads I = hg + 2k below HLOAD of each block
            auto land = [&](int blk) {  // block blk's loads have landed for this wave: zero its empty rows
                const uint32_t vm = rmask[blk % C::RING];
                if (vm != 0xffffffffu) zero_pieces<C, C::MAXK, C::NDW>(buf_of(blk), vm, hg, C::HLOAD, lane);
            };
            auto issue = [&](int blk) {
                issue_pieces<C, PAGED, C::MAXK, C::NDW, C::HLOAD % C::NDW == 0>(buf_of(blk), kvb,
                                                                                rofs[blk % C::RING], hg, C::HLOAD, lane);
            };
            if (nblk > 0) {
                issue(0);
                if (nblk > 1) issue(1);
                if (nblk > 2) issue(2);
                wait_blocks_left<C::LOADS_PER_WAVE>(min(nblk, 3) - 1);
                land(0);
                lds_barrier();  // block 0 visible
                publish(half_logits(0, std::false_type{}));
                if (nblk > 1) {
                    wait_blocks_left<C::LOADS_PER_WAVE>(min(nblk, 3) - 2);
                    land(1);
                }
                lds_barrier();  // mid-step of the prologue: block 1's rows visible
                v16f sp = nblk > 1 ? half_logits(1, std::false_type{}) : (v16f){};
                lds_barrier();  // end of the prologue
                for (int blk = 0; blk < nblk; ++blk) {
                    if (blk + 1 < nblk) publish(sp);  // block blk+1's half, computed in step blk-1
                    const bool more = blk + 3 < nblk;
                    if (more) issue(blk + 3);  // into the buffer block blk-1 used
                    if (blk + 2 < nblk) {
                        wait_blocks_left<C::LOADS_PER_WAVE>(more ? 1 : 0);
                        land(blk + 2);
                    }
                    lds_barrier();  // mid-step: block blk+2's rows visible
                    // block blk+2's half, under wave w-4's softmax of block blk+1
                    if (blk + 2 < nblk) sp = half_logits(blk + 2, std::false_type{});
                    lds_barrier();  // end of step blk
                }
            }
            lds_barrier();  // softmax denominators visible
            return;
        }

        // -------- first half, the sum of both halves, and the softmax --------
        const uint32_t sx_in = lds_addr(&sx[hg][0][lane]);
        const uint32_t p_own = lds_addr(&pl[hg][0][lane]);
        float m_run = -INFINITY;  // running max of the base-2 logits of this lane's head
        float l_run = 0.f;        // running sum over this lane's half of the block rows
        // Logits of block blk = own half + handed-over half (the same order in every step),
        // empty slots at -inf, online softmax, P^T and rescale factors published.
        auto softmax = [&](int blk, const v16f& s0) {
            float z[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const v4f b = __builtin_bit_cast(v4f, lds_read16(sx_in + r4 * (kWave * 16)));
#pragma unroll
                for (int e = 0; e < 4; ++e) z[4 * r4 + e] = s0[4 * r4 + e] + b[e];
            }
            const uint32_t vmask = rmask[blk % C::RING];
            if (vmask != 0xffffffffu) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int slot = 16 * (r >> 3) + 8 * half + (r & 7);
                    if (!((vmask >> slot) & 1u)) z[r] = -INFINITY;
                }
            }
            // max as a tree of three-input maxima (written out: the compiler would quiet every
            // input first), then across the lane halves with a lane swap instead of an LDS
            // permute
            auto mx = [](float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); };
            const float t0 = max3f(z[0], z[1], z[2]), t1 = max3f(z[3], z[4], z[5]);
            const float t2 = max3f(z[6], z[7], z[8]), t3 = max3f(z[9], z[10], z[11]);
            const float t4 = max3f(z[12], z[13], z[14]);
            const float m = max3f(max3f(t0, t1, t2), max3f(t3, t4, z[15]), t0);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
            const float mb = mx(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sm_log2;
            // lazy running max: O is rescaled only when a block max exceeds it by more than
            // kRescaleGap (alpha = 0 for the first block with a row, where O is still 0); both
            // lane halves hold the same values
            const bool bump = mb > m_run + kRescaleGap;
            const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mb) : 1.f;
            m_run = bump ? mb : m_run;
            l_run *= alpha;
            al[hg][mi] = alpha;
            // p = 2^(sm_log2 * z - m_run); masked rows give exact zeros, also while no row has
            // been seen (m_run = -inf is then replaced by 0)
            const float mref = m_run == -INFINITY ? 0.f : m_run;
            float ls = 0.f;
            v8bf pf[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(z[8 * u + e], sm_log2, -mref));
                    ls += pv;
                    pf[u][e] = (__bf16)pv;
                }
            l_run += ls;
#pragma unroll
            for (int u = 0; u < 2; ++u) lds_write16(p_own + u * (kWave * 16), __builtin_bit_cast(v4i, pf[u]));
        };
        if (nblk > 0) {
            lds_barrier();  // block 0 visible
            v16f s0 = half_logits(0, std::true_type{});
            lds_barrier();  // mid-step of the prologue: block 0's second half visible
            softmax(0, s0);
            lds_barrier();  // end of the prologue: block 0's P^T visible
            for (int blk = 0; blk < nblk; ++blk) {
                const bool next = blk + 1 < nblk;
                if (next) s0 = half_logits(blk + 1, std::true_type{});
                lds_barrier();  // mid-step: block blk+1's second half visible
                if (next) softmax(blk + 1, s0);
                lds_barrier();  // end of step blk
            }
        }
        const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        const float l_tot = __uint_as_float(sl[0]) + __uint_as_float(sl[1]);
        if (lane < 32) fin_l[hg][lane] = l_tot;
        lds_barrier();  // softmax denominators visible
        if (head >= H || lane >= 32) return;
        if (!SPLIT) {
            if (lse != nullptr)
                lse[(int64_t)ri.qrow * H + head] =
                    l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        } else {
            part_ml[((int64_t)row * n_split + split) * H + head] = make_float2(m_run, l_tot);
        }
        return;
    }

    // ---------------- value product ----------------
    const int vq = (wv & 1) + 2 * (wv >> 2);  // waves 2, 3, 6, 7 -> quarters 0..3
    const bool active = vq < C::NVW;          // has value tiles
    v16f oacc[2][C::VTW];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < C::VTW; ++t) oacc[g][t] = (v16f){};
    // value operand (tr16 read) of 16-row slice u, row quad h, tile t at
    // voff[h][t % TLV] + 64*TLV*(t / TLV) + 16*PITCH*u (rows 16 apart have the same swizzle);
    // tr16 source lane j of each 16-lane group points at block row 16u + 8*half + j/4 (+4 for
    // h = 1) and value columns cl*8 + sub/2 .. +3
    uint32_t voff[2][C::TLV];
    {
        const int vsub = 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
        const int cl = vsub >> 3, sub = (vsub & 7) * 2;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < C::TLV; ++t)
                voff[h][t] = RV::chunk(8 * half + (j16 >> 2) + 4 * h, 4 * (vq * C::VTW + t) + cl) + sub;
    }
    const uint32_t p_rd = lds_addr(&pl[0][0][lane]);

    // One 16-row slice u of block blk: O^T += V^T P^T over this wave's value tiles, both head
    // groups.
    auto values = [&](int blk, int u, const v8bf (&pf)[2][2]) {
        const uint32_t cb = buf_of(blk);
        uint32_t va_[2][C::TLV];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < C::TLV; ++t) va_[h][t] = opaque(cb + voff[h][t]);
        v8bf va[C::VTW];
#pragma unroll
        for (int t = 0; t < C::VTW; ++t) {
            const uint32_t imm = 64 * C::TLV * (t / C::TLV) + 16 * RV::PITCH * u;
            const v4s lo = ds_read_tr16(va_[0][t % C::TLV] + imm);
            const v4s hi = ds_read_tr16(va_[1][t % C::TLV] + imm);
            const v2i l2 = __builtin_bit_cast(v2i, lo), h2 = __builtin_bit_cast(v2i, hi);
            va[t] = __builtin_bit_cast(v8bf, (v4i){l2.x, l2.y, h2.x, h2.y});
        }
#pragma unroll
        for (int t = 0; t < C::VTW; ++t) {
            oacc[0][t] = mfma_bf16(va[t], pf[0][u], oacc[0][t]);
            oacc[1][t] = mfma_bf16(va[t], pf[1][u], oacc[1][t]);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int t = 0; t < C::VTW; ++t) pin_agpr(oacc[g][t]);
    };
    // P^T of block blk for both groups, and the rescale of O its softmax asked for.
    auto take_p = [&](v8bf (&pf)[2][2]) {
        const float a0 = al[0][mi], a1 = al[1][mi];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                pf[g][u] = __builtin_bit_cast(v8bf, lds_read16(p_rd + (2 * g + u) * (kWave * 16)));
        if (__ballot(a0 != 1.f || a1 != 1.f) != 0ull) {
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // MFMA results settle
#pragma unroll
            for (int t = 0; t < C::VTW; ++t) {
                scale_agpr(oacc[0][t], a0);
                scale_agpr(oacc[1][t], a1);
            }
            asm volatile("s_nop 4" ::: "memory");  // before the next MFMA reads them
        }
    };
    if (!active) {  // only the barriers
        if (nblk > 0)
            for (int b = 0; b < 2 * nblk + 3; ++b) lds_barrier();
        lds_barrier();
        return;
    }
    // Value waves 3, 6, 7 (quarters 1..3) issue the last VLOAD direct loads of each block,
    // I = HLOAD + vq - 1 + 3k: those of block b+3 after the second value half of step b (the
    // buffer block b-1 used; a value wave would otherwise wait at the end barrier there), and
    // they wait for block b+2's before the mid-step barrier of step b, where waves 4, 5 wait
    // for theirs.  Fewer loads then sit in the helpers' phase before that barrier.  These are
    // the only global loads of these waves, so their load counter holds only these.
    const bool loader = C::VLOAD > 0 && vq > 0;
    const int vfirst = C::HLOAD + vq - 1;
    auto vland = [&](int blk) {
        const uint32_t vm = rmask[blk % C::RING];
        if (vm != 0xffffffffu) zero_pieces<C, C::VMAXK, C::NVL>(buf_of(blk), vm, vfirst, C::INSTRS, lane);
    };
    auto vissue = [&](int blk) {
        issue_pieces<C, PAGED, C::VMAXK, C::NVL, (C::VLOAD > 0)>(buf_of(blk), kvb, rofs[blk % C::RING], vfirst, C::INSTRS, lane);
    };
    constexpr int VPER = C::VMAXK;
    if (nblk > 0) {
        if (loader) {
            vissue(0);
            if (nblk > 1) vissue(1);
            if (nblk > 2) vissue(2);
            wait_blocks_left<VPER>(min(nblk, 3) - 1);
            vland(0);
        }
        lds_barrier();  // block 0 visible
        if (loader && nblk > 1) {
            wait_blocks_left<VPER>(min(nblk, 3) - 2);
            vland(1);
        }
        lds_barrier();  // mid-step of the prologue: block 1 visible
        lds_barrier();  // end of the prologue: block 0's P^T visible
        // Value wave 2 stages the row offsets of block b + RING at the end of step b (after its
        // MFMAs; the value waves wait at the end barrier anyway; on a logit wave the staging sat
        // on the step's critical path).  It fetches each block's index slots IDS_AHEAD steps
        // before staging it, with direct loads into rid, so the wait for them rarely waits;
        // it issues no other global loads, so its load counter holds only these fetches.
        const bool stager = vq == 0;
        constexpr int IDS_AHEAD = 3;
        static_assert(IDS_AHEAD < C::RING, "the fetch slot of block b + IDS_AHEAD is free");
        auto fetch_ids = [&](int b) {  // lanes < kBlk: block b's slots -> rid[b % RING]
            const int j = j0 + b * kBlk + lane;
            if (lane < kBlk && j < j1) dma4(irow, (uint32_t)j * 4u, lds_addr(&rid[b % C::RING][0]));
        };
        if (stager && !dense)
            for (int b = C::RING; b < nblk && b < C::RING + IDS_AHEAD; ++b) fetch_ids(b);
        for (int blk = 0; blk < nblk; ++blk) {
            v8bf pf[2][2];
            take_p(pf);
            values(blk, 0, pf);
            if (loader && blk + 2 < nblk) {  // only block blk+2's loads are in flight
                wait_loads<0>();
                vland(blk + 2);
            }
            lds_barrier();  // mid-step: block blk+2 visible
            values(blk, 1, pf);
            if (loader && blk + 3 < nblk) vissue(blk + 3);
            if (stager && blk + C::RING < nblk) {
                const int b = blk + C::RING;
                const int j = j0 + b * kBlk + lane;
                int id = -1;
                if (dense) {
                    if (lane < kBlk && j < j1) id = j;
                } else {
                    // block b's fetch has landed once only the younger fetches may still fly
                    const int younger = min(nblk - 1, b + IDS_AHEAD - 1) - b;
                    if (younger >= 2) wait_loads<2>();
                    else if (younger == 1) wait_loads<1>();
                    else wait_loads<0>();
                    if (lane < kBlk && j < j1) id = rid[b % C::RING][lane];
                }
                stage(b, id);
                if (!dense && b + IDS_AHEAD < nblk) fetch_ids(b + IDS_AHEAD);
            }
            lds_barrier();  // end of step blk
        }
    }
    lds_barrier();  // softmax denominators visible

    // ---- epilogue ----
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int head = hh * 64 + g * 32 + mi;
        if (head >= H) continue;
        if (!SPLIT) {
            const float l_tot = fin_l[g][mi];
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            uint16_t* op = out + ((int64_t)ri.qrow * H + head) * DV;
#pragma unroll
            for (int t = 0; t < C::VTW; ++t)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int v = 32 * (vq * C::VTW + t) + 8 * rb + 4 * half;
                    const uint32_t w0 = (uint32_t)f2bf(oacc[g][t][4 * rb + 0] * inv) |
                                        ((uint32_t)f2bf(oacc[g][t][4 * rb + 1] * inv) << 16);
                    const uint32_t w1 = (uint32_t)f2bf(oacc[g][t][4 * rb + 2] * inv) |
                                        ((uint32_t)f2bf(oacc[g][t][4 * rb + 3] * inv) << 16);
                    *(v2i*)(op + v) = (v2i){(int)w0, (int)w1};
                }
        } else {
            const int64_t item = (int64_t)row * n_split + split;
            float* op = part_o + (item * H + head) * DV;
#pragma unroll
            for (int t = 0; t < C::VTW; ++t)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int v = 32 * (vq * C::VTW + t) + 8 * rb + 4 * half;
                    *(v4f*)(op + v) = (v4f){oacc[g][t][4 * rb + 0], oacc[g][t][4 * rb + 1],
                                            oacc[g][t][4 * rb + 2], oacc[g][t][4 * rb + 3]};
                }
        }
    }
}

// Merges the split partials of each (row, head): weights 2^(m_j - M) on the unnormalised
// partial outputs and sums, splits in ascending order.  Every split's (m, l) and partial
// output of the head are loaded before any is used, so the merge waits for one round of
// loads rather than one per split.  Lane l holds dims 4l..4l+3 of each 256-dim slice.
constexpr int kMaxSplit = 8;
template <int H, int DV>
__global__ __launch_bounds__(256) void mqa_combine_kernel(const float* __restrict__ part_o,
                                                          const float2* __restrict__ part_ml,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse, RowMap map,
                                                          int n_rows, int n_split) {
    static_assert(DV % 256 == 0 || DV == 64, "value width");
    constexpr int NV = DV >= 256 ? DV / 256 : 1;  // 4-float pieces per lane and split
    const int row = blockIdx.x;
    const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (row >= n_rows || head >= H) return;
    const int lane = threadIdx.x & 63;
    const bool live = DV >= 256 || lane < DV / 4;
    const RowInfo ri = row_info(map, row);
    float2 ml[kMaxSplit];
    v4f po[kMaxSplit][NV];
#pragma unroll
    for (int j = 0; j < kMaxSplit; ++j) {
        ml[j] = make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int i = 0; i < NV; ++i) po[j][i] = (v4f){0.f, 0.f, 0.f, 0.f};
        if (j < n_split) {
            const int64_t item = (int64_t)row * n_split + j;
            ml[j] = part_ml[item * H + head];
            const float* op = part_o + (item * H + head) * DV;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (live) po[j][i] = *(const v4f*)(op + 256 * i + 4 * lane);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxSplit; ++j) M = fmaxf(M, ml[j].x);
    float L = 0.f;
    v4f acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int j = 0; j < kMaxSplit; ++j) {
            if (ml[j].x == -INFINITY) continue;  // also the splits past n_split
            const float wgt = exp2f(ml[j].x - M);
            L += ml[j].y * wgt;
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[i][c] += wgt * po[j][i][c];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* o = out + ((int64_t)ri.qrow * H + head) * DV;
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (live) {
            const uint32_t w0 = (uint32_t)f2bf(acc[i][0] * inv) | ((uint32_t)f2bf(acc[i][1] * inv) << 16);
            const uint32_t w1 = (uint32_t)f2bf(acc[i][2] * inv) | ((uint32_t)f2bf(acc[i][3] * inv) << 16);
            *(v2i*)(o + 256 * i + 4 * lane) = (v2i){(int)w0, (int)w1};
        }
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
    const bool paged = map.pages != nullptr;
    if (n_split <= 1) {
        auto kern = paged ? sparse_mqa_kernel<H, DQK, DV, false, true> : sparse_mqa_kernel<H, DQK, DV, false, false>;
        hipLaunchKernelGGL(kern, dim3(grid_x<C>(n_rows)), dim3(C::THREADS), 0, st, a.q, a.kv, a.idx, a.topk, a.out,
                           a.lse, nullptr, nullptr, map, n_rows, 1, sm_log2, (int)a.mode);
        return hipGetLastError();
    }
    if (n_split > kMaxSplit) return hipErrorInvalidValue;  // the combine holds kMaxSplit splits
    float* part_o = (float*)ws;
    float2* part_ml = (float2*)(part_o + (size_t)n_rows * n_split * H * DV);
    auto kern = paged ? sparse_mqa_kernel<H, DQK, DV, true, true> : sparse_mqa_kernel<H, DQK, DV, true, false>;
    hipLaunchKernelGGL(kern, dim3(grid_x<C>(n_rows), n_split), dim3(C::THREADS), 0, st, a.q, a.kv, a.idx, a.topk,
                       a.out, a.lse, part_o, part_ml, map, n_rows, n_split, sm_log2, (int)a.mode);
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
