// Decode cache producer on gfx950: the indexer's rotary encoding and FP8 quantisation of the
// new tokens (DeepSeek-V3.2-Exp lightning-indexer walk-through, step 2: RoPE on the first 64
// dims of the indexer query and key, then FP8 codes for both, the key codes and their scale
// kept in the cache), plus the copy of the tokens' latent rows into the latent cache.
//
// Each new token has 65 rows of idx_dim values (its 64 query heads and its key) and one latent
// row.  One wave per row: lane l holds the pair (2l, 2l+1), which is exactly the pair the
// rotation mixes, so the rotation is in-lane and the row's amax one wave reduction; a 256-thread
// workgroup takes four rows of one token, the last one of each token also copies the latent
// row.  Bound: HBM (32 KiB of fp32 query per token in, 8 KiB of codes out), i.e. latency at
// decode sizes, hence one row per wave.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendRowsPerWg = kAppendThreads / kWave;

// One row of D values (D/2 <= 64 pairs, one per lane): rotate the first R/2 pairs by the
// table angle of position pos, then one scale (amax / 448, 1 for an all-zero row) and e4m3fn
// codes of x / scale clamped to +-448.  Every product, sum and quotient is a separately
// rounded float32 operation, so the rounding decisions are reproducible: contraction into
// FMAs is switched off for this function's expressions, and float32 division is correctly
// rounded (HIP's default).
template <int D>
__device__ __forceinline__ void rope_quant_row(const float* __restrict__ src, const float* __restrict__ cs,
                                               const float* __restrict__ sn, int lane, uint8_t* __restrict__ dst,
                                               float* __restrict__ scale_out) {
#pragma clang fp contract(off)
    constexpr int P = D / 2;  // pairs
    constexpr int RP = D / 4;  // rotated pairs (R = D / 2 dims)
    float x0 = 0.f, x1 = 0.f;
    if (lane < P) {
        const float2 v = *(const float2*)(src + 2 * lane);
        x0 = v.x;
        x1 = v.y;
        if (lane < RP) {
            const float c = cs[lane], s = sn[lane];
            const float r0 = x0 * c - x1 * s;
            const float r1 = x0 * s + x1 * c;
            x0 = r0;
            x1 = r1;
        }
    }
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    const float y0 = fminf(fmaxf(x0 / scale, -448.f), 448.f);
    const float y1 = fminf(fmaxf(x1 / scale, -448.f), 448.f);
    // round to nearest even to OCP e4m3fn (the format of gfx950's FP8 conversion)
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    if (lane < P) *(uint16_t*)(dst + 2 * lane) = (uint16_t)(packed & 0xffff);
    if (lane == 0) *scale_out = scale;
}

template <int H, int D, int DQK>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(
    const float* __restrict__ q_idx, const float* __restrict__ k_idx, const uint16_t* __restrict__ kv_new,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, uint8_t* __restrict__ q8,
    float* __restrict__ q_scale, uint8_t* __restrict__ k8_cache, float* __restrict__ k_scale_cache,
    uint16_t* __restrict__ kv_cache, RowMap map, int n_rows) {
    static_assert(D % 4 == 0 && D / 2 <= kWave, "one pair per lane");
    constexpr int NG = (H + 1 + kAppendRowsPerWg - 1) / kAppendRowsPerWg;  // workgroups per token
    const int row = blockIdx.x / NG, part = blockIdx.x % NG;
    if (row >= n_rows) return;
    const RowInfo ri = row_info(map, row);
    const int64_t crow = cache_row(map, ri, ri.pos);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const float* cs = rope_cos + (int64_t)ri.pos * (D / 4);
    const float* sn = rope_sin + (int64_t)ri.pos * (D / 4);
    // rows 0 .. H-1: query heads; row H: the key
    const int v = part * kAppendRowsPerWg + wv;
    if (v < H)
        rope_quant_row<D>(q_idx + ((int64_t)row * H + v) * D, cs, sn, lane, q8 + ((int64_t)row * H + v) * D,
                          q_scale + (int64_t)row * H + v);
    else if (v == H)
        rope_quant_row<D>(k_idx + (int64_t)row * D, cs, sn, lane, k8_cache + crow * D, k_scale_cache + crow);
    if (kv_new != nullptr && part == NG - 1) {  // the latent row, 16 bytes per thread
        constexpr int NP = DQK * 2 / 16;
        const uint4* s = (const uint4*)(kv_new + (int64_t)row * DQK);
        uint4* d = (uint4*)(kv_cache + crow * DQK);
        for (int i = tid; i < NP; i += kAppendThreads) d[i] = s[i];
    }
}

template <int H>
constexpr int append_groups() { return (H + 1 + kAppendRowsPerWg - 1) / kAppendRowsPerWg; }

}  // namespace

hipError_t launch_cache_append(const CacheAppendArgs& a, const RowMap& map, int n_rows, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    if (a.shape == Shape::Prod)
        hipLaunchKernelGGL((cache_append_kernel<64, 128, 576>), dim3(n_rows * append_groups<64>()), dim3(kAppendThreads), 0, st, a.q_idx,
                           a.k_idx, a.kv_new, a.rope_cos, a.rope_sin, a.q8, a.q_scale, a.k8_cache, a.k_scale_cache,
                           a.kv_cache, map, n_rows);
    else
        hipLaunchKernelGGL((cache_append_kernel<4, 32, 80>), dim3(n_rows * append_groups<4>()), dim3(kAppendThreads), 0, st, a.q_idx,
                           a.k_idx, a.kv_new, a.rope_cos, a.rope_sin, a.q8, a.q_scale, a.k8_cache, a.k_scale_cache,
                           a.kv_cache, map, n_rows);
    return hipGetLastError();
}

}  // namespace dsa
