// Index-row checker.  The selected positions are the gather addresses of the sparse attention
// (DeepSeek-V3.2-Exp lightning-indexer walk-through, step 4: the top-k indices feed the core
// attention), so index rows from outside the library are checked here on request.  The gathers
// themselves never load an entry that is out of range (they treat it as an empty slot); this
// kernel reports such entries, and the other ways a row can differ from what the top-k writes.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kCheckThreads = 256;

// One workgroup per query row: reads the row's topk slots once (and, for paged caches of known
// pool size, the page-table entry of each valid slot) and writes the OR of the flags it finds.
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(
    const int32_t* __restrict__ idx, int topk, RowMap map, int n_rows, uint32_t* __restrict__ row_flags,
    uint32_t* __restrict__ any_flags) {
    __shared__ uint32_t acc;
    const int row = blockIdx.x;
    if (row >= n_rows) return;
    if (threadIdx.x == 0) acc = 0u;
    __syncthreads();
    const RowInfo ri = row_info(map, row);
    const int32_t* irow = idx + (int64_t)row * topk;
    uint32_t f = 0u;
    for (int j = threadIdx.x; j < topk; j += kCheckThreads) {
        const int id = irow[j];
        if (id != -1) {
            if (id < -1 || id > ri.lim) {
                f |= kIdxOutOfRange;
            } else {
                if (id > ri.pos) f |= kIdxNotCausal;
                if (slot_row(map, ri, id) < 0) f |= kIdxBadPage;
            }
        }
        // the top-k's form: valid entries strictly ascending, then the -1 pads
        if (j + 1 < topk) {
            const int nx = irow[j + 1];
            if ((id == -1 && nx != -1) || (id >= 0 && nx >= 0 && nx <= id)) f |= kIdxNotSorted;
        }
    }
    if (f != 0u) atomicOr(&acc, f);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (row_flags != nullptr) row_flags[row] = acc;
        if (any_flags != nullptr && acc != 0u) atomicOr(any_flags, acc);
    }
}

}  // namespace

hipError_t launch_check_indices(const int32_t* idx, int topk, const RowMap& map, int n_rows, uint32_t* row_flags,
                                uint32_t* any_flags, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(check_indices_kernel, dim3(n_rows), dim3(kCheckThreads), 0, st, idx, topk, map, n_rows,
                       row_flags, any_flags);
    return hipGetLastError();
}

}  // namespace dsa
