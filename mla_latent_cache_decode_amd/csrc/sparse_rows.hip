// Pre-pass of the sparse (top-k) MLA decode.
//
// "DeepSeek-V3.2" record: the latent cache is unchanged, and a top-k
// selector (index_topk = 2048) picks, for every query token, the tokens it
// attends over.  The decode gathers those rows tile by tile; this pass turns
// each (sequence, query position) unit's index list into what the gather
// needs: the physical row id of every entry (page * page_size + slot,
// through the block table) and, per 64-entry tile, a mask of the entries
// that take part.  An entry takes part when 0 <= t < L - s_q + 1 + j (the
// query's causal context); padding (-1) and anything else does not.  One
// wave per tile; 4 bytes read and 4 written per entry.
#include "mla_internal.h"

namespace mla {
namespace {

__global__ __launch_bounds__(64) void sparse_rows_kernel(SparseRowsArgs a) {
    const int lane = threadIdx.x;
    const int u = blockIdx.x / a.tiles, p = blockIdx.x % a.tiles;
    const int b = u / a.s_q, j = u % a.s_q;
    const int n_vis = a.seq_lens[b] - a.s_q + 1 + j;
    const int k = p * 64 + lane;
    const int t = k < a.topk ? a.indices[(int64_t)u * a.topk + k] : -1;
    const bool valid = t >= 0 && t < n_vis;
    uint32_t row = kNoRow;
    if (valid) {
        const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.page_size];
        row = (uint32_t)((uint64_t)page * (uint32_t)a.page_size + (uint32_t)(t % a.page_size));
    }
    const uint64_t mask = __builtin_amdgcn_ballot_w64(valid);
    // token lane = 16 w + 8 g + x goes to pair w * 8 + x, element g
    const int w = lane >> 4, g = (lane >> 3) & 1, x = lane & 7;
    uint32_t* const dst = a.rows + ((int64_t)u * a.tiles + p) * 64;
    dst[(w * 8 + x) * 2 + g] = row;
    if (lane == 0) a.masks[(int64_t)u * a.tiles + p] = mask;
    // the row the decode fetches for entries that do not take part (their
    // weights are 0, and 0 x 0 keeps the product finite whatever the data;
    // as an fp8 row its codes and scales are 0 too, so it decodes to zeros)
    if (blockIdx.x == 0) {
        for (int i = lane; i < kSparseZeroRowBytes / 16; i += 64)
            *(uint4*)(a.zero_row + i * 16) = make_uint4(0, 0, 0, 0);
    }
}

}  // namespace

hipError_t launch_sparse_rows(const SparseRowsArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.units * a.tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sparse_rows_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
