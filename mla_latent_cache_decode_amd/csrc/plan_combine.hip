// Split-KV combine for the MLA decode.
//
// The log-sum-exp merge of a sequence's partial results,
//     lse = log sum_i exp(lse_i),   out = sum_i exp(lse_i - lse) * out_i,
// which is exact because each partial out_i is already normalised by its own
// softmax denominator (the partials are stored as fp16, the sums are fp32).  The decode kernel records, per sequence, how many
// splits it produced and where its partial slots start; a sequence served
// by a single worker was finished by the decode kernel and is skipped here.
#include "mla_internal.h"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineRows = 2;          // query rows per block, 128 threads x 4 dims each
constexpr int kUnroll = 8;               // partial loads in flight per thread

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    __shared__ float s_w[kCombineRows][kMaxSplits];
    __shared__ float s_red[kCombineRows][2];
    const int M = a.rows;
    const int row_blocks = (M + kCombineRows - 1) / kCombineRows;
    const int b = blockIdx.x / row_blocks;
    const int r = threadIdx.x >> 7;                       // row within the block
    const int row = (blockIdx.x % row_blocks) * kCombineRows + r;
    const int t = threadIdx.x & 127;
    if (b >= a.batch) return;
    const int n = a.plan.seq_nsplit[b];
    if (n == 1) return;                                   // finished by the decode kernel
    const bool live = row < M;
    const float ninf = -__builtin_inff();
    f32x4* o = (f32x4*)(a.out + ((int64_t)b * M + (live ? row : 0)) * kDc) + t;
    if (n <= 0) {                                         // empty sequence
        if (live) {
            *o = f32x4{0.f, 0.f, 0.f, 0.f};
            if (a.lse && t == 0) a.lse[(int64_t)b * M + row] = ninf;
        }
        return;
    }
    const int base = a.plan.seq_slot[b];
    // stage the split LSEs of this row and their max (128 threads per row)
    float mx = ninf;
    for (int i = t; i < n; i += 128) {
        const float v = live ? a.plan.part_lse[(int64_t)(base + i) * M + row] : ninf;
        s_w[r][i] = v;
        mx = fmaxf(mx, v);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((t & 63) == 0) s_red[r][t >> 6] = mx;
    __syncthreads();
    mx = fmaxf(s_red[r][0], s_red[r][1]);
    const bool dead = mx == ninf;                         // no visible token in any split
    float sum = 0.f;
    if (!dead) {
        for (int i = t; i < n; i += 128) {
            const float e = expf(s_w[r][i] - mx);
            s_w[r][i] = e;
            sum += e;
        }
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    __syncthreads();                                      // s_red reuse; s_w complete
    if ((t & 63) == 0) s_red[r][t >> 6] = sum;
    __syncthreads();
    // no barrier below: rows may leave independently
    if (!live) return;
    if (dead) {
        *o = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.lse && t == 0) a.lse[(int64_t)b * M + row] = ninf;
        return;
    }
    sum = s_red[r][0] + s_red[r][1];
    const float inv = 1.0f / sum;
    // partials are fp16 (see the decode epilogue), four dims per thread
    const uint16_t* src = a.plan.part_o + ((int64_t)base * M + row) * kDc + t * 4;
    const int64_t stride = (int64_t)M * kDc;
    auto load4 = [&](int i) -> f32x4 {
        const f16x4 h = *(const f16x4*)(src + i * stride);
        return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int i = 0;
    for (; i + kUnroll <= n; i += kUnroll) {
        f32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load4(i + u);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += s_w[r][i + u] * v[u];
    }
    for (; i < n; ++i) acc += s_w[r][i] * load4(i);
    *o = acc * inv;
    if (a.lse && t == 0) a.lse[(int64_t)b * M + row] = mx + logf(sum);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    const int row_blocks = (a.rows + kCombineRows - 1) / kCombineRows;
    const int64_t blocks = (int64_t)a.batch * row_blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
