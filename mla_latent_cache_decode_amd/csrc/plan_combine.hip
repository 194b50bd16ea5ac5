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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Two shapes of the same merge, chosen by the expected split count:
//  * many splits per sequence (few, long sequences): one row per block,
//    the row's splits dealt to WPR waves in contiguous ranges, partial sums
//    reduced through LDS;
//  * few splits per sequence: a wave merges 4 rows at once, splits in
//    chunks of 64 merged online.
// Either way a lane owns 8 dims (one 16-byte fp16 load per split and row)
// and many split loads are in flight together, so the merge is bound by HBM
// rate rather than by load latency.
constexpr int kMergeRows = 4;
constexpr int kLoadBatch = 16;      // split loads in flight per wave, one row
constexpr int kRowBatch = 2;        // splits per row per batch, 4 rows

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ void acc_add(f32x4 (&acc)[2], float w, const f16x8& h) {
    acc[0] += w * f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    acc[1] += w * f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
}
__device__ __forceinline__ void store_row(const CombineArgs& a, int b, int row, int t, const f32x4 (&acc)[2],
                                          float mx, float sum) {
    float* o = a.out + ((int64_t)b * a.rows + row) * kDc + t * 8;
    const bool dead = !(sum > 0.f);                       // no visible token (or no split)
    const float inv = dead ? 0.f : 1.0f / sum;
    *(f32x4*)o = acc[0] * inv;
    *(f32x4*)(o + 4) = acc[1] * inv;
    if (a.lse && t == 0) a.lse[(int64_t)b * a.rows + row] = dead ? -__builtin_inff() : mx + logf(sum);
}

template <int WPR>
__global__ __launch_bounds__(WPR * 64) void combine_split_parallel(CombineArgs a) {
    // LDS: partial sums of waves 1.. [WPR - 1][2][64], reductions [2][WPR],
    // then the split weights [splits]
    extern __shared__ f32x4 s_acc[];
    float* const s_red = (float*)(s_acc + (WPR - 1) * 2 * 64);
    float* const s_w = s_red + 2 * WPR;
    const int M = a.rows;
    const int b = blockIdx.x / M, row = blockIdx.x % M;
    const int tid = threadIdx.x, wave = tid >> 6, t = tid & 63;
    const int n = a.plan.seq_nsplit[b];
    if (n == 1) return;                                   // finished by the decode kernel
    const int base = a.plan.seq_slot[b];
    float mx = -__builtin_inff();
    for (int i = tid; i < n; i += WPR * 64) {
        const float v = a.plan.part_lse[(int64_t)(base + i) * M + row];
        s_w[i] = v;
        mx = fmaxf(mx, v);
    }
    mx = wave_max(mx);
    if (t == 0) s_red[wave] = mx;
    __syncthreads();
    mx = s_red[0];
#pragma unroll
    for (int q = 1; q < WPR; ++q) mx = fmaxf(mx, s_red[q]);
    float sum = 0.f;
    for (int i = tid; i < n; i += WPR * 64) {
        const float e = mx == -__builtin_inff() ? 0.f : expf(s_w[i] - mx);
        s_w[i] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    if (t == 0) s_red[WPR + wave] = sum;
    __syncthreads();                                      // weights and sums visible
    sum = 0.f;
#pragma unroll
    for (int q = 0; q < WPR; ++q) sum += s_red[WPR + q];
    const int per = (max(n, 0) + WPR - 1) / WPR;
    const int lo = min(wave * per, max(n, 0)), hi = min(lo + per, max(n, 0));
    const int64_t stride = (int64_t)M * kDc;
    const uint16_t* src = a.plan.part_o + ((int64_t)base * M + row) * kDc + t * 8;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 1
    for (int i = lo; i < hi; i += kLoadBatch) {
        f16x8 v[kLoadBatch];
        // bounds are wave-uniform: the tail batch issues only its loads
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u)
            if (i + u < hi) v[u] = *(const f16x8*)(src + (i + u) * stride);
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u)
            if (i + u < hi) acc_add(acc, s_w[i + u], v[u]);
    }
    if (wave > 0) {
        s_acc[((wave - 1) * 2 + 0) * 64 + t] = acc[0];
        s_acc[((wave - 1) * 2 + 1) * 64 + t] = acc[1];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < WPR - 1; ++q) {
            acc[0] += s_acc[(q * 2 + 0) * 64 + t];
            acc[1] += s_acc[(q * 2 + 1) * 64 + t];
        }
        store_row(a, b, row, t, acc, mx, sum);
    }
}

__global__ __launch_bounds__(256) void combine_row_parallel(CombineArgs a) {
    const int M = a.rows;
    const int rblocks = (M + 4 * kMergeRows - 1) / (4 * kMergeRows);
    const int b = blockIdx.x / rblocks;
    const int wave = threadIdx.x >> 6, t = threadIdx.x & 63;
    const int row0 = (blockIdx.x % rblocks) * 4 * kMergeRows + wave * kMergeRows;
    if (row0 >= M) return;
    const int n = a.plan.seq_nsplit[b];
    if (n == 1) return;                                   // finished by the decode kernel
    const int nr = min(kMergeRows, M - row0);           // rows of this wave
    const int base = a.plan.seq_slot[b];
    const int64_t stride = (int64_t)M * kDc;              // between split slots
    const uint16_t* const src0 = a.plan.part_o + ((int64_t)base * M + row0) * kDc + t * 8;
    const float ninf = -__builtin_inff();
    float mx[kMergeRows], sum[kMergeRows];
    f32x4 acc[kMergeRows][2];
#pragma unroll
    for (int j = 0; j < kMergeRows; ++j) {
        mx[j] = ninf;
        sum[j] = 0.f;
        acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 1
    for (int c = 0; c < n; c += 64) {
        const int cn = min(64, n - c);
        // this chunk's LSEs (lane = split), then weights against the new max
        float w[kMergeRows];
#pragma unroll
        for (int j = 0; j < kMergeRows; ++j)
            w[j] = (t < cn && j < nr) ? a.plan.part_lse[(int64_t)(base + c + t) * M + row0 + j] : ninf;
#pragma unroll
        for (int j = 0; j < kMergeRows; ++j) {
            const float m_new = fmaxf(mx[j], wave_max(w[j]));
            // rows with nothing visible so far keep weight 0
            const float scale = m_new == ninf ? 0.f : expf(mx[j] - m_new);
            w[j] = m_new == ninf ? 0.f : expf(w[j] - m_new);
            sum[j] = sum[j] * scale + wave_sum(w[j]);
            acc[j][0] *= scale;
            acc[j][1] *= scale;
            mx[j] = m_new;
        }
#pragma unroll 1
        for (int i = 0; i < cn; i += kRowBatch) {
            constexpr int kU = kRowBatch;
            f16x8 v[kMergeRows][kU];
            // bounds are wave-uniform: the tail batch issues only its loads
#pragma unroll
            for (int u = 0; u < kU; ++u)
#pragma unroll
                for (int j = 0; j < kMergeRows; ++j)
                    if (i + u < cn && j < nr) v[j][u] = *(const f16x8*)(src0 + (c + i + u) * stride + j * kDc);
#pragma unroll
            for (int u = 0; u < kU; ++u)
#pragma unroll
                for (int j = 0; j < kMergeRows; ++j)
                    if (i + u < cn && j < nr) {
                        // the weight of split c + i + u sits in lane i + u
                        const float wu =
                            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w[j]), i + u));
                        acc_add(acc[j], wu, v[j][u]);
                    }
        }
    }
#pragma unroll
    for (int j = 0; j < kMergeRows; ++j)
        if (j < nr) store_row(a, b, row0 + j, t, acc[j], mx[j], sum[j]);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int max_splits, hipStream_t stream) {
    if ((int64_t)a.batch * a.rows == 0) return hipSuccess;
    // expected splits per sequence: the workers spread over the batch
    const int per_seq = max_splits / max(a.batch, 1);
    if (per_seq >= 32) {
        const size_t lds = (size_t)(max_splits + 2 * 8) * sizeof(float) + 7 * 2 * 64 * 16;
        hipLaunchKernelGGL(combine_split_parallel<8>, dim3((unsigned)(a.batch * a.rows)), dim3(512), lds, stream, a);
    } else {
        const int rblocks = (a.rows + 4 * kMergeRows - 1) / (4 * kMergeRows);
        hipLaunchKernelGGL(combine_row_parallel, dim3((unsigned)(a.batch * rblocks)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace mla
