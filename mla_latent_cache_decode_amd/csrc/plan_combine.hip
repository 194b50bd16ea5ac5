// Split-KV combine for the MLA decode.
//
// The log-sum-exp merge of a sequence's partial results,
//     lse = log sum_i exp(lse_i),   out = sum_i exp(lse_i - lse) * out_i,
// which is exact because each partial out_i is already normalised by its own
// softmax denominator (the partials are stored as fp16, the sums are fp32).
// The decode kernel records, per sequence, how many splits it produced and
// where its partial slots start; a sequence served by a single worker was
// finished by the decode kernel and is skipped here.
#include "mla_internal.h"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One kernel shape, two instantiations chosen by the expected split count.
// A block merges RPB rows; each row's splits are dealt to WPR waves in
// contiguous ranges (WPR = 4, RPB = 1 for few long sequences with many
// splits; WPR = 1, RPB = 4 when sequences have few splits).  A lane owns 8
// dims of the row: one 16-byte fp16 load per split (rows of d_c <= 512 dims;
// lanes past d_c / 8 idle).
//
// Latency is the cost to beat: the whole merge is one round of loads.  Each
// wave issues the row's split LSEs and its first kLoadBatch partial rows
// together, and forms the max and the sum while the partial rows are still
// in flight.  Loads go through buffer descriptors that end at the wave's
// last split, so a batch never branches around its loads (branches would
// make the compiler wait for every load at the join) and the lanes of a
// short batch read zeros without touching memory.

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Buffer descriptor over [base, base + bytes); both wave-uniform.  Loads at
// or past `bytes` return zeros and read nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, int i) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
}
__device__ __forceinline__ f16x8 load_row8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void acc_add(f32x4 (&acc)[2], float w, const f16x8& h) {
    acc[0] += w * f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    acc[1] += w * f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
}

__device__ __forceinline__ void store_row(const CombineArgs& a, int b, int row, int t, const f32x4 (&acc)[2],
                                          float mx, float sum) {
    float* o = a.out + ((int64_t)b * a.rows + row) * a.d_c + t * 8;
    const bool dead = !(sum > 0.f);                       // no visible token (or no split)
    const float inv = dead ? 0.f : 1.0f / sum;
    if (t * 8 < a.d_c) {
        *(f32x4*)o = acc[0] * inv;
        *(f32x4*)(o + 4) = acc[1] * inv;
    }
    if (a.lse && t == 0) a.lse[(int64_t)b * a.rows + row] = dead ? -__builtin_inff() : mx + logf(sum);
}

// LB: partial rows in flight per wave (16 when a row's splits are many; 8
// when they are few, which halves the registers and doubles the waves in
// flight)
template <int WPR, int RPB, int LB>
__global__ __launch_bounds__(WPR * RPB * 64) void combine_kernel(CombineArgs a) {
    constexpr int kLoadBatch = LB;
    // partial sums of waves 1 .. WPR - 1 of each row, reduced by its wave 0
    __shared__ f32x4 s_acc[WPR > 1 ? RPB * (WPR - 1) * 2 * 64 : 1];
    const int M = a.rows;                                 // a multiple of 32, so of RPB
    const int tid = threadIdx.x, wave = tid >> 6, t = tid & 63;
    const int rw = wave / WPR, part = wave % WPR;
    const int rblocks = M / RPB;
    const int b = blockIdx.x / rblocks;
    const int row = (blockIdx.x % rblocks) * RPB + rw;
    const int n = max(a.plan.seq_nsplit[b], 0);
    if (n == 1) return;                                   // finished by the decode kernel
    const float ninf = -__builtin_inff();
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (n == 0) {                                         // an empty sequence: nothing visible
        if (part == 0) store_row(a, b, row, t, acc, ninf, 0.f);
        return;
    }
    const int base = a.plan.seq_slot[b];
    const int per = (n + WPR - 1) / WPR;
    const int lo = min(part * per, n), hi = min(lo + per, n);
    const uint32_t stride = (uint32_t)M * a.d_c * 2;      // bytes between split slots of a row
    // a lane past the row's d_c / 8 loads from past the descriptor's range:
    // zeros, no memory touched (its sums are not stored)
    const uint32_t t_off = t * 8 < a.d_c ? (uint32_t)t * 16 : 0x80000000u;
    const float* const lse_row = a.plan.part_lse + (int64_t)row * a.plan.slots + base;
    const __amdgpu_buffer_rsrc_t r_lse = make_rsrc(lse_row, (uint32_t)n * 4);
    const __amdgpu_buffer_rsrc_t r_own = make_rsrc(lse_row + lo, (uint32_t)(hi - lo) * 4);
    // partial rows of this wave's splits j .. j + kLoadBatch - 1 (one
    // descriptor per batch keeps every offset far inside 32 bits)
    auto batch_rsrc = [&](int j) {
        return make_rsrc(a.plan.part_o + ((int64_t)(base + lo + j) * M + row) * a.d_c,
                         (uint32_t)max(min(kLoadBatch, hi - lo - j), 0) * stride);
    };

    // the round of loads: LSEs first, then the partial rows
    float l_a = load_f32(r_lse, t);
    float l_b = load_f32(r_lse, 64 + t);
    float l_own = load_f32(r_own, t);
    f16x8 v[kLoadBatch];
    {
        const __amdgpu_buffer_rsrc_t r_o = batch_rsrc(0);
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) v[u] = load_row8(r_o, u * stride + t_off);
    }
    l_a = t < n ? l_a : ninf;
    l_b = 64 + t < n ? l_b : ninf;
    l_own = t < hi - lo ? l_own : ninf;

    // max and sum over every split of the row (each wave forms them itself)
    float mx = fmaxf(l_a, l_b);
    for (int c = 128; c < n; c += 64) mx = fmaxf(mx, c + t < n ? load_f32(r_lse, c + t) : ninf);
    mx = wave_max(mx);
    const bool dead = mx == ninf;                         // no visible token in any split
    float sum = dead ? 0.f : expf(l_a - mx) + expf(l_b - mx);
    for (int c = 128; c < n && !dead; c += 64) sum += c + t < n ? expf(load_f32(r_lse, c + t) - mx) : 0.f;
    sum = wave_sum(sum);

    // this wave's splits, 64 weights at a time (lane u holds split c + u's)
#pragma unroll 1
    for (int c = 0; c < hi - lo; c += 64) {
        if (c > 0) {
            const float l = load_f32(r_own, c + t);
            l_own = c + t < hi - lo ? l : ninf;
        }
        const float w = dead ? 0.f : expf(l_own - mx);
        const int cn = min(64, hi - lo - c);
#pragma unroll 1
        for (int i = 0; i < cn; i += kLoadBatch) {
            if (c > 0 || i > 0) {                         // the first batch is already loaded
                const __amdgpu_buffer_rsrc_t r_o = batch_rsrc(c + i);
#pragma unroll
                for (int u = 0; u < kLoadBatch; ++u) v[u] = load_row8(r_o, u * stride + t_off);
            }
#pragma unroll
            for (int u = 0; u < kLoadBatch; ++u) {
                // past the wave's range the load gave zeros; its lane index
                // may still be a real split of the next chunk, so mask it
                const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i + u));
                acc_add(acc, i + u < cn ? wu : 0.f, v[u]);
            }
        }
    }
    if constexpr (WPR > 1) {
        if (part > 0) {
            s_acc[((rw * (WPR - 1) + part - 1) * 2 + 0) * 64 + t] = acc[0];
            s_acc[((rw * (WPR - 1) + part - 1) * 2 + 1) * 64 + t] = acc[1];
        }
        __syncthreads();
        if (part > 0) return;
#pragma unroll
        for (int q = 0; q < WPR - 1; ++q) {
            acc[0] += s_acc[((rw * (WPR - 1) + q) * 2 + 0) * 64 + t];
            acc[1] += s_acc[((rw * (WPR - 1) + q) * 2 + 1) * 64 + t];
        }
    }
    store_row(a, b, row, t, acc, mx, sum);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int max_splits, hipStream_t stream) {
    if ((int64_t)a.batch * a.rows == 0) return hipSuccess;
    if (a.rows % 32 != 0) return hipErrorInvalidValue;
    // expected splits per sequence: the workers spread over the batch
    const int per_seq = max_splits / max(a.batch, 1);
    if (per_seq >= 32) {
        // four waves of 16 loads each cover 64 splits in one round (eight
        // waves of 8: the same on the long-context step, 0.5 us slower on a
        // single 1024-token sequence)
        hipLaunchKernelGGL((combine_kernel<4, 1, 16>), dim3((unsigned)(a.batch * a.rows)), dim3(256), 0, stream, a);
    } else if (per_seq >= 6) {
        // lengths vary: the longest sequences have about twice the mean split count
        hipLaunchKernelGGL((combine_kernel<1, 4, 16>), dim3((unsigned)(a.batch * (a.rows / 4))), dim3(256), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((combine_kernel<1, 4, 8>), dim3((unsigned)(a.batch * (a.rows / 4))), dim3(256), 0, stream,
                           a);
    }
    return hipGetLastError();
}

}  // namespace mla
