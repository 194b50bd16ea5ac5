// Device-side work planner and split-KV combine for the MLA decode.
//
// Planner: sequence lengths stay on the device (no host round trip).  One
// workgroup lays the batch's pages end to end on a cost axis, each sequence
// charged `overhead` extra units for its query load and epilogue, and cuts
// that axis into num_workers equal quotas.  Every (worker, sequence) overlap
// with at least one page is a segment; a sequence covered by one segment is
// finished by the decode kernel itself, otherwise each of its segments owns a
// partial slot in the workspace.  Segments are stored in worker order, so a
// worker's segments are contiguous.
//
// Combine: the log-sum-exp merge of a sequence's partial results,
//     lse = log sum_i exp(lse_i),   out = sum_i exp(lse_i - lse) * out_i,
// which is exact because each partial out_i is already normalised by its
// own softmax denominator.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 1024;

// Inclusive-to-exclusive block scan of one int per thread; returns the
// exclusive prefix and writes the block total into *total.
__device__ int block_excl_scan(int v, int* sbuf, int* total) {
    const int tid = threadIdx.x;
    sbuf[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int add = tid >= off ? sbuf[tid - off] : 0;
        __syncthreads();
        sbuf[tid] += add;
        __syncthreads();
    }
    const int incl = sbuf[tid];
    *total = sbuf[kPlanThreads - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
    __shared__ int sbuf[kPlanThreads];
    __shared__ int s_red[kPlanThreads / 64];
    const int tid = threadIdx.x;
    const int B = a.batch;
    const int G = a.num_workers;
    const int c = a.overhead_units;

    // total cost T
    int local = 0;
    for (int b = tid; b < B; b += kPlanThreads) {
        const int L = a.seq_lens[b];
        const int pages = L > 0 ? (L + kPage - 1) / kPage : 0;
        local += pages > 0 ? pages + c : 0;
    }
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    if ((tid & 63) == 0) s_red[tid >> 6] = local;
    __syncthreads();
    int64_t T = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) T += s_red[i];
    const int64_t Q = max(max((T + G - 1) / G, (int64_t)a.min_quota), (int64_t)1);

    int carry_cost = 0, carry_seg = 0, carry_slot = 0;
    for (int base = 0; base < B; base += kPlanThreads) {
        const int b = base + tid;
        int pages = 0;
        if (b < B) {
            const int L = a.seq_lens[b];
            pages = L > 0 ? (L + kPage - 1) / kPage : 0;
        }
        const int cost = pages > 0 ? pages + c : 0;
        int tot;
        const int64_t C = block_excl_scan(cost, sbuf, &tot) + (int64_t)carry_cost;
        carry_cost += tot;
        const int64_t A = C + c;
        const int64_t E = A + pages;
        const int n = pages > 0 ? (int)((E - 1) / Q - A / Q + 1) : 0;
        const int seg0 = block_excl_scan(n, sbuf, &tot) + carry_seg;
        carry_seg += tot;
        const int slot0 = block_excl_scan(n > 1 ? n : 0, sbuf, &tot) + carry_slot;
        carry_slot += tot;
        if (b < B) {
            a.plan.seq_nsplit[b] = n;
            a.plan.seq_slot[b] = slot0;
            const int64_t w0 = A / Q;
            for (int k = 0; k < n; ++k) {
                const int64_t w = w0 + k;
                const int lo = (int)(max(w * Q, A) - A);
                const int hi = (int)(min((w + 1) * Q, E) - A);
                a.plan.segs[seg0 + k] = make_int4(b, lo, hi, n > 1 ? slot0 + k : -1);
                a.plan.seg_worker[seg0 + k] = (int)w;
            }
        }
    }
    const int S = carry_seg;
    if (tid == 0) {
        a.plan.header[0] = (int)Q;
        a.plan.header[1] = S;
    }
    __threadfence_block();
    __syncthreads();

    // worker_start[w] = first segment whose worker is >= w (segments are sorted by worker)
    for (int w = tid; w <= G; w += kPlanThreads) {
        int lo = 0, hi = S;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (a.plan.seg_worker[mid] < w) lo = mid + 1;
            else hi = mid;
        }
        a.plan.worker_start[w] = lo;
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One block = 2 query rows of one sequence; 128 threads x 4 dims per row.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int M = a.rows;
    const int row_blocks = (M + 1) / 2;
    const int b = blockIdx.x / row_blocks;
    const int row = (blockIdx.x % row_blocks) * 2 + (threadIdx.x >> 7);
    const int t = threadIdx.x & 127;
    if (b >= a.batch || row >= M) return;
    const int n = a.plan.seq_nsplit[b];
    if (n == 1) return;                                   // finished by the decode kernel
    f32x4* o = (f32x4*)(a.out + ((int64_t)b * M + row) * kDc) + t;
    const float ninf = -__builtin_inff();
    if (n == 0) {                                         // empty sequence
        *o = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.lse && t == 0) a.lse[(int64_t)b * M + row] = ninf;
        return;
    }
    const int base = a.plan.seq_slot[b];
    float mx = ninf;
    for (int i = 0; i < n; ++i) mx = fmaxf(mx, a.plan.part_lse[(int64_t)(base + i) * M + row]);
    if (mx == ninf) {                                     // no visible token in any split
        *o = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.lse && t == 0) a.lse[(int64_t)b * M + row] = ninf;
        return;
    }
    float wsum = 0.f;
    for (int i = 0; i < n; ++i) wsum += expf(a.plan.part_lse[(int64_t)(base + i) * M + row] - mx);
    const float lse_tot = mx + logf(wsum);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n; ++i) {
        const float w = expf(a.plan.part_lse[(int64_t)(base + i) * M + row] - lse_tot);
        const f32x4 v = *((const f32x4*)(a.plan.part_o + ((int64_t)(base + i) * M + row) * kDc) + t);
        acc += w * v;
    }
    *o = acc;
    if (a.lse && t == 0) a.lse[(int64_t)b * M + row] = lse_tot;
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    const int row_blocks = (a.rows + 1) / 2;
    const int64_t blocks = (int64_t)a.batch * row_blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
