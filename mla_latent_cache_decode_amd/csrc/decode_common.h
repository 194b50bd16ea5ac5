// Device code shared by the decode kernels: types, the LDS tile swizzle,
// lane-pair reductions, the work plan and buffer descriptors.
#pragma once

#include "mla_internal.h"

#include <type_traits>
#include <utility>

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kChunks = kD / 8;                 // 72 chunks of 8 halves (16 B) per row
constexpr int kTileBytes = kPage * kD * 2;      // 73728: one page of 16-bit elements
constexpr int kKSteps = kD / 16;                // 36 MFMA k-steps for Q.K^T
constexpr int kMdBlocks = kDc / 32;             // 16 output blocks of 32 dims

static_assert(kChunks % 8 == 0, "row must be whole 64-dim column blocks");

#define LGKMCNT0_IMM 0xC07F
#define VMCNT0_IMM 0x0F70
// wait until at most n (< 64) vector-memory operations are outstanding
#define VMCNT_IMM(n) (0x0F70 | ((n) & 15) | ((((n) >> 4) & 3) << 14))

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Read-only per-call metadata (block table, lengths) is read through the
// constant address space so the loads are scalar (SMEM): a vector load here
// would have to wait on vmcnt, which also counts the in-flight page loads.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
    return *(const CONST_AS T*)p;
}

// Slot swizzle of token t: bits (t1, t2, t3) of t become slot bits (2, 1, 0).
// LDS serves 16 lanes of a 128-bit access per pass over 64 banks.  A row
// read of 16 consecutive tokens (Q.K^T fragments, fp8 stores) then hits 16
// distinct 16-byte slots: even tokens cover slots 0..7 of the 256-byte bank
// window, odd tokens 8..15, each through a bijection of (t1, t2, t3).  The
// transposed PV reads touch tokens T, T+1, T+2, T+3 (T = 0 mod 4) in four
// adjacent chunks; slot bit 2 = t1 separates T from T+2 (and T+1 from T+3).
__device__ __forceinline__ int sw(int t) { return (((t >> 1) & 1) << 2) | (((t >> 2) & 1) << 1) | ((t >> 3) & 1); }

// The token (of 16) whose row lane i of a 16-lane group converts and stores.
// 16-byte LDS stores are served 8 lanes (128 bytes) per pass, unlike 16-byte
// reads (16 lanes, 256 bytes): tokens t and t + 1 differ only in address
// bit 7, so they share banks within a 128-byte pass.  Even tokens in lanes
// 0 .. 7 and odd ones in lanes 8 .. 15 give each pass 8 tokens with distinct
// sw(t), i.e. 8 distinct 16-byte bank groups (SQ_LDS_BANK_CONFLICT per
// decode: fp4_b64 5.7M -> 0 cycles, fp8_b64 6.0M -> 1.5M; the reads, 16
// lanes a pass, stay conflict-free either way).
__device__ __forceinline__ int store_token(int i) { return ((i & 7) << 1) | ((i >> 3) & 1); }

// byte offset of (token t, chunk c) inside a tile (16-bit elements)
__device__ __forceinline__ int tile_off(int t, int c) {
    return (((c >> 3) << 9) + (t << 3) + ((c & 7) ^ sw(t))) << 4;
}

// Lanes l and l^32 hold the two halves of one head's tokens.  permlane32_swap
// with both operands = v returns (v[l % 32], v[l % 32 + 32]) in some order, so
// a symmetric combination of the pair is the head-wide reduction.
__device__ __forceinline__ float pair_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float pair_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Workgroup barrier without a memory fence: a fence would make the compiler
// wait for every in-flight page load as well.
// Callers wait for exactly what they need (s_waitcnt) before it; the empty
// asm statements stop the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// o * alpha for a 32x32 accumulator block that lives in AGPRs.  Written as
// asm so the 256-register O accumulator keeps AGPRs as its home: a plain
// VALU multiply would make the register allocator move all of O into arch
// VGPRs and spill.  Only the lazy-rescale path uses it; the last MFMA that
// wrote o is a whole tile (>= 72 MFMAs) earlier and the next MFMA that reads
// it is behind the softmax, so no extra wait states are needed.
// kGrouped: four elements per asm block (four reads, four multiplies, four
// writes, each through its own temporary), so that the three steps of an
// element do not wait on each other; one element per block serialises them
// (about 5k cycles for the 256 elements of O), but leaves the register
// allocator more freedom (the fp4 kernel spills inside its loop with the
// grouped form).
template <bool kGrouped>
__device__ __forceinline__ void scale_acc16(f32x16& o, float alpha) {
    if constexpr (!kGrouped) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = o[r], tmp;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(tmp)
                         : "v"(alpha));
            o[r] = x;
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float x0 = o[4 * q + 0], x1 = o[4 * q + 1], x2 = o[4 * q + 2], x3 = o[4 * q + 3];
        float t0, t1, t2, t3;
        asm volatile(
            "v_accvgpr_read_b32 %4, %0\n\tv_accvgpr_read_b32 %5, %1\n\t"
            "v_accvgpr_read_b32 %6, %2\n\tv_accvgpr_read_b32 %7, %3\n\t"
            "v_mul_f32 %4, %4, %8\n\tv_mul_f32 %5, %5, %8\n\t"
            "v_mul_f32 %6, %6, %8\n\tv_mul_f32 %7, %7, %8\n\t"
            "v_accvgpr_write_b32 %0, %4\n\tv_accvgpr_write_b32 %1, %5\n\t"
            "v_accvgpr_write_b32 %2, %6\n\tv_accvgpr_write_b32 %3, %7"
            : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
            : "v"(alpha));
        o[4 * q + 0] = x0; o[4 * q + 1] = x1; o[4 * q + 2] = x2; o[4 * q + 3] = x3;
    }
}

// The lane id, hidden from loop-invariant code motion.  Lane-derived
// offsets are recomputed from it per tile (a handful of VALU ops) instead of
// being hoisted out of the page loop, where they would occupy registers for
// the whole kernel and push the register allocator into spilling.
__device__ __forceinline__ int opaque_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// A copy of a lane value that the compiler must materialise where it is
// used: offsets derived from it are then computed next to their load instead
// of being hoisted out of the page loop (18 live offsets would spill).
__device__ __forceinline__ int pinned(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// One 1 KiB direct-to-LDS load: lane i's 16 bytes at buffer offset voff land
// at LDS address dst + 16 i.  Issued as asm: the compiler cannot tell that it
// does not alias the tile being read and would otherwise wait for it
// (vmcnt(0)) before every LDS read.  Completion is waited for explicitly.
// The cache is streamed once per workgroup: non-temporal (nt) loads keep it
// from displacing other data in the caches (measured -3.5 % on the long
// context workload).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, uint32_t dst) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(r), "{m0}"(dst) : "memory");
}

// The same load for data that other workgroups read too (the queries): a
// temporal load, so the line stays in the L2 for them.
__device__ __forceinline__ void dma16_shared(__amdgpu_buffer_rsrc_t r, int voff, uint32_t dst) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(dst) : "memory");
}

// bf16 pair -> fp16 pair (round to nearest even; exact inside the fp16 range)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d) {
    const float lo = __builtin_bit_cast(float, d << 16);
    const float hi = __builtin_bit_cast(float, d & 0xFFFF0000u);
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)lo, (_Float16)hi});
}

// ---------------------------------------------------------------------------
// work plan
// ---------------------------------------------------------------------------

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off);
        if (lane >= off) v += t;
    }
    return v;
}

// Exclusive scan of two ints over the NT threads of the block, with the totals.
template <int NT>
__device__ __forceinline__ void block_scan2(int& a, int& b, int& ta, int& tb, int* sbuf, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const int ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
    __syncthreads();
    if (lane == 63) {
        sbuf[wave * 2 + 0] = ia;
        sbuf[wave * 2 + 1] = ib;
    }
    __syncthreads();
    int pa = 0, pb = 0;
    ta = tb = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        if (w < wave) {
            pa += sbuf[w * 2 + 0];
            pb += sbuf[w * 2 + 1];
        }
        ta += sbuf[w * 2 + 0];
        tb += sbuf[w * 2 + 1];
    }
    a = pa + ia - a;
    b = pb + ib - b;
}

struct WorkerStart {
    int b;          // first sequence this worker serves (batch if none)
    int64_t cost;   // cost-axis position where sequence b starts
    int slot;       // first partial slot of sequence b
    int64_t quota;  // cost units per worker
};

// Length of sequence (or sparse unit) b on the work plan's token axis.
__device__ __forceinline__ int plan_len(const DecodeArgs& a, int b) {
    return a.sparse_topk > 0 ? a.sparse_topk : a.seq_lens[b];
}

// The worker's starting point on the cost axis.  With write_info it also
// records, for every sequence whose cost position lies in this worker's
// quota, the number of segments it is split into and its first partial slot
// (read by the combine); only the first row group does that.
// The same plan for a batch of at most 64 sequences: one wave holds every
// length, so each wave forms the whole plan with wave-level scans on its
// own -- no workgroup barrier and no LDS (the planner sits at the head of
// every workgroup's critical path).  Wave 0 of the first row group writes
// the per-sequence records.
__device__ WorkerStart plan_worker_wave(const DecodeArgs& a, int worker, bool write_info, int tid) {
    const int B = a.batch, G = a.num_workers, c = a.overhead_units;
    const int lane = tid & 63;
    const int L = lane < B ? plan_len(a, lane) : 0;
    const int pages = L > 0 ? (L + kPage - 1) / kPage : 0;
    const int cost_in = pages > 0 ? pages + c : 0;
    const int cost_incl = wave_incl_scan(cost_in, lane);
    // results are wave-uniform: readfirstlane keeps them in SGPRs for the
    // segment loop (as VGPRs they would crowd the tile loop's registers)
    const int total = __builtin_amdgcn_readfirstlane(__shfl(cost_incl, 63));
    const int64_t Q = max(max(((int64_t)total + G - 1) / G, (int64_t)a.min_quota), (int64_t)1);
    const int64_t w_lo = (int64_t)worker * Q;
    const int64_t C = cost_incl - cost_in;                  // where sequence `lane` starts
    const int64_t A = C + c, E = A + pages;
    const int n = pages > 0 ? (int)((E - 1) / Q - A / Q + 1) : 0;
    const int slot_in = n > 1 ? n : 0;
    const int slot = wave_incl_scan(slot_in, lane) - slot_in;
    if (write_info && tid < 64 && lane < B) {
        const int64_t owner = pages > 0 ? A / Q : min(C / Q, (int64_t)G - 1);
        if (owner == worker) {
            a.plan.seq_nsplit[lane] = n;
            a.plan.seq_slot[lane] = slot;
        }
    }
    // the first sequence whose pages reach past w_lo
    const unsigned long long m = __builtin_amdgcn_ballot_w64(lane < B && pages > 0 && E > w_lo);
    WorkerStart ws;
    ws.quota = Q;
    if (m) {
        const int first = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(m));
        ws.b = first;
        ws.cost = __builtin_amdgcn_readfirstlane(__shfl((int)C, first));   // C < 2^31 for 64 sequences
        ws.slot = __builtin_amdgcn_readfirstlane(__shfl(slot, first));
    } else {
        ws.b = B;
        ws.cost = 0;
        ws.slot = 0;
    }
    return ws;
}

// NT: threads of the block (a multiple of 64, at most 512; sbuf holds 32 ints)
template <int NT = kDecodeThreads>
__device__ WorkerStart plan_worker(const DecodeArgs& a, int worker, bool write_info, int* sbuf, int tid) {
    static_assert(NT % 64 == 0 && NT <= 512, "block of whole waves, at most 8");
    if (a.batch <= 64) return plan_worker_wave(a, worker, write_info, tid);
    const int B = a.batch, G = a.num_workers, c = a.overhead_units;
    int t_cost = 0;
    const int my_len = tid < B ? plan_len(a, tid) : 0;      // reused by the first chunk
    {
        int local = my_len > 0 ? (my_len + kPage - 1) / kPage + c : 0, zero = 0, tz;
        for (int b = tid + NT; b < B; b += NT) {
            const int L = plan_len(a, b);
            local += L > 0 ? (L + kPage - 1) / kPage + c : 0;
        }
        block_scan2<NT>(local, zero, t_cost, tz, sbuf, tid);
    }
    const int64_t Q = max(max(((int64_t)t_cost + G - 1) / G, (int64_t)a.min_quota), (int64_t)1);
    const int64_t w_lo = (int64_t)worker * Q, w_hi = w_lo + Q;

    WorkerStart ws;
    ws.b = B;
    ws.cost = 0;
    ws.slot = 0;
    ws.quota = Q;
    int64_t carry_cost = 0;
    int carry_slot = 0;
    for (int base = 0; base < B; base += NT) {
        const int b = base + tid;
        int pages = 0;
        if (b < B) {
            const int L = base == 0 ? my_len : plan_len(a, b);
            pages = L > 0 ? (L + kPage - 1) / kPage : 0;
        }
        // a sequence's segment count depends on its cost prefix, so two scans
        int cost_ex = pages > 0 ? pages + c : 0, zero = 0, tc, tz;
        block_scan2<NT>(cost_ex, zero, tc, tz, sbuf, tid);
        const int64_t C = carry_cost + cost_ex;
        const int64_t A = C + c, E = A + pages;
        const int n = pages > 0 ? (int)((E - 1) / Q - A / Q + 1) : 0;
        int slot_ex = n > 1 ? n : 0, zero2 = 0, ts, tz2;
        block_scan2<NT>(slot_ex, zero2, ts, tz2, sbuf, tid);
        const int slot = carry_slot + slot_ex;
        if (write_info && b < B) {
            const int64_t owner = pages > 0 ? A / Q : min(C / Q, (int64_t)G - 1);
            if (owner == worker) {
                a.plan.seq_nsplit[b] = n;
                a.plan.seq_slot[b] = slot;
            }
        }
        if (ws.b == B) {
            // first sequence of this chunk whose pages reach past w_lo
            const bool cand = b < B && pages > 0 && E > w_lo;
            const unsigned long long m = __builtin_amdgcn_ballot_w64(cand);
            __syncthreads();
            if ((tid & 63) == 0) sbuf[16 + (tid >> 6)] = m ? (int)__builtin_ctzll(m) + (tid & ~63) : NT;
            __syncthreads();
            int first = NT;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) first = min(first, sbuf[16 + w]);
            if (first < NT) {
                __syncthreads();
                if (tid == first) {
                    sbuf[24] = (int)(C & 0x3FFFFFFF);
                    sbuf[25] = (int)(C >> 30);
                    sbuf[26] = slot;
                }
                __syncthreads();
                ws.b = base + first;
                ws.cost = ((int64_t)sbuf[25] << 30) | (int64_t)sbuf[24];
                ws.slot = sbuf[26];
            }
        }
        carry_cost += tc;
        carry_slot += ts;
        // stop once past this worker's quota: the sequences it owns are then
        // done too -- except for the last worker, which owns every empty
        // sequence at the end of the cost axis (position total, which equals
        // its w_hi when total is a multiple of the worker count) and so must
        // scan every chunk
        if (carry_cost >= w_hi && worker < G - 1) break;
    }
    __syncthreads();
    return ws;
}

// Page blocks of PS tokens (a power of two, 16 .. 256) under 64-token tiles
// ("DeepSeek-R1" record, engine kernel constraint (1): decode kernels are
// instantiated per page-block size; 64 is the common one, 32 the block of a
// ratio-2 compressed layer).  When PS < 64 a tile spans kRanges pages, one
// per run of kRangeTok consecutive tokens, and each wave loads from one of
// them only (kWavesPerRange waves per page), so a wave still needs a single
// block-table entry and a single buffer descriptor per tile.  When PS >= 64
// a tile lies inside one page, at row (p * 64) % PS.
template <int PS, int NW = kDecodeThreads / 64>
struct PageGeom {
    static_assert(PS >= 16 && PS <= 256 && (PS & (PS - 1)) == 0, "page block: a power of two in 16 .. 256");
    static constexpr int kRanges = PS < kPage ? kPage / PS : 1;
    static constexpr int kRangeTok = kPage / kRanges;
    static constexpr int kWavesPerRange = NW / kRanges;
    static_assert(kWavesPerRange >= 1, "every page of a tile needs a wave");
    // first token (within a tile) of the pages wave w loads from
    __device__ static constexpr int tok0(int wave) { return kRanges == 1 ? 0 : (wave / kWavesPerRange) * kRangeTok; }
    // block-table entry, and row inside that page, of token tok0 of tile p
    // (written per case so that the page-block size of 64 compiles to plain p)
    __device__ static constexpr int entry(int p, int t0) {
        if constexpr (PS < kPage) return p * kRanges + t0 / PS;
        else return p / (PS / kPage);
    }
    __device__ static constexpr int row_in_page(int p, int t0) {
        if constexpr (PS <= kPage) return 0;
        else return (p % (PS / kPage)) * kPage;
    }
    // block-table entries a segment ending at tile p_hi may touch
    __device__ static constexpr int entries(int p_hi) {
        if constexpr (PS < kPage) return p_hi * kRanges;
        else return (p_hi + PS / kPage - 1) / (PS / kPage);
    }
};

// Buffer descriptor over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, int bytes) {
    // both inputs are wave-uniform; say so, or the compiler wraps each load
    // in a waterfall loop
    const uint64_t b = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint8_t* ub = (const uint8_t*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}

// Four consecutive dims of a split's normalised partial output as fp16.
// O / l is a weighted mean of cache values that already passed through fp16
// for the P.V product, so it is inside the fp16 range; the rounding (2^-11
// relative) is far below the output tolerance and halves the bytes the
// split writes and the combine reads.
__device__ __forceinline__ void store_partial4(uint16_t* dst, f32x4 v) {
    const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *(u32x2*)dst = __builtin_bit_cast(u32x2, h);
}

// Workgroups are dealt to the 8 XCDs round robin (block i on XCD i % 8).
// When the worker count G is a multiple of 8, XCD x serves workers
// x * G/8 .. (x + 1) * G/8 - 1, all row groups of each: consecutive workers,
// which the cost-axis plan gives adjacent splits of one sequence, then share
// an L2 and fetch that sequence's queries from HBM once per XCD, and the row
// groups of one worker read each page through the same L2 at about the same
// time, so the cache is fetched from HBM once.
__device__ __forceinline__ void block_role(int G, int& worker, int& rg) {
    if (G % 8 == 0) {
        const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
        const int R = (int)gridDim.x / G;
        rg = j % R;
        worker = xcd * (G / 8) + j / R;
    } else {
        worker = blockIdx.x % G;
        rg = blockIdx.x / G;
    }
}

// Launch a decode kernel: with profile events, through the dispatch that
// records its own start and end timestamps into them; otherwise a plain
// launch (what a captured HIP graph then holds).
template <int NT = kDecodeThreads, typename Kernel>
hipError_t launch_with_events(Kernel kernel, dim3 grid, hipStream_t stream, hipEvent_t ev_start,
                              hipEvent_t ev_stop, const DecodeArgs& a) {
    if (ev_start && ev_stop)
        hipExtLaunchKernelGGL(kernel, grid, dim3(NT), 0, stream, ev_start, ev_stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace mla
