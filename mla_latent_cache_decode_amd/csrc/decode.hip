// Split-KV MLA decode kernels for gfx950 (CDNA4).
//
// What one workgroup computes ("DeepSeek R1 Architecture & Deployment Guide",
// section 1.1): for 128 query rows (heads of one or more query positions) and
// a contiguous range of cache pages of one sequence,
//     S = K Q^T      over the 576-element shared row (latent c, then RoPE k_R),
//     online softmax of S over the tokens,
//     O = V^T P^T    with V = the first 512 elements (the latent c) of the
//                    same rows, since the value up-projection is absorbed
//                    into the output projection downstream.
// Partial results (O/l, lse) of a split go to the workspace for the LSE
// combine; a sequence served by one worker is finished here directly.
//
// Mapping onto CDNA4:
//  * Work plan.  Every workgroup derives its own share from seq_lens: the
//    batch's pages are laid end to end on a cost axis (each sequence charged
//    a fixed overhead for its query load and epilogue) and cut into
//    num_workers equal quotas.  A (worker, sequence) overlap is a segment.
//    No separate planning launch, no host round trip.
//  * 4 waves x 32 rows.  Each wave holds its 32 query rows as MFMA B-operands
//    in registers (36 k-steps x 8 halves) and its O^T accumulator (512 x 32
//    fp32, 256 AGPRs).  Heads are the MFMA N dimension in both products, so
//    softmax statistics of a head live in one lane pair (l, l^32) and the S^T
//    accumulator is directly the B-operand of the PV product.
//  * One 64-token page is one tile.  The workgroup copies it HBM->LDS with
//    buffer loads straight into LDS (no VGPR staging), double buffered, and
//    every wave reuses it for all of its heads: the cache is read from HBM
//    once per workgroup.  Rows past the visible tokens are never fetched (the
//    descriptor size excludes them; the LDS receives zeros).
//  * LDS tile layout: 9 column blocks of 64 dims; within a block, token t's
//    16-byte chunk c sits at slot t*8 + (c ^ sw(t)).  The swizzle keeps the
//    row-wise 128-bit reads of Q.K^T and the transposed 64-bit reads of the
//    PV operand (ds_read_b64_tr_b16) free of bank conflicts.
//  * Both products run as fp16 MFMA with fp32 accumulation.  A landed bf16
//    page is converted to fp16 in place, once per workgroup (exact for
//    values inside the fp16 range: bf16 carries fewer significand bits).
//    fp16 matters for P: its rounding error is 8x below bf16's, which keeps
//    the softmax weights accurate even when the reference max is stale.
//  * Lazy rescaling: the running max is only raised when a tile's max
//    exceeds it by more than 2^15 (in exp2 units), so O is rarely rescaled
//    after the first tile; exponentials stay <= 2^15, inside fp16 range.
//  * Queries are scaled per head by a power of two into [2^14, 2^15) before
//    the fp16 conversion (exact), and the factor is folded into that head's
//    softmax scale, so any query magnitude is representable.
//  * FP8 pages (e4m3 codes + e8m0 per 32) land in an LDS staging buffer and
//    are dequantised once per workgroup into the same fp16 tile layout
//    (exact for values inside the fp16 range).
//  * Operand fragments are read from LDS two MFMA steps ahead of use; the
//    step order is pinned with scheduling barriers.
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

#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr int kChunks = kD / 8;                 // 72 chunks of 8 halves (16 B) per row
constexpr int kTileBytes = kPage * kD * 2;      // 73728: one page of 16-bit elements
constexpr int kKSteps = kD / 16;                // 36 MFMA k-steps for Q.K^T
constexpr int kMdBlocks = kDc / 32;             // 16 output blocks of 32 dims
constexpr int kPvSteps = 4 * kMdBlocks;         // 64 MFMA steps for P.V
constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;   // 18 LDS-direct loads
constexpr int kFp8StageBytes = kPage * kFp8RowBytes;   // 38912
constexpr int kFp8Loads = kFp8StageBytes / 1024;       // 38
constexpr float kRescaleTau = 15.0f;            // log2 units: p <= 2^15 stays inside fp16
constexpr int kQkAhead = 2;                     // K fragment prefetch distance (k-steps)
constexpr int kPvAhead = 2;                     // V fragment prefetch distance (steps)

constexpr int kLdsTiles = 2 * kTileBytes;                       // 147456
constexpr int kLdsTilesFp8 = kTileBytes + 2 * kFp8StageBytes;   // 151552
constexpr int kScanInts = 16;                                   // planner scratch

static_assert(kChunks % 8 == 0, "row must be whole 64-dim column blocks");
static_assert(kFp8StageBytes % 1024 == 0, "fp8 page must be whole 1 KiB load groups");

// s_waitcnt immediate for "vmcnt <= n", other counters unconstrained (gfx9 encoding).
#define VMCNT_IMM(n) ((((n) & 0xF)) | ((((n) >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8))
#define LGKMCNT0_IMM 0xC07F

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Read-only per-call metadata (block table, lengths) is read through the
// constant address space so the loads are scalar (SMEM): a vector load here
// would have to wait on vmcnt, which also counts the in-flight page prefetch.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
    return *(const CONST_AS T*)p;
}

__device__ __forceinline__ int sw(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

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
// wait for the in-flight LDS-direct prefetch of the next page as well.
// Callers wait for exactly what they need (s_waitcnt) before it; the empty
// asm statements stop the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x * alpha for an accumulator element that lives in an AGPR.  Written as
// asm so the 256-register O accumulator keeps AGPRs as its home: a plain
// VALU multiply would make the register allocator move all of O into arch
// VGPRs and spill.  Only the (rare) lazy-rescale path uses it; the last MFMA
// that wrote x is a whole tile (>= 72 MFMAs) earlier and the next MFMA that
// reads it is behind the softmax, so no extra wait states are needed.
__device__ __forceinline__ float scale_acc(float x, float alpha) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(alpha));
    return x;
}

// The lane id, hidden from loop-invariant code motion.  Lane-derived
// offsets are recomputed from it per tile (a handful of VALU ops) instead of
// being hoisted out of the page loop, where they would occupy registers for
// the whole kernel and push the register allocator into spilling.
__device__ __forceinline__ int opaque_lane() {
    int l = __lane_id();
    asm volatile("" : "+v"(l));
    return l;
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

// Exclusive scan of two ints over the 256 threads, with the totals.
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
    for (int w = 0; w < 4; ++w) {
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

// The worker's starting point on the cost axis.  With write_info it also
// records, for every sequence whose cost position lies in this worker's
// quota, the number of segments it is split into and its first partial slot
// (read by the combine); only the first row group does that.
__device__ WorkerStart plan_worker(const DecodeArgs& a, int worker, bool write_info, int* sbuf, int tid) {
    const int B = a.batch, G = a.num_workers, c = a.overhead_units;
    int t_cost = 0;
    const int my_len = tid < B ? a.seq_lens[tid] : 0;      // reused by the first chunk
    {
        int local = my_len > 0 ? (my_len + kPage - 1) / kPage + c : 0, zero = 0, tz;
        for (int b = tid + kDecodeThreads; b < B; b += kDecodeThreads) {
            const int L = a.seq_lens[b];
            local += L > 0 ? (L + kPage - 1) / kPage + c : 0;
        }
        block_scan2(local, zero, t_cost, tz, sbuf, tid);
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
    for (int base = 0; base < B; base += kDecodeThreads) {
        const int b = base + tid;
        int pages = 0;
        if (b < B) {
            const int L = base == 0 ? my_len : a.seq_lens[b];
            pages = L > 0 ? (L + kPage - 1) / kPage : 0;
        }
        // a sequence's segment count depends on its cost prefix, so two scans
        int cost_ex = pages > 0 ? pages + c : 0, zero = 0, tc, tz;
        block_scan2(cost_ex, zero, tc, tz, sbuf, tid);
        const int64_t C = carry_cost + cost_ex;
        const int64_t A = C + c, E = A + pages;
        const int n = pages > 0 ? (int)((E - 1) / Q - A / Q + 1) : 0;
        int slot_ex = n > 1 ? n : 0, zero2 = 0, ts, tz2;
        block_scan2(slot_ex, zero2, ts, tz2, sbuf, tid);
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
            if ((tid & 63) == 0) sbuf[8 + (tid >> 6)] = m ? (int)__builtin_ctzll(m) + (tid & ~63) : kDecodeThreads;
            __syncthreads();
            int first = kDecodeThreads;
#pragma unroll
            for (int w = 0; w < 4; ++w) first = min(first, sbuf[8 + w]);
            if (first < kDecodeThreads) {
                __syncthreads();
                if (tid == first) {
                    sbuf[12] = (int)(C & 0x3FFFFFFF);
                    sbuf[13] = (int)(C >> 30);
                    sbuf[14] = slot;
                }
                __syncthreads();
                ws.b = base + first;
                ws.cost = ((int64_t)sbuf[13] << 30) | (int64_t)sbuf[12];
                ws.slot = sbuf[14];
            }
        }
        carry_cost += tc;
        carry_slot += ts;
        // stop once past this worker's quota (sequences owned by it are then done too)
        if (carry_cost >= w_hi) break;
    }
    __syncthreads();
    return ws;
}

// ---------------------------------------------------------------------------
// page loaders (global -> LDS directly, 16 bytes per lane)
// ---------------------------------------------------------------------------

// Buffer descriptor over [base, base + bytes): lanes whose offset falls past
// `bytes` read zeros, which is how rows beyond the visible tokens are kept
// out of the tile (they are never fetched, and the LDS gets finite zeros).
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

// bf16 page into the swizzled tile.  Load instruction n (0..71) fills tile
// slots [64n, 64n + 64); lane i of it carries token ((n & 7) << 3) + (i >> 3)
// of column block n >> 3.  The lane part of the source offset is the
// constant lane_off (< 8 rows), the rest is a uniform offset.  A full page
// uses one descriptor; a partial page (the last of a sequence) gives every
// load its own descriptor whose size admits only rows below n_valid.  Wave w
// issues instructions 18w .. 18w+17, one per load(i) call, so the caller can
// spread them over other work.
struct Bf16PageLoader {
    const uint8_t* page;
    LDS_AS uint8_t* tile;
    int wave, lane_off, n_valid;
    __amdgpu_buffer_rsrc_t full;

    __device__ __forceinline__ Bf16PageLoader(const uint8_t* page_, LDS_AS uint8_t* tile_, int wave_,
                                              int lane_off_, int n_valid_)
        : page(page_), tile(tile_), wave(wave_), lane_off(lane_off_), n_valid(n_valid_) {
        full = make_rsrc(page, kPage * kBf16RowBytes);
    }
    __device__ __forceinline__ void load(int i) const {
        const int n = wave * kLoadsPerWave + i;
        const int row_blk = (n & 7) << 3;
        if (n_valid >= kPage) {
            const int soff = row_blk * kBf16RowBytes + ((n >> 3) << 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(full, (LDS_AS void*)(tile + n * 1024), 16, lane_off, soff, 0,
                                                     0);
        } else {
            const int rows = min(max(n_valid - row_blk, 0), 8);
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(page + row_blk * kBf16RowBytes + ((n >> 3) << 7), rows * kBf16RowBytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(tile + n * 1024), 16, lane_off, 0, 0, 0);
        }
    }
};

// fp8 page, row-major into a staging buffer; waves 0,1 issue 10 loads, 2,3 issue 9.
__device__ __forceinline__ void load_page_fp8(const uint8_t* page, LDS_AS uint8_t* stage, int wave,
                                              int lane, int n_valid) {
    const int valid_bytes = n_valid * kFp8RowBytes;
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const int n = wave + 4 * i;
        if (n < kFp8Loads) {
            const int bytes = min(max(valid_bytes - n * 1024, 0), 1024);
            const __amdgpu_buffer_rsrc_t r = make_rsrc(page + n * 1024, bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(stage + n * 1024), 16, lane * 16, 0, 0,
                                                     0);
        }
    }
}

__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
    // 2^(e-127); e = 0 is the fp32 subnormal 2^-127, e = 255 is NaN
    uint32_t bits = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : (e << 23));
    return __builtin_bit_cast(float, bits);
}

// Dequantise a staged fp8 page into the fp16 tile (all 256 threads, 18
// units of 8 values each, in two batches of 9: a batch's reads are all
// issued before its first conversion so the LDS round trips overlap).
__device__ __forceinline__ void convert_fp8_page(const LDS_AS uint8_t* stage, LDS_AS uint8_t* tile,
                                                 int tid) {
    constexpr int kUnits = kPage * kChunks / kDecodeThreads;
    constexpr int kBatch = kUnits / 2;
    static_for<0, 2>([&](auto h_c) {
        constexpr int h = decltype(h_c)::value;
        u32x2 codes[kBatch];
        uint32_t sc[kBatch];
        static_for<0, kBatch>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            const int u = tid + kDecodeThreads * (h * kBatch + k);
            const int t = u / kChunks;
            const int c = u - t * kChunks;
            const LDS_AS uint8_t* row = stage + t * kFp8RowBytes;
            codes[k] = *(const LDS_AS u32x2*)(row + c * 8);
            sc[k] = row[kD + (c >> 2)];
        });
        static_for<0, kBatch>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            const int u = tid + kDecodeThreads * (h * kBatch + k);
            const int t = u / kChunks;
            const int c = u - t * kChunks;
            const float scale = e8m0_to_float(sc[k]);
            f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[k][0], scale, false);
            f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[k][0], scale, true);
            f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[k][1], scale, false);
            f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[k][1], scale, true);
            f16x8 v = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            *(LDS_AS f16x8*)(tile + tile_off(t, c)) = v;
        });
    });
}

// Convert a landed bf16 tile to fp16 in place (all 256 threads, 18 chunks
// of 16 bytes each, read and written by the same thread), in two batches
// of 9 whose reads are all issued before the first conversion.  If a loader
// is given, its 18 page loads (into the other buffer) are interleaved with
// the conversions, so the load path works in the background.
struct NoLoads {
    __device__ __forceinline__ void load(int) const {}
};

template <typename Loader>
__device__ __forceinline__ void convert_bf16_tile(LDS_AS uint8_t* tile, int tid, Loader ld) {
    constexpr int kUnits = kTileBytes / 16 / kDecodeThreads;
    constexpr int kBatch = kUnits / 2;
    LDS_AS uint8_t* base = tile + tid * 16;
    static_for<0, 2>([&](auto h_c) {
        constexpr int h = decltype(h_c)::value;
        u32x4 v[kBatch];
        static_for<0, kBatch>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            v[k] = *(const LDS_AS u32x4*)(base + (h * kBatch + k) * kDecodeThreads * 16);
        });
        static_for<0, kBatch>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            ld.load(h * kBatch + k);
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __builtin_bit_cast(float, v[k][i] << 16);
                const float hi = __builtin_bit_cast(float, v[k][i] & 0xFFFF0000u);
                const f16x2 hv = {(_Float16)lo, (_Float16)hi};
                r[i] = __builtin_bit_cast(uint32_t, hv);
            }
            *(LDS_AS u32x4*)(base + (h * kBatch + k) * kDecodeThreads * 16) = r;
        });
    });
}

// ---------------------------------------------------------------------------
// per-tile compute of one wave: 32 heads x 64 tokens
// ---------------------------------------------------------------------------
struct WaveState {
    f32x16 o[kMdBlocks];     // O^T accumulator: dims x heads
    float m;                 // running max (log2 units, lane's head)
    float l;                 // partial sum of exp over this lane's half of the tokens
    bool o_zero;             // nothing accumulated yet (wave-uniform)
};

__device__ __forceinline__ void compute_tile(const LDS_AS uint8_t* tile, const f16x8 (&qf)[kKSteps],
                                             WaveState& st, int n_valid, float scale_log2) {
    const int lane = opaque_lane();
    const int hi = lane >> 5;

    // ---- S^T = K Q^T : two 32-token blocks (two independent MFMA chains).
    // Fragment of k-step ks: token (lane & 31) [+32], chunk 2*ks + hi, i.e.
    // tile_off(lane & 31, 2*(ks & 3) + hi) + (ks >> 2) * 8192 [+ 4096].
    int k_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) k_off[k] = tile_off(lane & 31, 2 * k + hi);
    f32x16 s0 = {}, s1 = {};
    f16x8 kf[kQkAhead + 1][2];
    auto read_k = [&](auto ks_c, f16x8 (&dst)[2]) {
        constexpr int ks = decltype(ks_c)::value;
        const LDS_AS uint8_t* base = tile + k_off[ks & 3] + (ks >> 2) * 8192;
        dst[0] = *(const LDS_AS f16x8*)(base);
        dst[1] = *(const LDS_AS f16x8*)(base + 4096);
    };
    static_for<0, kQkAhead>([&](auto i) { read_k(i, kf[decltype(i)::value]); });
    static_for<0, kKSteps>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        if constexpr (ks + kQkAhead < kKSteps)
            read_k(std::integral_constant<int, ks + kQkAhead>{}, kf[(ks + kQkAhead) % (kQkAhead + 1)]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks % (kQkAhead + 1)][0], qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks % (kQkAhead + 1)][1], qf[ks], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    });
    // the scores feed VALU work (softmax): keep them in arch VGPRs
    asm volatile("" : "+v"(s0), "+v"(s1));

    // ---- softmax.  Tokens >= n_valid (tail of the sequence / causal limit)
    // are masked branch-free: excluded from the max and given p = 0.  The
    // token of register r is c_r + 4*hi (+32 for s1); compare c_r with nv_lane.
    const int nv_lane = n_valid - (hi << 2);
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int c_r = ((r >> 2) << 3) + (r & 3);
        mx = fmaxf(mx, c_r < nv_lane ? s0[r] : -__builtin_inff());
        mx = fmaxf(mx, c_r + 32 < nv_lane ? s1[r] : -__builtin_inff());
    }
    mx = pair_max(mx);
    const float mx2 = mx * scale_log2;
    const bool need = mx2 > st.m + kRescaleTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mx2 : st.m;
        if (!st.o_zero) {
            const float alpha = need ? fast_exp2(st.m - m_new) : 1.0f;
#pragma unroll
            for (int md = 0; md < kMdBlocks; ++md) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[md][r] = scale_acc(st.o[md][r], alpha);
            }
            st.l *= alpha;
        }
        st.m = m_new;
    }
    const float neg_m = -st.m;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int c_r = ((r >> 2) << 3) + (r & 3);
        const float p0 = c_r < nv_lane ? fast_exp2(fmaf(s0[r], scale_log2, neg_m)) : 0.f;
        const float p1 = c_r + 32 < nv_lane ? fast_exp2(fmaf(s1[r], scale_log2, neg_m)) : 0.f;
        s0[r] = p0;
        s1[r] = p1;
        lsum += p0 + p1;
    }
    st.l += lsum;
    f16x8 pf[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pf[0][e] = (_Float16)s0[e];
        pf[1][e] = (_Float16)s0[8 + e];
        pf[2][e] = (_Float16)s1[e];
        pf[3][e] = (_Float16)s1[8 + e];
    }

    // ---- O^T += V^T P^T.  Step s covers (kb = s >> 4, md = s & 15); its V^T
    // fragment is two transposed reads (tokens kb*16 + e4*8 + tok_lane, dims
    // md*32 + dim_lane).  The reads are issued as asm because the compiler
    // cannot tell they do not alias the page prefetch still in flight and
    // would wait for it (vmcnt(0)); the lgkmcnt wait is tied to the
    // fragment so the MFMA cannot move above it, and fragment buffers rotate
    // so a read never overwrites an operand of the MFMA issued just before.
    __builtin_amdgcn_sched_barrier(0);
    uint32_t vp[2];
    {
        const int g = lane >> 4, li = lane & 15;
        const int tok = ((g >> 1) << 2) + (li >> 2);
        const int dim = ((g & 1) << 4) + ((li & 3) << 2);
#pragma unroll
        for (int m = 0; m < 2; ++m)
            vp[m] = (uint32_t)(uintptr_t)(tile + tile_off(tok, (m * 32 + dim) >> 3) + (dim & 7) * 2);
    }
    constexpr int kVBufs = kPvAhead + 2;
    f16x8 vf[kVBufs];
    auto read_v = [&](auto step_c) -> f16x8 {
        constexpr int step = decltype(step_c)::value;
        constexpr int kb_ = step >> 4, md = step & 15;
        constexpr int off = (md >> 1) * 8192 + kb_ * 16 * 128;
        f16x4 v0, v1;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v0) : "v"(vp[md & 1]), "i"(off));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v1) : "v"(vp[md & 1]), "i"(off + 8 * 128));
        return f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    };
    static_assert(kPvAhead == 2, "the lgkmcnt immediates below assume two steps in flight");
    static_for<0, kPvAhead>([&](auto i) { vf[decltype(i)::value] = read_v(i); });
    static_for<0, kPvSteps>([&](auto step_c) {
        constexpr int step = decltype(step_c)::value;
        constexpr int ahead = (step + kPvAhead < kPvSteps) ? kPvAhead : (kPvSteps - 1 - step);
        if constexpr (step + kPvAhead < kPvSteps) {
            vf[(step + kPvAhead) % kVBufs] = read_v(std::integral_constant<int, step + kPvAhead>{});
            // the previous MFMA's operand stays allocated across this read
            if constexpr (step > 0) asm volatile("" ::"v"(vf[(step - 1) % kVBufs]));
        }
        if constexpr (ahead == 2) asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(vf[step % kVBufs]));
        else if constexpr (ahead == 1) asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(vf[step % kVBufs]));
        else asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vf[step % kVBufs]));
        st.o[step & 15] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[step % kVBufs], pf[step >> 4], st.o[step & 15],
                                                                  0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);     // keep [read s+ahead, wait, mfma s] in order
    });
    // keep the accumulator's home in AGPRs (it is only touched by MFMA in the
    // steady state); VALU users copy out and back
#pragma unroll
    for (int md = 0; md < kMdBlocks; ++md) asm volatile("" : "+a"(st.o[md]));
    st.o_zero = false;
}

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------
template <bool kFp8>
__global__ __launch_bounds__(kDecodeThreads, 1) void mla_decode_kernel(DecodeArgs a) {
    constexpr int kTileRegion = kFp8 ? kLdsTilesFp8 : kLdsTiles;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kTileRegion + kScanInts * 4];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
    int* sbuf = (int*)(smem + kTileRegion);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.num_workers;
    const int worker = blockIdx.x % G;
    const int rg = blockIdx.x / G;
    const int M = a.s_q * a.n_h;
    const int row0 = rg * kRowsPerGroup + wave * kRowsPerWave;
    const bool active = row0 < M;
    const int j_wave = (active ? row0 : M - 1) / a.n_h;
    const int j_last = min(rg * kRowsPerGroup + kRowsPerGroup - 1, M - 1) / a.n_h;

    const WorkerStart start = plan_worker(a, worker, rg == 0, sbuf, tid);
    if (start.b >= a.batch) return;
    const int64_t Q = start.quota;
    const int64_t w_lo = (int64_t)worker * Q, w_hi = w_lo + Q;

    // zero the LDS once so that nothing in it is ever uninitialised
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int off = tid * 16; off < kTileRegion; off += kDecodeThreads * 16) *(LDS_AS f32x4*)(lds + off) = z;
    }
    __syncthreads();

    LDS_AS uint8_t* tile_c = lds;                          // fp8: the single fp16 tile
    LDS_AS uint8_t* bufs[2];
    if (kFp8) {
        bufs[0] = lds + kTileBytes;
        bufs[1] = lds + kTileBytes + kFp8StageBytes;
    } else {
        bufs[0] = lds;
        bufs[1] = lds + kTileBytes;
    }

    int64_t cost = start.cost;
    int slot_base = start.slot;
    for (int b = start.b; b < a.batch; ++b) {
        const int L = ld_const(a.seq_lens + b);
        const int pages = L > 0 ? (L + kPage - 1) / kPage : 0;
        if (pages == 0) continue;
        const int64_t A = cost + a.overhead_units, E = A + pages;
        if (A >= w_hi) break;
        cost = E;
        const int n = (int)((E - 1) / Q - A / Q + 1);
        const int this_slot_base = slot_base;
        slot_base += n > 1 ? n : 0;
        if (E <= w_lo) continue;
        const int p_lo = (int)(max(w_lo, A) - A);
        const int p_hi = (int)(min(w_hi, E) - A);
        const int split = (int)(max(w_lo, A) / Q - A / Q);
        const int slot = n > 1 ? this_slot_base + split : -1;

        const int n_vis = L - a.s_q + 1 + j_wave;           // tokens this wave may see
        const int n_load = L - a.s_q + 1 + j_last;          // tokens the workgroup loads
        const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks;

        // issue(p, phys, dst): load logical page p (physical page phys).  The
        // block-table entry is read a tile ahead of its use (next_phys), so
        // the scalar load's latency is not on the issue path.
        auto bf16_loader = [&](int p, int phys, LDS_AS uint8_t* dst) {
            const int ol = opaque_lane();
            const int ld_tok = ol >> 3;                           // bf16 loader lane offset
            return Bf16PageLoader(a.kv + (int64_t)phys * a.page_bytes, dst, wave,
                                  ld_tok * kBf16RowBytes + (((ol & 7) ^ sw(ld_tok)) << 4),
                                  min(max(n_load - p * kPage, 0), kPage));
        };
        auto issue = [&](int p, int phys, LDS_AS uint8_t* dst) {
            if (kFp8) {
                load_page_fp8(a.kv + (int64_t)phys * a.page_bytes, dst, wave, opaque_lane(),
                              min(max(n_load - p * kPage, 0), kPage));
            } else {
                const Bf16PageLoader ld = bf16_loader(p, phys, dst);
#pragma unroll
                for (int i = 0; i < kLoadsPerWave; ++i) ld.load(i);
            }
        };
        auto phys_of = [&](int p) -> int { return p < p_hi ? ld_const(bt + p) : 0; };

        // this wave's 32 query rows as MFMA B operands (q_abs || q_R): bf16
        // loaded, scaled per head by 2^-sh so the head's max |q| lands in
        // [2^14, 2^15), converted to fp16 (exact up to fp16 subnormals); the
        // head's softmax scale absorbs 2^sh
        f16x8 qf[kKSteps];
        float scale_lane;
        WaveState st;
        st.m = -__builtin_inff();
        st.l = 0.f;
        st.o_zero = true;
#pragma unroll
        for (int md = 0; md < kMdBlocks; ++md) st.o[md] = f32x16{};
        {
            const int lane = tid & 63;
            const int row = active ? row0 + (lane & 31) : 0;
            const uint16_t* qrow = a.q + ((int64_t)b * M + row) * kD + (lane >> 5) * 8;
            float qmax = 0.f;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                const bf16x8 qb = *(const bf16x8*)(qrow + ks * 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf((float)qb[e]));
                qf[ks] = __builtin_bit_cast(f16x8, qb);          // raw bits for now
            }
            qmax = pair_max(qmax);
            // exponent of qmax (a normal or zero float after the bf16 widening)
            const int ex = qmax > 0.f ? (int)((__builtin_bit_cast(uint32_t, qmax) >> 23) & 0xFF) - 127 : 14;
            const int sh = ex - 14;
            const float down = __builtin_bit_cast(float, (uint32_t)(127 - sh) << 23);   // 2^-sh
            const float up = __builtin_bit_cast(float, (uint32_t)(127 + sh) << 23);     // 2^sh
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                const bf16x8 qb = __builtin_bit_cast(bf16x8, qf[ks]);
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[ks][e] = (_Float16)((float)qb[e] * down);
            }
            scale_lane = a.scale_log2 * up;
        }

        // Page pipeline.  bf16: two LDS tiles, a landed page is converted in
        // place.  fp8: two staging buffers and one fp16 tile.  Per tile two
        // workgroup barriers: "page p+1 landed and everyone is done with the
        // tile" and "page p+1 converted".
        auto wait_loads = [&](bool keep_one_page) {
            // every load instruction is issued (rows past the end read zeros),
            // so the counts are exact; the query loads are older than any page
            if (keep_one_page) {
                if (kFp8) {
                    if (wave < 2) __builtin_amdgcn_s_waitcnt(VMCNT_IMM(10));
                    else __builtin_amdgcn_s_waitcnt(VMCNT_IMM(9));
                } else {
                    __builtin_amdgcn_s_waitcnt(VMCNT_IMM(kLoadsPerWave));
                }
            } else {
                __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
            }
        };
        // convert page p; bf16 may carry the loads of the page after next
        auto convert = [&](int p, auto ld) {
            if (kFp8) convert_fp8_page(bufs[(p - p_lo) & 1], tile_c, wave * 64 + opaque_lane());
            else convert_bf16_tile(bufs[(p - p_lo) & 1], wave * 64 + opaque_lane(), ld);
            __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
            wg_barrier();
        };

        // prefetch (after the query loads, so that waiting for a page also
        // covers the query fragments)
        issue(p_lo, phys_of(p_lo), bufs[0]);
        if (p_lo + 1 < p_hi) issue(p_lo + 1, phys_of(p_lo + 1), bufs[1]);
        const int ahead = kFp8 ? 3 : 2;          // the page a tile's end issues
        int next_phys = phys_of(p_lo + ahead - 1);
        wait_loads(p_lo + 1 < p_hi);
        wg_barrier();
        convert(p_lo, NoLoads{});
        if (kFp8 && p_lo + 2 < p_hi) issue(p_lo + 2, next_phys, bufs[0]);

        for (int p = p_lo; p < p_hi; ++p) {
            next_phys = phys_of(p + ahead);
            const LDS_AS uint8_t* tile = kFp8 ? tile_c : bufs[(p - p_lo) & 1];
            // inactive waves (rows beyond M) compute on row 0's query and
            // discard the result: keeping the call unconditional keeps the
            // accumulators out of control-flow merges
            compute_tile(tile, qf, st, min(max(n_vis - p * kPage, 0), kPage), scale_lane);

            __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);           // this wave's LDS reads retired
            if (p + 1 < p_hi) {
                // fp8 keeps page p+2 in flight; bf16 has only page p+1 outstanding
                wait_loads(kFp8 && p + 2 < p_hi);
                wg_barrier();
                if (kFp8) {
                    convert(p + 1, NoLoads{});
                    if (p + 3 < p_hi) issue(p + 3, next_phys, bufs[(p + 1 - p_lo) & 1]);
                } else if (p + 2 < p_hi) {
                    convert(p + 1, bf16_loader(p + 2, next_phys, bufs[(p - p_lo) & 1]));
                } else {
                    convert(p + 1, NoLoads{});
                }
            } else {
                wg_barrier();       // buffers are reused by the next segment
            }
        }

        // epilogue: normalise and write final output or the split's partial
        if (active) {
            const int lane = tid & 63;
            const float l_tot = pair_sum(st.l);
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            const float lse_v = l_tot > 0.f ? (st.m + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                            : -__builtin_inff();
            const int row = row0 + (lane & 31);
            float* dst = slot < 0 ? a.out + ((int64_t)b * M + row) * kDc
                                  : a.plan.part_o + ((int64_t)slot * M + row) * kDc;
            const int hi = lane >> 5;
#pragma unroll
            for (int md = 0; md < kMdBlocks; ++md) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 v = {st.o[md][r4 * 4 + 0] * inv, st.o[md][r4 * 4 + 1] * inv,
                               st.o[md][r4 * 4 + 2] * inv, st.o[md][r4 * 4 + 3] * inv};
                    *(f32x4*)(dst + md * 32 + r4 * 8 + hi * 4) = v;
                }
            }
            if (lane < 32) {
                if (slot < 0) {
                    if (a.lse) a.lse[(int64_t)b * M + row] = lse_v;
                } else {
                    a.plan.part_lse[(int64_t)slot * M + row] = lse_v;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int row_groups, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_kernel<false>, dim3(a.num_workers * row_groups), dim3(kDecodeThreads), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int row_groups, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_kernel<true>, dim3(a.num_workers * row_groups), dim3(kDecodeThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace mla
