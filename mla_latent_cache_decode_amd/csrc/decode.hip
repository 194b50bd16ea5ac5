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
//  * 4 waves x 32 rows.  Each wave holds its 32 query rows as MFMA B-operands
//    in registers (36 k-steps x 8 bf16) and its O^T accumulator (512 x 32
//    fp32, 256 registers).  Heads are the MFMA N dimension in both products,
//    so softmax statistics of a head live in one lane pair (l, l^32) and the
//    S^T accumulator is directly the B-operand of the PV product.
//  * One 64-token page is one tile.  The whole workgroup copies it HBM->LDS
//    with direct-to-LDS loads (no VGPR staging), double buffered, and every
//    wave reuses it for all of its heads: the cache is read from HBM once per
//    workgroup.
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
#include "mla_internal.h"

#include <type_traits>
#include <utility>

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_tr __attribute__((__vector_size__(4 * sizeof(__fp16))));   // tr-read builtin type
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr int kChunks = kD / 8;                 // 72 chunks of 8 bf16 (16 B) per row
constexpr int kTileBytes = kPage * kD * 2;      // 73728: one page as bf16
constexpr int kKSteps = kD / 16;                // 36 MFMA k-steps for Q.K^T
constexpr int kMdBlocks = kDc / 32;             // 16 output blocks of 32 dims
constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;   // 18 direct-to-LDS loads
constexpr int kFp8StageBytes = kPage * kFp8RowBytes;   // 38912
constexpr int kFp8Loads = kFp8StageBytes / 1024;       // 38
constexpr float kRescaleTau = 15.0f;            // log2 units: p <= 2^15 stays inside fp16

constexpr int kLdsBf16 = 2 * kTileBytes;                        // 147456
constexpr int kLdsFp8 = kTileBytes + 2 * kFp8StageBytes;        // 151552

static_assert(kChunks % 8 == 0, "row must be whole 64-dim column blocks");
static_assert(kFp8StageBytes % 1024 == 0, "fp8 page must be whole 1 KiB load groups");

// s_waitcnt immediate for "vmcnt <= n", other counters unconstrained (gfx9 encoding).
#define VMCNT_IMM(n) ((((n) & 0xF)) | ((((n) >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8))

#define CONST_AS __attribute__((address_space(4)))

// Read-only per-call metadata (block table, lengths, plan) is read through
// the constant address space so the loads are scalar (SMEM): a vector load
// here would have to wait on vmcnt, which also counts the in-flight page
// prefetch.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
    return *(const CONST_AS T*)p;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
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
// wait for the in-flight direct-to-LDS prefetch of the next page as well.
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

// ---------------------------------------------------------------------------
// page loaders (direct global -> LDS, 16 bytes per lane)
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
// load its own descriptor whose size admits only rows below n_valid.
__device__ __forceinline__ void load_page_bf16(const uint8_t* page, LDS_AS uint8_t* tile, int wave,
                                               int lane_off, int n_valid) {
    if (n_valid >= kPage) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(page, kPage * kBf16RowBytes);
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
            const int n = wave * kLoadsPerWave + i;
            const int soff = ((n & 7) << 3) * kBf16RowBytes + ((n >> 3) << 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(tile + n * 1024), 16, lane_off, soff,
                                                     0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
            const int n = wave * kLoadsPerWave + i;
            const int row_blk = (n & 7) << 3;
            const int rows = min(max(n_valid - row_blk, 0), 8);
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(page + row_blk * kBf16RowBytes + ((n >> 3) << 7), rows * kBf16RowBytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(tile + n * 1024), 16, lane_off, 0, 0, 0);
        }
    }
}

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

// Dequantise a staged fp8 page into the fp16 tile (all 256 threads).
__device__ __forceinline__ void convert_fp8_page(const LDS_AS uint8_t* stage, LDS_AS uint8_t* tile,
                                                 int tid) {
#pragma unroll 6
    for (int k = 0; k < kPage * kChunks / kDecodeThreads; ++k) {
        const int u = tid + kDecodeThreads * k;
        const int t = u / kChunks;
        const int c = u - t * kChunks;
        const LDS_AS uint8_t* row = stage + t * kFp8RowBytes;
        const u32x2 codes = *(const LDS_AS u32x2*)(row + c * 8);
        const float scale = e8m0_to_float(row[kD + (c >> 2)]);
        f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[0], scale, false);
        f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[0], scale, true);
        f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[1], scale, false);
        f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[1], scale, true);
        f16x8 v = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        *(LDS_AS f16x8*)(tile + tile_off(t, c)) = v;
    }
}

// Convert a landed bf16 tile to fp16 in place (all 256 threads, 18 chunks
// of 16 bytes each; a chunk is read and written by the same thread).
__device__ __forceinline__ void convert_bf16_tile(LDS_AS uint8_t* tile, int tid) {
#pragma unroll 6
    for (int k = 0; k < kTileBytes / 16 / kDecodeThreads; ++k) {
        LDS_AS u32x4* p = (LDS_AS u32x4*)(tile + (tid + kDecodeThreads * k) * 16);
        const u32x4 v = *p;
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __builtin_bit_cast(float, v[i] << 16);
            const float hi = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
            const f16x2 h = {(_Float16)lo, (_Float16)hi};
            r[i] = __builtin_bit_cast(uint32_t, h);
        }
        *p = r;
    }
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

// The lane id, hidden from loop-invariant code motion.  Lane-derived
// offsets are recomputed from it per tile (a handful of VALU ops) instead of
// being hoisted out of the page loop, where they would occupy registers for
// the whole kernel and push the register allocator into spilling.
__device__ __forceinline__ int opaque_lane() {
    int l = __lane_id();
    asm volatile("" : "+v"(l));
    return l;
}

// Lane-constant byte offsets into a tile (see tile_off):
//   k_off[k]  Q.K^T A-operand: token (lane & 31), chunk 2*ks + (lane >> 5) for
//             ks & 3 == k; add (ks >> 2) * 8192 + mb * 4096.
//   v_off[m]  PV A-operand (transposed read): token tok_lane, dims
//             md*32 + dim_lane for md & 1 == m; add (md >> 1) * 8192 +
//             (kb * 16 + e4 * 8) * 128.
struct LaneOffsets {
    int k_off[4];
    int v_off[2];
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
    LaneOffsets o;
    const int t = lane & 31;
    const int hi = lane >> 5;
#pragma unroll
    for (int k = 0; k < 4; ++k) o.k_off[k] = tile_off(t, 2 * k + hi);
    const int g = lane >> 4;
    const int li = lane & 15;
    const int tok = ((g >> 1) << 2) + (li >> 2);
    const int dim = ((g & 1) << 4) + ((li & 3) << 2);
#pragma unroll
    for (int m = 0; m < 2; ++m) o.v_off[m] = tile_off(tok, (m * 32 + dim) >> 3) + (dim & 7) * 2;
    return o;
}

__device__ __forceinline__ void compute_tile(const LDS_AS uint8_t* tile, const f16x8 (&qf)[kKSteps],
                                             WaveState& st, int n_valid, float scale_log2) {
    const int lane = opaque_lane();
    const LaneOffsets lo = lane_offsets(lane);
    const int hi = lane >> 5;
    const LDS_AS uint8_t* kp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) kp[k] = tile + lo.k_off[k];

    // S^T = K Q^T : two 32-token blocks.  Fragments are read one k-step
    // ahead; the scheduling groups keep that order so at most two k-steps of
    // fragments are live (the scheduler would otherwise hoist every read).
    f32x16 s0 = {}, s1 = {};
    f16x8 ka[2], kb[2];
    ka[0] = *(const LDS_AS f16x8*)(kp[0]);
    kb[0] = *(const LDS_AS f16x8*)(kp[0] + 4096);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + 1 < kKSteps) {
            const LDS_AS uint8_t* base = kp[(ks + 1) & 3] + ((ks + 1) >> 2) * 8192;
            ka[(ks + 1) & 1] = *(const LDS_AS f16x8*)(base);
            kb[(ks + 1) & 1] = *(const LDS_AS f16x8*)(base + 4096);
        }
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks & 1], qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[ks & 1], qf[ks], s1, 0, 0, 0);
        if (ks + 1 < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                          // 2 MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
    // the scores feed VALU work (softmax): keep them in arch VGPRs
    asm volatile("" : "+v"(s0), "+v"(s1));

    // tokens >= n_valid (tail of the sequence / causal limit) are masked
    // branch-free: excluded from the max here and given p = 0 below.  Token of
    // register r is c_r + 4*hi (+32 for s1), so compare c_r with nv_lane.
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

    // P = exp2(S*scale_log2 - m); masked entries are exactly 0
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

    // O^T += V^T P^T ; V^T fragments through transposed LDS reads, one
    // (kb, md) step ahead of their MFMA.  The reads are issued as asm: the
    // compiler cannot tell that they do not alias the page prefetch still
    // in flight and would otherwise wait for it (vmcnt(0)) here.  The
    // lgkmcnt wait is tied to the fragment registers so the MFMA cannot be
    // scheduled above it.
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t vp0 = (uint32_t)(uintptr_t)(tile + lo.v_off[0]);
    const uint32_t vp1 = (uint32_t)(uintptr_t)(tile + lo.v_off[1]);
    // three rotating fragment buffers: a read never targets the registers of
    // the MFMA issued just before it (no write-after-read on its operands)
    f16x8 vf[3];
    auto read_v = [&](auto step_c) -> f16x8 {
        constexpr int step = decltype(step_c)::value;
        constexpr int kb_ = step >> 4, md = step & 15;
        constexpr int off = (md >> 1) * 8192 + kb_ * 16 * 128;
        f16x4 v0, v1;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v0) : "v"((md & 1) ? vp1 : vp0), "i"(off));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(v1)
                     : "v"((md & 1) ? vp1 : vp0), "i"(off + 8 * 128));
        return f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    };
    vf[0] = read_v(std::integral_constant<int, 0>{});
    static_for<0, 4 * kMdBlocks>([&](auto step_c) {
        constexpr int step = decltype(step_c)::value;
        if constexpr (step + 1 < 4 * kMdBlocks) {
            vf[(step + 1) % 3] = read_v(std::integral_constant<int, step + 1>{});
            // the previous MFMA's operand stays allocated across this read
            if constexpr (step > 0) asm volatile("" ::"v"(vf[(step + 2) % 3]));
            asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(vf[step % 3]));
        } else {
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vf[step % 3]));
        }
        st.o[step & 15] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[step % 3], pf[step >> 4], st.o[step & 15],
                                                                  0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);     // keep [read s+1, wait, mfma s] in order
    });
    __builtin_amdgcn_sched_barrier(0);
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
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kFp8 ? kLdsFp8 : kLdsBf16];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.num_workers;
    const int worker = blockIdx.x % G;
    const int rg = blockIdx.x / G;
    const int M = a.s_q * a.n_h;
    const int row0 = rg * kRowsPerGroup + wave * kRowsPerWave;
    const bool active = row0 < M;
    const int j_wave = (active ? row0 : M - 1) / a.n_h;
    const int j_last = min(rg * kRowsPerGroup + kRowsPerGroup - 1, M - 1) / a.n_h;

    // values the compiler cannot prove uniform are made so explicitly, so
    // descriptors and LDS bases stay in SGPRs (no waterfall loops)
    const int seg_begin = ld_const(a.plan.worker_start + worker);
    const int seg_end = ld_const(a.plan.worker_start + worker + 1);
    if (seg_begin >= seg_end) return;

    // zero the LDS once so rows that are never loaded hold finite values
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int off = tid * 16; off < (kFp8 ? kLdsFp8 : kLdsBf16); off += kDecodeThreads * 16)
            *(LDS_AS f32x4*)(lds + off) = z;
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

    for (int s = seg_begin; s < seg_end; ++s) {
        const int32_t* sg = (const int32_t*)(a.plan.segs + s);    // {b, page_lo, page_hi, slot}
        const int b = ld_const(sg + 0);
        const int p_lo = ld_const(sg + 1);
        const int p_hi = ld_const(sg + 2);
        const int slot = ld_const(sg + 3);
        const int L = ld_const(a.seq_lens + b);
        const int n_vis = L - a.s_q + 1 + j_wave;           // tokens this wave may see
        const int n_load = L - a.s_q + 1 + j_last;          // tokens the workgroup loads
        const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks;

        auto page_ptr = [&](int p) -> const uint8_t* {
            return a.kv + (int64_t)ld_const(bt + p) * a.page_bytes;
        };
        auto issue = [&](int p, LDS_AS uint8_t* dst) {
            const int nv = min(max(n_load - p * kPage, 0), kPage);
            const int ol = opaque_lane();
            if (kFp8) {
                load_page_fp8(page_ptr(p), dst, wave, ol, nv);
            } else {
                const int ld_tok = ol >> 3;                       // bf16 loader lane offset
                load_page_bf16(page_ptr(p), dst, wave, ld_tok * kBf16RowBytes + (((ol & 7) ^ sw(ld_tok)) << 4), nv);
            }
        };

        // this wave's 32 query rows as MFMA B operands (q_abs || q_R): bf16
        // loaded, scaled per head by 2^-a so the head's max |q| lands in
        // [2^14, 2^15), converted to fp16 (exact up to fp16 subnormals); the
        // head's softmax scale absorbs 2^a
        f16x8 qf[kKSteps];
        float scale_lane;
        WaveState st;
        st.m = -__builtin_inff();
        st.l = 0.f;
        st.o_zero = true;
#pragma unroll
        for (int md = 0; md < kMdBlocks; ++md) st.o[md] = f32x16{};
        {
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

        // prefetch the first two pages of the segment (after the query loads,
        // so that waiting for page p_lo also covers the query fragments)
        issue(p_lo, bufs[0]);
        if (p_lo + 1 < p_hi) issue(p_lo + 1, bufs[1]);

        for (int p = p_lo; p < p_hi; ++p) {
            const int sb = (p - p_lo) & 1;
            // wait for page p: the only loads allowed to stay in flight are
            // page p+1's (every load instruction is issued, so counts are exact)
            if (p + 1 < p_hi) {
                if (kFp8) {
                    if (wave < 2) __builtin_amdgcn_s_waitcnt(VMCNT_IMM(10));
                    else __builtin_amdgcn_s_waitcnt(VMCNT_IMM(9));
                } else {
                    __builtin_amdgcn_s_waitcnt(VMCNT_IMM(kLoadsPerWave));
                }
            } else {
                __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
            }
            wg_barrier();

            const LDS_AS uint8_t* tile;
            if (kFp8) {
                convert_fp8_page(bufs[sb], tile_c, wave * 64 + opaque_lane());
                __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): LDS writes done
                wg_barrier();
                if (p + 2 < p_hi) issue(p + 2, bufs[sb]);
                tile = tile_c;
            } else {
                convert_bf16_tile(bufs[sb], wave * 64 + opaque_lane());
                __builtin_amdgcn_s_waitcnt(0xC07F);
                wg_barrier();
                tile = bufs[sb];
            }

            // inactive waves (rows beyond M) compute on row 0's query and
            // discard the result: keeping the call unconditional keeps the
            // accumulators out of control-flow merges
            compute_tile(tile, qf, st, min(max(n_vis - p * kPage, 0), kPage), scale_lane);

            if (!kFp8) {
                __builtin_amdgcn_s_waitcnt(0xC07F);       // this wave's LDS reads retired
                wg_barrier();
                if (p + 2 < p_hi) issue(p + 2, bufs[sb]);
            }
        }
        if (kFp8) {
            // the next segment (or exit) must not convert into the tile while
            // another wave still reads it
            __builtin_amdgcn_s_waitcnt(0xC07F);
            wg_barrier();
        }

        // epilogue: normalise and write final output or the split's partial
        if (active) {
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
