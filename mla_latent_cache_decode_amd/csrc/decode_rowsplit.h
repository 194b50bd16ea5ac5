// Row-split softmax and P.V shared by the quantised-cache decode kernels
// ("DeepSeek R1 Architecture & Deployment Guide", section 1.1: softmax of the
// scores over the context, then the softmax-weighted sum of the latent rows).
// Each wave owns 32 query rows and their O^T accumulator (MD blocks of 32
// dims x 32 rows: 512 dims, 256 AGPRs, or 448 for the fp8 cache's narrow
// row); its S^T scores (two 32-token blocks) are the B operand of P.V after
// the softmax, so no weights are exchanged between waves.
#pragma once

#include "decode_common.h"

namespace mla {
namespace {

constexpr int kPvSteps = 4 * kMdBlocks;         // 64 MFMA steps for P.V at 512 dims
// Lazy max with weights offset by 2^-8: the running max m of a row is raised
// only when a tile's max exceeds it by more than kRescaleTau (log2 units), and
// the fp16 weights are p = 2^(s - m - kPOffset) <= 2^(kRescaleTau - kPOffset)
// = 2^15, inside fp16.  The offset cancels in O / l and is added back to the
// LSE.  Without it the threshold could only be 15, and on the fp8 workload
// with its 1 % of x20 outliers 11 % of a wave's tiles rescaled its 256 O
// accumulators (fp8_b64 decode 185 -> 153 us with the rescale skipped); a
// threshold of 23 cuts the tiles that rescale about tenfold.  What the
// offset costs: weights under 2^-14 (s < m - 6) are fp16 subnormals and
// under 2^-25 (s < m - 17) zero.  A CPU model of this arithmetic against
// float64 (tests/test_softmax_weights_model.py, on the fp8 recipe's small
// workload) gives max |err| / RMS 1.0e-2 with and without the offset, and on
// twenty full-size fp8_b64 sequences up to 1.1e-2 with it and 9.5e-3
// without (the fp8 bound is 4e-2).  The row sum l adds
// the unrounded weights: summing the fp16-rounded ones instead is better
// without an offset but, with it, lets a row whose weights are mostly
// subnormal drift (up to 2.8e-2 on the same sequences).
constexpr float kRescaleTau = 23.0f;
constexpr float kPOffset = 8.0f;
constexpr int kPvAhead = 2;                     // V fragment prefetch distance (steps)
constexpr int kPMakeAt = 6;                     // P.V step (within a 16-step block) that builds the next P fragment

// per-wave state of the online softmax and the O accumulator (MD blocks of
// 32 dims)
template <int MD = kMdBlocks>
struct WaveState {
    f32x16 o[MD];            // O^T accumulator: dims x heads
    float m;                 // running max (log2 units, lane's head)
    float l;                 // partial sum of exp over this lane's half of the tokens
    bool o_zero;             // nothing accumulated yet (wave-uniform)
};

// Softmax of the tile's scores s0 (tokens 0..31) and s1 (tokens 32..63) in
// S^T MFMA layout, then O^T += V^T P^T with V^T read from the fp16 tile
// `vtile` (token t's 16-byte chunk c at tile_off(t, c)).  pv_hook(step) runs
// inside P.V step `step` (compile-time).  Tokens of the tile that take part:
// the first n_valid (dense), or the set bits of `mask` (sparse: bit t =
// token t).  Lazy rescaling: the running max is raised only when the tile's
// max exceeds it by more than kRescaleTau, and O is then rescaled in place.
// `lane` is the caller's opaque_lane(); kGroupRescale picks scale_acc16's form.
template <bool kSparse, int MD = kMdBlocks, bool kGroupRescale = false, typename PvHook>
__device__ __forceinline__ void softmax_pv(const LDS_AS uint8_t* vtile, WaveState<MD>& st, f32x16& s0, f32x16& s1,
                                           int n_valid, uint64_t mask, float scale_log2, int lane, PvHook&& pv_hook) {
    constexpr int kSteps = 4 * MD;              // P.V MFMA steps: 4 token blocks x MD dim blocks
    const int hi = lane >> 5;
    const LDS_AS uint8_t* tile = vtile;

    // The first P.V steps' V^T fragments are read before the softmax, so
    // that their LDS latency passes under it (the tile is complete: the
    // callers' barrier).
    // vp[m][e]: tokens 8e + tok (the swizzle sees bit 3 of the token, which
    // flips the low slot bit: address ^ 16), dims m*32 + dim; the step's
    // column block and 16-token block are added as immediate offsets
    const LDS_AS uint8_t* vp[2][2];
    {
        const int g = lane >> 4, li = lane & 15;
        const int tok = ((g >> 1) << 2) + (li >> 2);
        const int dim = ((g & 1) << 4) + ((li & 3) << 2);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int o = tile_off(tok, (m * 32 + dim) >> 3) + (dim & 7) * 2;
            vp[m][0] = tile + o;
            vp[m][1] = tile + (o ^ 16) + 8 * 128;
        }
    }
    constexpr int kVBufs = kPvAhead + 2;
    f16x8 vf[kVBufs];
    auto read_v = [&](auto step_c) -> f16x8 {
        constexpr int step = decltype(step_c)::value;
        constexpr int kb_ = step / MD, md = step % MD;
        constexpr int off = (md >> 1) * 8192 + kb_ * 16 * 128;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp[md & 1][0] + off));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp[md & 1][1] + off));
        return __builtin_bit_cast(f16x8, i16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    };
    static_for<0, kPvAhead>([&](auto i) { vf[decltype(i)::value] = read_v(i); });
    __builtin_amdgcn_sched_barrier(0);

    // ---- softmax.  Tokens >= n_valid (tail of the sequence / causal limit)
    // are masked: excluded from the max and given p = 0.  The token of
    // register r is c_r + 4*hi (+32 for s1); compare c_r with nv_lane.
    const int nv_lane = n_valid - (hi << 2);
    const uint64_t m_lane = mask >> (hi << 2);
    // does token c + 4 hi of the tile take part (c compile-time)
    auto vis = [&](int c) -> bool {
        if constexpr (kSparse) return (m_lane >> c) & 1;
        else return c < nv_lane;
    };
    float mx = -__builtin_inff();
    if (kSparse ? mask == ~0ull : n_valid >= kPage) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c_r = ((r >> 2) << 3) + (r & 3);
            mx = fmaxf(mx, vis(c_r) ? s0[r] : -__builtin_inff());
            mx = fmaxf(mx, vis(c_r + 32) ? s1[r] : -__builtin_inff());
        }
    }
    mx = pair_max(mx);
    const float mx2 = mx * scale_log2;
    const bool need = mx2 > st.m + kRescaleTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mx2 : st.m;
        if (!st.o_zero) {
            const float alpha = need ? fast_exp2(st.m - m_new) : 1.0f;
#pragma unroll
            for (int md = 0; md < MD; ++md) scale_acc16<kGroupRescale>(st.o[md], alpha);
            st.l *= alpha;
        }
        st.m = m_new;
    }
    // P fragment kb (tokens of S^T registers 8(kb&1) .. +7 of s0 / s1) in
    // fp16; fragment 0 now, the others inside the P.V loop, where their
    // exponentials issue between MFMAs
    const float neg_m = -(st.m + kPOffset);
    float lsum = 0.f;
    auto make_p = [&](auto kb_c) -> f16x8 {
        constexpr int kb = decltype(kb_c)::value;
        const f32x16& sv = kb < 2 ? s0 : s1;
        f16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r = (kb & 1) * 8 + e;
            const int c_r = ((r >> 2) << 3) + (r & 3) + (kb >= 2 ? 32 : 0);
            const float x = vis(c_r) ? fast_exp2(fmaf(sv[r], scale_log2, neg_m)) : 0.f;
            lsum += x;
            f[e] = (_Float16)x;
        }
        return f;
    };
    f16x8 pf[4];
    pf[0] = make_p(std::integral_constant<int, 0>{});

    // ---- O^T += V^T P^T.  Step s covers (kb = s / MD, md = s % MD); its V^T
    // fragment is two transposed reads (tokens kb*16 + e4*8 + tok_lane, dims
    // md*32 + dim_lane), issued kPvAhead steps ahead into rotating buffers.
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, kSteps>([&](auto step_c) {
        constexpr int step = decltype(step_c)::value;
        if constexpr (step + kPvAhead < kSteps)
            vf[(step + kPvAhead) % kVBufs] = read_v(std::integral_constant<int, step + kPvAhead>{});
        st.o[step % MD] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[step % kVBufs], pf[step / MD], st.o[step % MD],
                                                                  0, 0, 0);
        // VALU and memory work issues while the MFMA runs
        if constexpr ((step % MD) == kPMakeAt && (step / MD) < 3)
            pf[(step / MD) + 1] = make_p(std::integral_constant<int, (step / MD) + 1>{});
        pv_hook(step_c);
        __builtin_amdgcn_sched_barrier(0);
    });
    // keep the accumulator's home in AGPRs (it is only touched by MFMA in the
    // steady state); VALU users copy out and back
#pragma unroll
    for (int md = 0; md < MD; ++md) asm volatile("" : "+a"(st.o[md]));
    st.l += lsum;
    st.o_zero = false;
}

// Epilogue of a row-split wave: normalise O by the row sums and write the
// final fp32 output (a sequence one worker serves whole) or the split's fp16
// partial and its LSE.  A partial row (1 KiB) goes through `stage`, 32 KiB of
// LDS that is idle after the last tile's barrier: each wave stages its own
// 32 rows, 8-byte slot s of row r at slot s ^ (r & 31) (the rows of one store
// pass hit distinct banks), then stores whole rows, one 1 KiB store each;
// stored directly, every instruction scatters 16 bytes over 32 rows
// (fp8_b64: 199.9 -> 191.0 us per decode with the staging).  Callers place a
// workgroup barrier before the staged bytes are reused.
template <int MD = kMdBlocks>
__device__ __forceinline__ void rowsplit_epilogue(const DecodeArgs& a, const WaveState<MD>& st, LDS_AS uint8_t* stage,
                                                  int b, int M, int row0, int slot, bool active) {
    constexpr int DC = 32 * MD;                 // dims of an output row
    if (!active) return;
    const int lane = opaque_lane();
    const float l_tot = pair_sum(st.l);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (st.m + kPOffset + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                    : -__builtin_inff();
    const int row = row0 + (lane & 31);
    const int hi = lane >> 5;
    if (slot < 0) {
        float* dst = a.out + ((int64_t)b * M + row) * DC + hi * 4;
#pragma unroll
        for (int md = 0; md < MD; ++md) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 v = {st.o[md][r4 * 4 + 0] * inv, st.o[md][r4 * 4 + 1] * inv, st.o[md][r4 * 4 + 2] * inv,
                                 st.o[md][r4 * 4 + 3] * inv};
                *(f32x4*)(dst + md * 32 + r4 * 8) = v;
            }
        }
        if (lane < 32 && a.lse) a.lse[(int64_t)b * M + row] = lse_v;
        return;
    }
    const int r = lane & 31;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f16x4 h = {(_Float16)(st.o[md][r4 * 4 + 0] * inv), (_Float16)(st.o[md][r4 * 4 + 1] * inv),
                             (_Float16)(st.o[md][r4 * 4 + 2] * inv), (_Float16)(st.o[md][r4 * 4 + 3] * inv)};
            const int s = md * 8 + r4 * 2 + hi;       // 8-byte slot: dims 4s .. 4s + 3
            *(LDS_AS u32x2*)(stage + r * 1024 + ((s ^ r) << 3)) = __builtin_bit_cast(u32x2, h);
        }
    }
    if (lane < 32) a.plan.part_lse[(int64_t)row * a.plan.slots + slot] = lse_v;
    __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
    // row j of this wave: lane l stores logical slots 2l, 2l + 1 (lanes
    // past the row's DC / 8 have nothing to store)
    if (4 * MD < 64 && lane >= 4 * MD) return;
    uint16_t* const pbase = a.plan.part_o + ((int64_t)slot * M + row0) * DC + lane * 8;
    for (int j = 0; j < kRowsPerWave; ++j) {
        u32x4 v = *(const LDS_AS u32x4*)(stage + j * 1024 + (((2 * lane) ^ (j & 30)) << 3));
        if (j & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        *(u32x4*)(pbase + j * DC) = v;
    }
}

}  // namespace
}  // namespace mla
