// Split-KV MLA decode of the fp8 latent cache with block-scaled fp8 matrix
// products for Q.K^T, on gfx950 (CDNA4).
//
// The cache row is the "DeepSeek-R1" record's engine constraint (2) format:
// e4m3 codes over every dimension (RoPE included), then one e8m0 scale per
// 32 codes.  gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies e4m3
// operands and applies one e8m0 scale per 32 consecutive k-elements of each
// row of A and of each column of B, in hardware, so the K operand is the
// raw cache bytes: no dequantisation on the Q.K^T side.  The query must then
// be in the same format; one e4m3 term is too coarse (its rounding error,
// multiplied by the cache's outliers, exceeds the fp8 tolerance), so each
// query row is carried as two terms q ~ q_hi + q_lo, each e4m3 codes with
// its own e8m0 scale per 32 (q_lo encodes the residual q - q_hi), and each
// k-step issues two scaled MFMAs.  The scores are exact fp32 sums of the
// two terms' products with the cache's values ("DeepSeek R1 Architecture &
// Deployment Guide", section 1.1: the absorbed query against the 576-element
// latent row).
//
// Mapping onto CDNA4 (one workgroup of 4 waves per CU, 160 KiB of LDS):
//  * A first kernel writes the two-term query rows into the workspace, each
//    term in the cache's own row format.
//  * Pages move HBM -> LDS raw (608-byte rows; 528 at the narrow latent
//    width, see Fp8Dims) with direct-to-LDS buffer loads, double buffered:
//    page p + 1 is fetched while tile p is computed.  With pages of 64
//    tokens or more the tile is the page's bytes in order (each load one
//    aligned KiB), up to a swap of chunk pairs that keeps row reads
//    conflict-free (lin_flip).  Gathered rows (the sparse decode) and tiles
//    made of several smaller pages use column blocks instead: a row is five
//    128-byte blocks (the last one also holds the first bytes of the next
//    row, which are not used), token t's 16-byte chunk c at tile_off(t, c).
//    Rows past the visible tokens are never fetched (the descriptor size
//    excludes them).
//  * Q.K^T: wave w owns query rows 32w .. 32w + 31; per 64-deep k-step and
//    32-token block one K fragment (32 bytes per lane from the raw page) and
//    its scale bytes feed two scaled MFMAs (q_hi, q_lo).  The latent part of
//    both query terms lives in VGPRs, the RoPE part in LDS.
//  * Meanwhile each wave dequantises the latent part (V) of its own 16
//    tokens of the page into an fp16 V tile (v_cvt_scalef32_pk_f16_fp8 with
//    the row's e8m0 scale of each 32 codes).
//  * Softmax and P.V as in the other quantised-cache kernel: row-split, the
//    S^T accumulator is the B operand of fp16 P.V MFMAs, lazy rescaling.
//  * Two workgroup barriers per tile: V tile complete, and page p + 1 landed
//    (tile p's raw page and V tile no longer read).
#include "decode_rowsplit.h"

namespace mla {
namespace {

constexpr int kMxColBlocks = 5;                         // 128-byte column blocks of a raw row in LDS
constexpr int kMxChunks = 8 * kMxColBlocks;             // 40 chunks of 16 bytes (a row and some spare)
constexpr int kMxRawBytes = kMxColBlocks * kPage * 128; // 40960: one raw page of 64 rows
constexpr int kMxQrBytes = 4096;                        // per wave: q_R fragments, 2 terms x 2 halves x 1 KiB
constexpr int kMxPiecesPerWave = 2 * kMxColBlocks;      // 10 pieces of 1 KiB: 16 tokens x 5 column blocks

// Shapes per latent width DC (values at DC = 512 / 448)
template <int DC>
struct MxShape {
    typedef Fp8Dims<DC> F;
    static constexpr int kVtBytes = kPage * DC * 2;                         // 65536 / 57344: the fp16 V tile
    static constexpr int kLds = 2 * kMxRawBytes + kVtBytes + 4 * kMxQrBytes;  // 163840 / 155648
    static constexpr int kSteps = F::kD / 64;            // 9 / 8 k-steps of 64 dims
    static constexpr int kQRegSteps = DC / 64;           // 8 / 7 k-steps (the latent part) whose Q fragments live in VGPRs
    static constexpr int kFrags = 2 * kSteps;            // K fragments per tile: (k-step, 32-token block)
    static constexpr int kVPieces = DC / 16 / 4;         // 8 / 7 V chunks of 16 codes per lane per tile
    static constexpr int kScaleChunk = F::kD / 16;       // 36 / 32: the chunk holding a row's first 16 scale bytes
    static constexpr bool kHiScales = F::kD / 32 > 16;   // scale bytes past the first 16 (D = 576: two)
    // the last column block's chunks past the row (fetched from inside the
    // row by the sparse gather, see dma_sparse): 38, 39 / 33 .. 39
    static constexpr int kRowChunks = (F::kRowBytes + 15) / 16;
    static constexpr int kSpareShift = kRowChunks == 38 ? 2 : 8;
    static_assert(kLds <= 163840, "a CU's LDS");
    static_assert(F::kRowBytes <= kMxChunks * 16 && F::kRowBytes > (kMxChunks - 8) * 16,
                  "five column blocks cover a row");
    static_assert(kRowChunks - kSpareShift >= 0 && kMxChunks - 1 - kSpareShift < kRowChunks,
                  "spare chunks map inside the row");
    static_assert(kScaleChunk * 16 == F::kD && (kHiScales || F::kD / 32 <= 16), "scales follow the codes");
};
static_assert(MxShape<kDc>::kLds == 163840, "the kernel takes all of a CU's LDS at 512 dims");

// Linear page layout (dense decode with pages of 64 tokens or more): the 64
// rows of a tile lie in LDS as they lie in memory, so every 1 KiB load is one
// aligned KiB of the page (eight whole 128-byte lines; 128-byte row pieces at
// a 608- or 528-byte stride straddle lines: on fp8_b64 they fetched 392.6 MB
// per decode against 359.1 MB now, and took 1.7x the L1 -> L2 requests; the
// decode is 4 % faster at 528-byte rows, as fast at 608).  Rows of r chunks
// of 16 bytes: chunk c of token t sits at chunk r t + (c ^ lin_flip(t, r)).
// A 128-bit read of 16 consecutive tokens (t0 = 0 mod 16) at one chunk is
// served in one pass over the 64 banks when the 16 chunk indices are
// distinct mod 16: with r = 33 (528-byte rows) r t = t mod 16 already is;
// with r = 38 (608-byte rows) r t = 6 t mod 16 repeats after 8 tokens (even
// residues only), and the flip moves tokens 8 .. 15 of each 16 to odd
// chunks.  The flip swaps the chunks of a pair (2j, 2j + 1) of one row,
// which lie in one KiB of the page since r t is even.  The flip is bit 3 of
// t for an even r, none for an odd r.
__device__ __forceinline__ int lin_flip(int t, int r) { return (t >> 3) & ~r & 1; }

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// two-term query quantisation
// ---------------------------------------------------------------------------

// The e8m0 exponent of a block with largest magnitude amax: the smallest e
// with amax / 2^(e - 127) <= 448 (the largest e4m3 value, Guide section 4),
// clamped to 0 .. 254.  amax = f * 2^x with f in [1, 2): 448 = 1.75 * 2^8,
// so e - 127 = x - 8, plus one when f > 1.75.
__device__ __forceinline__ int e8m0_of(float amax) {
    const uint32_t b = __builtin_bit_cast(uint32_t, amax);
    const int x = (int)((b >> 23) & 0xFF);
    if (!(amax > 0.f) || x == 0) return 0;      // zero, or below 2^-126: clamped to the smallest scale
    const int e = x - 8 + ((b & 0x7FFFFF) > 0x600000 ? 1 : 0);
    return min(max(e, 0), 254);
}

// 32 values -> 32 e4m3 codes at scale 2^(e - 127) (round to nearest even;
// |v| / 2^(e - 127) <= 448 by the choice of e, so nothing saturates)
__device__ __forceinline__ void encode32(const float (&v)[32], int e, uint32_t (&codes)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int w = 0;
        w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(v[4 * i + 0], 127 - e),
                                            __builtin_amdgcn_ldexpf(v[4 * i + 1], 127 - e), w, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(v[4 * i + 2], 127 - e),
                                            __builtin_amdgcn_ldexpf(v[4 * i + 3], 127 - e), w, true);
        codes[i] = (uint32_t)w;
    }
}

// One thread per (query row, 32-dim block): q_hi = the block in e4m3 with
// its e8m0 scale; q_lo = the residual q - q_hi (exact in fp32) encoded the
// same way.  Row r of qx holds q_hi's row (576 codes, 18 scales, padding)
// then q_lo's, in the cache's row format.
template <int DC>
__global__ __launch_bounds__(256) void quantize_q_mx_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ qx,
                                                             int64_t rows) {
    typedef Fp8Dims<DC> F;
    constexpr int kD = F::kD;
    constexpr int kGroups = kD / 32;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < rows * kGroups;
         gid += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = gid / kGroups;
        const int g = (int)(gid - row * kGroups);
        const uint16_t* src = q + row * kD + 32 * g;
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 w = *(const u32x4*)(src + 8 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __builtin_bit_cast(float, w[j] << 16);
                v[8 * i + 2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
            }
        }
        uint8_t* dst = qx + row * F::kQxRowBytes;
#pragma unroll
        for (int term = 0; term < 2; ++term) {
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
            const int e = e8m0_of(amax);
            uint32_t codes[8];
            encode32(v, e, codes);
            u32x4* out = (u32x4*)(dst + term * F::kRowBytes + 32 * g);
            out[0] = u32x4{codes[0], codes[1], codes[2], codes[3]};
            out[1] = u32x4{codes[4], codes[5], codes[6], codes[7]};
            dst[term * F::kRowBytes + kD + g] = (uint8_t)e;
            if (term == 0) {
                // the residual of each value: q - decode(code) * 2^(e - 127)
                static_for<0, 32>([&](auto i_c) {
                    constexpr int i = decltype(i_c)::value;
                    const float d = __builtin_amdgcn_cvt_f32_fp8((int)codes[i >> 2], i & 3);
                    v[i] -= __builtin_amdgcn_ldexpf(d, e - 127);
                });
            }
        }
    }
}

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------

// The per-lane e8m0 scale operand of the scaled MFMA for a row (a token of
// the page, or a query row) whose scale bytes 0..15 are `lo` and 16..19
// `hi`: k-step s of half h (lanes 32h ..) uses byte 2s + h (the 32-dim block
// its k-elements fall in); byte 2s + h lands in dword s / 4, byte s % 4, so
// that the MFMA's byte select is the same for every lane.
struct MxScales {
    uint32_t d[3];
};
__device__ __forceinline__ MxScales mx_scales(const u32x4& lo, uint32_t hi, int h) {
    const uint32_t sel = 0x06040200u + (h ? 0x01010101u : 0u);
    MxScales s;
    s.d[0] = __builtin_amdgcn_perm(lo[1], lo[0], sel);
    s.d[1] = __builtin_amdgcn_perm(lo[3], lo[2], sel);
    s.d[2] = __builtin_amdgcn_perm(hi, hi, sel);
    return s;
}

// acc += A B^T over 64 dims with A's and B's per-32 e8m0 scales (byte S of
// the scale dwords).  A: 32 rows x 64 e4m3, B: 32 columns x 64 e4m3, both
// in the MFMA's lane layout (lane l: row / column l % 32, k-elements
// 16 (l / 32) .. + 15 and 32 + 16 (l / 32) .. + 15).  Issued as asm so the
// accumulator stays in arch VGPRs (the 256 AGPRs hold O); kZero starts the
// chain from an inline zero.  Hazards the compiler cannot see: scale or
// operand VGPRs written by VALU need 2 wait states before this reads them
// (callers order that), and a VALU read of acc needs 19 after the last MFMA
// (mx_scores_ready).
template <int S, bool kZero>
__device__ __forceinline__ void mfma_mx(f32x16& acc, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb) {
    static_assert(S >= 0 && S < 4, "scale byte");
    if constexpr (kZero)
        asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[%5,%5,0] op_sel_hi:[%6,%6,0]"
                     : "=v"(acc)
                     : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(S & 1), "n"(S >> 1));
    else
        asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%5,0] op_sel_hi:[%6,%6,0]"
                     : "+v"(acc)
                     : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(S & 1), "n"(S >> 1));
}
// a 16-pass XDL result needs 19 wait states before a VALU read
__device__ __forceinline__ void mx_scores_ready(f32x16& s0, f32x16& s1) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
}

// The same 1 KiB direct-to-LDS load with a 64-bit address per lane (the
// sparse gather: every token row can sit anywhere in the cache).  No
// instruction offset: it would move the LDS destination as well.
__device__ __forceinline__ void dma16_gather(uint64_t addr, uint32_t dst) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(addr), "{m0}"(dst) : "memory");
}

// kSparse: the top-k decode ("DeepSeek-V3.2" record).  A unit (one query
// position of one sequence, n_h rows) attends to the rows its index list
// selects; tile p holds entries 64p .. 64p + 63, gathered row by row (wave w
// gathers tokens 16w .. 16w + 15).  The kernel turns the list into rows in
// its page pipeline: during tile p the entries of tile p + 3 are loaded;
// those of tile p + 2 become the tile's mask (a ballot of 0 <= t < the
// query's causal context) and, for each lane's two tokens, block-table
// loads; tile p + 1's rows (page * block + slot) feed its gathers.  The mask
// takes the place of the length mask.  Entries that do not take part are
// fetched from a row of zeros (codes and scales 0: their values are 0).
__device__ __attribute__((aligned(256))) uint8_t g_sparse_zero_row[kSparseZeroRowBytes] = {};

// kWin (sparse only): the caller has declared that the whole cache lies in
// the first kGatherWindow bytes from its base; rows are then gathered with
// 32-bit buffer offsets.
template <int DC, int PS, bool kSparse, bool kWin = false>
__global__ __launch_bounds__(kDecodeThreads, 1) void mla_decode_mx_kernel(DecodeArgs a) {
    typedef PageGeom<kSparse ? 16 : PS> Geom;
    typedef MxShape<DC> X;
    typedef Fp8Dims<DC> F;
    constexpr int kD = F::kD;
    constexpr int kRowBytes = F::kRowBytes;
    constexpr int kMxQRegSteps = X::kQRegSteps, kMxFrags = X::kFrags, kMxVPieces = X::kVPieces;
    constexpr int kMxScaleChunk = X::kScaleChunk;
    static_assert(kRowBytes <= kSparseZeroRowBytes, "the zero row covers a row");
    static_assert(Geom::kRangeTok % 16 == 0, "a wave's 16 tokens lie in one page");
    // the tile is one run of 64 rows of one page: the linear layout
    constexpr bool kLin = !kSparse && PS >= kPage;
    constexpr int kR = X::kRowChunks;       // chunks of 16 bytes per row (38 / 33)
    static_assert(kR * 16 == kRowBytes && kR * 1024 <= kMxRawBytes, "a linear page fits its buffer");
    static_assert(kR <= 4 * kMxPiecesPerWave, "the waves' loads cover a page");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[X::kLds];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
    int* sbuf = (int*)smem;                 // planner scratch; dead before the first page lands

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int worker, rg;
    block_role(a.num_workers, worker, rg);
    const int M = a.s_q * a.n_h;
    const int row0 = rg * kRowsPerGroup + wave * kRowsPerWave;
    const bool active = row0 < M;
    const int j_wave = (active ? row0 : M - 1) / a.n_h;
    const int j_last = min(rg * kRowsPerGroup + kRowsPerGroup - 1, M - 1) / a.n_h;

    const WorkerStart start = plan_worker(a, worker, rg == 0, sbuf, tid);
    if (start.b >= a.batch) return;
    const int64_t Q = start.quota;
    const int64_t w_lo = (int64_t)worker * Q, w_hi = w_lo + Q;

    LDS_AS uint8_t* const raws[2] = {lds, lds + kMxRawBytes};
    LDS_AS uint8_t* const vt = lds + 2 * kMxRawBytes;
    LDS_AS uint8_t* const qr = lds + 2 * kMxRawBytes + X::kVtBytes + wave * kMxQrBytes;
    const int lane0 = tid & 63;
    // first token (within a tile) of the page this wave loads from; the
    // wave loads and dequantises tokens 16w .. 16w + 15
    const int tok0 = Geom::tok0(wave);
    // direct-to-LDS source offset of this lane inside a piece: token i >> 3
    // of the piece's 8, the chunk whose swizzled slot is i & 7 (pieces of
    // odd token groups flip the slot's low bit: address ^ 16)
    const int dma_lane = (lane0 >> 3) * kRowBytes + (((lane0 & 7) ^ sw(lane0 >> 3)) << 4);
    // linear layout: load k of wave w is the page's KiB 4k + w; its lane l
    // writes chunk 64 (4k + w) + l = 256 k + lin_lane
    const int lin_lane = 64 * wave + lane0;
    const int lin16 = lin_lane << 4;
    // bit 4 + k: the chunk flip of that lane in load k, formed once (each
    // load then takes a shift, a bit select and an add instead of a
    // division by the row's chunk count)
    uint32_t lin_mask = 0;
    if constexpr (kLin && kR % 2 == 0) {
#pragma unroll
        for (int k = 0; 4 * k < kR; ++k)
            lin_mask |= (uint32_t)lin_flip((256 * k + lin_lane) / kR, kR) << (4 + k);
    }

    int64_t cost = start.cost;
    int slot_base = start.slot;
    for (int b = start.b; b < a.batch; ++b) {
        const int L = kSparse ? a.sparse_topk : ld_const(a.seq_lens + b);
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

        const int n_vis = L - a.s_q + 1 + j_wave;       // tokens this wave's rows see
        const int n_load = L - a.s_q + 1 + j_last;      // tokens the workgroup loads

        // block-table entries by vector loads, a tile ahead of their use: the
        // entry of the page holding token tok0 of tile p.  Entries the segment
        // cannot touch read 0; an entry past the sequence's last page may be
        // read but is not used (its rows are past n_load)
        const __amdgpu_buffer_rsrc_t bt = make_rsrc((const uint8_t*)(a.block_table + (int64_t)b * a.max_blocks),
                                                    (PS < kPage ? min(Geom::entries(p_hi), a.max_blocks)
                                                                : Geom::entries(p_hi)) * 4);
        auto load_phys = [&](int p) -> int {
            return __builtin_amdgcn_raw_buffer_load_b32(bt, Geom::entry(p, tok0) * 4, 0, 0);
        };
        // descriptor over the rows of tile p in the wave's page that the
        // workgroup loads (none past p_hi)
        auto page_rsrc = [&](int p, int phys) {
            const int rows = __builtin_amdgcn_readfirstlane(
                p < p_hi ? min(max(n_load - p * kPage - tok0, 0), Geom::kRangeTok) : 0);
            return make_rsrc(a.kv + (int64_t)__builtin_amdgcn_readfirstlane(phys) * a.page_bytes +
                                 Geom::row_in_page(p, tok0) * kRowBytes,
                             rows * kRowBytes);
        };
        // piece k of this wave: token group g = 2 wave + (k & 1) (tokens
        // 8g .. 8g + 7), column block k >> 1; it lands at g * 1024 of that
        // column block
        auto dma_piece = [&](__amdgpu_buffer_rsrc_t r, LDS_AS uint8_t* buf, auto k_c) {
            constexpr int k = decltype(k_c)::value, gl = k & 1, cb = k >> 1;
            const int g = 2 * wave + gl;
            const int off = (8 * g - tok0) * kRowBytes + cb * 128;
            int lane_off;
            if constexpr (kRowBytes % 32 == 0) {
                // the row part of dma_lane is a multiple of 32: bit 4 is the chunk's low bit
                lane_off = pinned(dma_lane) ^ (gl << 4);
            } else {
                // a 528-byte stride moves bit 4 with the token: flip the chunk's low
                // bit itself (+16 for an even chunk, -16 for an odd one)
                const int l = opaque_lane();
                const int flip = gl ? 16 - ((((l & 7) ^ sw(l >> 3)) & 1) << 5) : 0;
                lane_off = pinned(dma_lane) + flip;
            }
            dma16(r, lane_off + off, (uint32_t)(uintptr_t)(buf + cb * 8192 + g * 1024));
        };
        // linear layout: KiB i = 4k + w of the tile's rows (kR KiB in all);
        // LDS chunk n holds the page's chunk n ^ lin_flip(n / kR) (the flip
        // is an involution on a row's chunk pairs)
        auto dma_lin = [&](__amdgpu_buffer_rsrc_t r, LDS_AS uint8_t* buf, auto k_c) {
            constexpr int k = decltype(k_c)::value;
            if constexpr (4 * k < kR) {
                if (4 * k + 3 < kR || 4 * k + wave < kR) {
                    // (256 k + lin_lane) ^ flip, in bytes: the flip is bit 4
                    // of the byte offset, which 4096 k leaves clear.  Three
                    // instructions in one block (as separate expressions the
                    // compiler hoists each load's flip out of the page loop
                    // and spills it)
                    int off;
                    if constexpr (kR % 2 == 0)
                        asm volatile("v_lshrrev_b32 %0, %1, %2\n\tv_and_b32 %0, 16, %0\n\tv_xad_u32 %0, %0, %3, %4"
                                     : "=&v"(off)
                                     : "n"(k), "v"(lin_mask), "v"(lin16), "s"(4096 * k));
                    else
                        off = pinned(lin16) + 4096 * k;
                    dma16(r, off, (uint32_t)(uintptr_t)(buf + (4 * k + wave) * 1024));
                }
            }
        };
        auto dma_page = [&](__amdgpu_buffer_rsrc_t r, LDS_AS uint8_t* buf, auto k_c) {
            if constexpr (kLin) dma_lin(r, buf, k_c);
            else dma_piece(r, buf, k_c);
        };

        // sparse gather plan.  Unit b is query position j of sequence b_seq;
        // its entries read through r_idx (entry k of the list at 4k), the
        // block table of b_seq through r_bt.
        const int sq = kSparse ? a.sparse_sq : 1;
        const int b_seq = kSparse ? b / sq : b;
        const int n_ctx = kSparse ? ld_const(a.seq_lens + b_seq) - sq + 1 + (b - b_seq * sq) : 0;
        const __amdgpu_buffer_rsrc_t r_idx =
            make_rsrc((const uint8_t*)(a.sparse_indices + (kSparse ? (int64_t)b * L : 0)), kSparse ? L * 4 : 0);
        const __amdgpu_buffer_rsrc_t r_bt =
            make_rsrc((const uint8_t*)(a.block_table + (int64_t)b_seq * a.max_blocks), kSparse ? a.max_blocks * 4 : 0);
        const int pshift = __builtin_ctz((unsigned)a.page_size);
        // entry 64p + lane of the list (entries past topk are masked below)
        auto load_idx = [&](int p) -> int {
            return __builtin_amdgcn_raw_buffer_load_b32(r_idx, (p * kPage + pinned(lane0)) * 4, 0, 0);
        };
        // tile p's mask (bit t: entry 64p + t is a token of the query's
        // context) and, for this lane's two tokens 16w + x and 16w + 8 + x
        // (x = lane >> 3 of a piece), their block-table entries in flight and
        // their slots in the page (0xFFFF: no token)
        struct SparsePend {
            uint32_t e0, e1, slots;
        };
        auto expand = [&](int iv, int p, uint64_t& mask) -> SparsePend {
            const int l = pinned(lane0);
            const bool valid = p < p_hi && p * kPage + l < L && iv >= 0 && iv < n_ctx;
            const uint64_t m = __builtin_amdgcn_ballot_w64(valid);
            mask = m;
            const int s0 = wave * 16 + (l >> 3), s1 = s0 + 8;
            const int t0 = __shfl(iv, s0), t1 = __shfl(iv, s1);
            const bool v0 = (m >> s0) & 1, v1 = (m >> s1) & 1;
            SparsePend r;
            r.e0 = __builtin_amdgcn_raw_buffer_load_b32(r_bt, (v0 ? t0 >> pshift : 0) * 4, 0, 0);
            r.e1 = __builtin_amdgcn_raw_buffer_load_b32(r_bt, (v1 ? t1 >> pshift : 0) * 4, 0, 0);
            r.slots = (v0 ? (uint32_t)(t0 & (a.page_size - 1)) : 0xFFFFu) |
                      ((v1 ? (uint32_t)(t1 & (a.page_size - 1)) : 0xFFFFu) << 16);
            return r;
        };
        // the two tokens' cache rows (page * block + slot), kNoRow for none
        auto rows_of = [&](const SparsePend& q) -> u32x2 {
            const uint32_t s0 = q.slots & 0xFFFFu, s1 = q.slots >> 16;
            return u32x2{s0 == 0xFFFFu ? kNoRow : (q.e0 << pshift) + s0, s1 == 0xFFFFu ? kNoRow : (q.e1 << pshift) + s1};
        };
        // kWin: one buffer descriptor over the window and a 32-bit offset per
        // lane; an entry that does not take part -- or a row past the window,
        // should the caller's declaration be wrong -- gets an offset past the
        // window, which the range check turns into zeros.  Otherwise 64-bit
        // addresses; entries that do not take part read the row of zeros.
        const __amdgpu_buffer_rsrc_t r_win = make_rsrc(a.kv, (int)kGatherWindow);
        const uint8_t* const zero_row = g_sparse_zero_row;
        // piece k of tile p (row ids rw): token 16w + 8 (k & 1) + (i >> 3),
        // column block k >> 1, as dma_piece.  The last column block's chunks
        // past the row (never read: 38 and 39 of a 608-byte row, 33 .. 39 of
        // a 528-byte one) are fetched from chunks kSpareShift lower, inside
        // the row, so that no lane reads past its row.
        auto dma_sparse = [&](const u32x2& rw, int p, LDS_AS uint8_t* buf, auto k_c) {
            constexpr int k = decltype(k_c)::value, gl = k & 1, cb = k >> 1;
            const uint32_t row = rw[gl];
            const bool live = p < p_hi && row != kNoRow;
            const int l = pinned(lane0);
            int c = (l & 7) ^ sw(l >> 3) ^ gl;
            if constexpr (cb == kMxColBlocks - 1) c = 8 * cb + c >= X::kRowChunks ? c - X::kSpareShift : c;
            const int chunk = (cb * 8 + c) << 4;
            const uint32_t dst = (uint32_t)(uintptr_t)(buf + cb * 8192 + (2 * wave + gl) * 1024);
            if constexpr (kWin) {
                constexpr uint32_t kRowMax = (kGatherWindow - kRowBytes) / kRowBytes;
                const bool in = live && row <= kRowMax;
                dma16(r_win, (int)(in ? row * (uint32_t)kRowBytes + chunk : kGatherNone), dst);
            } else {
                const uint8_t* base = live ? a.kv + (uint64_t)row * kRowBytes : zero_row;
                dma16_gather((uint64_t)(base + chunk), dst);
            }
        };

        // segment prologue: the first block-table entries (sparse: the first
        // lists and their block-table entries), the first page as soon as
        // its entries land, then the queries
        int phys_next = 0;
        uint64_t mk_cur = ~0ull, mk_next = ~0ull;   // sparse: masks of tiles p and p + 1
        SparsePend pend;                            // sparse: tile p + 1's block-table entries in flight
        int iv = 0;                                 // sparse: the lane's entry of tile p + 2
        if constexpr (kSparse) {
            const int iv0 = load_idx(p_lo), iv1 = load_idx(p_lo + 1);
            iv = load_idx(p_lo + 2);
            const SparsePend pend0 = expand(iv0, p_lo, mk_cur);
            pend = expand(iv1, p_lo + 1, mk_next);
            const u32x2 rw0 = rows_of(pend0);
            static_for<0, kMxPiecesPerWave>([&](auto k) { dma_sparse(rw0, p_lo, raws[0], k); });
        } else {
            const int phys0 = load_phys(p_lo);
            phys_next = load_phys(p_lo + 1);
            const __amdgpu_buffer_rsrc_t r0 = page_rsrc(p_lo, phys0);
            static_for<0, kMxPiecesPerWave>([&](auto k) { dma_page(r0, raws[0], k); });
        }
        // this wave's 32 query rows, both terms, as MFMA B operands: lane i
        // holds row i & 31, chunks 4s + h and 4s + 2 + h (h = i >> 5) of
        // k-step s; the RoPE step (the last) goes to LDS
        i32x8 qf[2][kMxQRegSteps];
        MxScales qs[2];
        {
            const int h = lane0 >> 5;
            const int row = active ? row0 + (lane0 & 31) : row0;
            const uint8_t* qrow = (const uint8_t*)a.qx + ((int64_t)b * M + (active ? row : 0)) * F::kQxRowBytes;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int s = 0; s < kMxQRegSteps; ++s) {
                    const u32x4 c0 = *(const u32x4*)(qrow + t * kRowBytes + (4 * s + h) * 16);
                    const u32x4 c1 = *(const u32x4*)(qrow + t * kRowBytes + (4 * s + 2 + h) * 16);
                    qf[t][s] = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                                     (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
                }
                const u32x4 slo = *(const u32x4*)(qrow + t * kRowBytes + kD);
                const uint32_t shi = X::kHiScales ? *(const uint32_t*)(qrow + t * kRowBytes + kD + 16) : 0u;
                qs[t] = mx_scales(slo, shi, h);
                // the previous segment's last tile has retired its q_R reads (barrier)
                const u32x4 r0 = *(const u32x4*)(qrow + t * kRowBytes + (4 * kMxQRegSteps + h) * 16);
                const u32x4 r1 = *(const u32x4*)(qrow + t * kRowBytes + (4 * kMxQRegSteps + 2 + h) * 16);
                *(LDS_AS u32x4*)(qr + t * 2048 + lane0 * 16) = r0;
                *(LDS_AS u32x4*)(qr + t * 2048 + 1024 + lane0 * 16) = r1;
            }
        }
        WaveState<F::kMdBlocks> st;
        st.m = -__builtin_inff();
        st.l = 0.f;
        st.o_zero = true;
#pragma unroll
        for (int md = 0; md < F::kMdBlocks; ++md) st.o[md] = f32x16{};
        __builtin_amdgcn_s_waitcnt(VMCNT0_IMM);
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();

        for (int p = p_lo; p < p_hi; ++p) {
            const LDS_AS uint8_t* raw = raws[(p - p_lo) & 1];
            LDS_AS uint8_t* const rnext = raws[(p - p_lo + 1) & 1];
            __amdgpu_buffer_rsrc_t r_next;
            int phys_after = 0;
            u32x2 rw_next;
            uint64_t mk_after = ~0ull;
            if constexpr (kSparse) {
                // tile p + 1's rows (its block-table entries landed during
                // tile p - 1), tile p + 2's mask and entries, tile p + 3's list
                rw_next = rows_of(pend);
                pend = expand(iv, p + 2, mk_after);
                iv = load_idx(p + 3);
            } else {
                r_next = page_rsrc(p + 1, phys_next);
                phys_after = load_phys(p + 2);
            }
            const int n_valid = min(max(n_vis - p * kPage, 0), kPage);

            const int lane = opaque_lane();
            const int h = lane >> 5;
            // byte of (token t, chunk c) in the raw tile
            auto raw_off = [&](int t, int c) {
                if constexpr (kLin) return (kR * t + (c ^ lin_flip(t, kR))) << 4;
                else return tile_off(t, c);
            };
            // K fragment f = (k-step s = f >> 1, block f & 1): token 32 (f & 1) +
            // (lane & 31), chunks 4s + h and 4s + 2 + h.  Column blocks: chunk
            // 4s + h + 2c sits in column block s / 2 at slot (4 (s & 1) + 2c + h)
            // ^ sw(token): k_off[2 (s & 1) + c]; block 1's token is 32 further
            // (same sw).  Linear: the flip only touches the chunk's low bit (h),
            // so k_off[0] + 64 s + 32 c (block 1: + 32 rows, same flip).
            int k_off[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) k_off[j] = raw_off(lane & 31, 2 * j + h);
            auto read_k = [&](auto f_c) -> i32x8 {
                constexpr int f = decltype(f_c)::value, s = f >> 1, blk = f & 1;
                u32x4 c0, c1;
                if constexpr (kLin) {
                    const LDS_AS uint8_t* base = raw + k_off[0] + blk * 32 * kRowBytes + 64 * s;
                    c0 = *(const LDS_AS u32x4*)(base);
                    c1 = *(const LDS_AS u32x4*)(base + 32);
                } else {
                    const LDS_AS uint8_t* base = raw + (s >> 1) * 8192 + blk * 4096;
                    c0 = *(const LDS_AS u32x4*)(base + k_off[2 * (s & 1)]);
                    c1 = *(const LDS_AS u32x4*)(base + k_off[2 * (s & 1) + 1]);
                }
                return i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2],
                             (int)c1[3]};
            };
            // the scale bytes of the lane's two tokens (blocks 0 and 1)
            MxScales ks[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int t = 32 * blk + (lane & 31);
                const u32x4 slo = *(const LDS_AS u32x4*)(raw + raw_off(t, kMxScaleChunk));
                const uint32_t shi = X::kHiScales ? *(const LDS_AS uint32_t*)(raw + raw_off(t, kMxScaleChunk + 1)) : 0u;
                ks[blk] = mx_scales(slo, shi, h);
            }
            // V dequantisation: lane i of wave w converts token 16w +
            // store_token(i & 15), chunks c = 4k + (i >> 4) (codes 16c .. 16c + 15, scale byte c / 2)
            // into fp16 chunks 2c, 2c + 1 of the V tile
            const int v_tok = 16 * wave + store_token(lane & 15);
            const u32x4 v_sc = *(const LDS_AS u32x4*)(raw + raw_off(v_tok, kMxScaleChunk));
            const int v_src = raw_off(v_tok, lane >> 4);            // chunk 4k + (i >> 4) adds k * 4 chunks
            const int v_dst = tile_off(v_tok, 2 * (lane >> 4));
            u32x4 v_codes;
            auto v_read = [&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                if constexpr (kLin) {
                    // 4k chunks further in the row; the flip keeps to bit 0
                    v_codes = *(const LDS_AS u32x4*)(raw + v_src + 64 * k);
                } else {
                    // chunk 4k + j: column block k / 2, slot 4 (k & 1) + j (j = i >> 4)
                    v_codes = *(const LDS_AS u32x4*)(raw + (k >> 1) * 8192 + (v_src ^ ((4 * (k & 1)) << 4)));
                }
            };
            auto v_store = [&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                const uint32_t e = __builtin_amdgcn_ubfe(v_sc[k >> 1], (uint32_t)((k & 1) * 16 + ((lane >> 5) << 3)), 8);
                // 2^(e - 127) as fp32 bits e << 23 (e = 255, a NaN scale, also sets
                // the top mantissa bit; e = 0 gives 0, which every e4m3 value times
                // 2^-127 rounds to in fp16 anyway)
                const float scale = __builtin_bit_cast(float, (((e + 1) >> 8) << 22) | (e << 23));
                LDS_AS uint8_t* d = vt + k * 8192;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 hv;
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        hv[2 * qq + 0] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v_codes[2 * c + qq], scale, false));
                        hv[2 * qq + 1] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v_codes[2 * c + qq], scale, true));
                    }
                    *(LDS_AS u32x4*)(d + (v_dst ^ (c << 4))) = hv;
                }
            };

            // ---- S^T = K Q^T: fragment f = (k-step s = f >> 1, block f & 1),
            // two scaled MFMAs each (q_hi, q_lo).  Hooks: V dequantisation
            // (read at even fragments, convert and store at odd ones), the
            // pieces of page p + 1.
            f32x16 s0, s1;
            i32x8 kf[2];
            i32x8 qrf[2];          // the RoPE step's query fragments, read from LDS
            kf[0] = read_k(std::integral_constant<int, 0>{});
            static_for<0, kMxFrags>([&](auto f_c) {
                constexpr int f = decltype(f_c)::value, s = f >> 1, blk = f & 1;
                if constexpr (f + 1 < kMxFrags) kf[(f + 1) & 1] = read_k(std::integral_constant<int, f + 1>{});
                if constexpr (f == kMxFrags - 4) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const u32x4 c0 = *(const LDS_AS u32x4*)(qr + t * 2048 + lane0 * 16);
                        const u32x4 c1 = *(const LDS_AS u32x4*)(qr + t * 2048 + 1024 + lane0 * 16);
                        qrf[t] = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                                       (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
                    }
                }
                f32x16& acc = blk ? s1 : s0;
                if constexpr (f == 0) asm volatile("s_nop 4" ::: "memory");   // the scale VGPRs were just written
                if constexpr (s < kMxQRegSteps) {
                    mfma_mx<s % 4, s == 0>(acc, kf[f & 1], qf[0][s], ks[blk].d[s / 4], qs[0].d[s / 4]);
                    mfma_mx<s % 4, false>(acc, kf[f & 1], qf[1][s], ks[blk].d[s / 4], qs[1].d[s / 4]);
                } else {
                    mfma_mx<s % 4, false>(acc, kf[f & 1], qrf[0], ks[blk].d[s / 4], qs[0].d[s / 4]);
                    mfma_mx<s % 4, false>(acc, kf[f & 1], qrf[1], ks[blk].d[s / 4], qs[1].d[s / 4]);
                }
                if constexpr (f % 2 == 0 && f / 2 < kMxVPieces) v_read(std::integral_constant<int, f / 2>{});
                if constexpr (f % 2 == 1 && f / 2 < kMxVPieces) v_store(std::integral_constant<int, f / 2>{});
                if constexpr (f < kMxPiecesPerWave) {
                    if constexpr (kSparse) dma_sparse(rw_next, p + 1, rnext, std::integral_constant<int, f>{});
                    else dma_page(r_next, rnext, std::integral_constant<int, f>{});
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            mx_scores_ready(s0, s1);
            // the V tile is complete once every wave's stores have retired
            __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
            wg_barrier();

            softmax_pv<kSparse, F::kMdBlocks, true>(vt, st, s0, s1, n_valid, mk_cur, a.scale_log2, lane, [](auto) {});
            if constexpr (kSparse) {
                mk_cur = mk_next;
                mk_next = mk_after;
            } else {
                phys_next = phys_after;
            }
            // page p + 1 landed; tile p's raw page and the V tile are no longer read
            __builtin_amdgcn_s_waitcnt(VMCNT0_IMM);
            __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
            wg_barrier();
        }
        // the last tile fetched page p_hi through a zero-size descriptor:
        // nothing was read and its zeros are never used

        rowsplit_epilogue<F::kMdBlocks>(a, st, lds + wave * (kRowsPerWave * 1024), b, M, row0, slot, active);
        // the next segment's first page lands in these bytes
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();
    }
}

template <int DC>
hipError_t launch_quantize_q_mx_dc(const DecodeArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.batch * a.s_q * a.n_h;
    const int64_t threads = rows * (Fp8Dims<DC>::kD / 32);
    const int64_t blocks = std::min<int64_t>((threads + 255) / 256, (int64_t)1 << 20);
    hipLaunchKernelGGL(quantize_q_mx_kernel<DC>, dim3((unsigned)blocks), dim3(256), 0, stream, a.q, a.qx, rows);
    return hipGetLastError();
}

template <int DC>
hipError_t launch_decode_fp8_mx_dc(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                   hipEvent_t ev_stop) {
    const dim3 grid(a.num_workers * row_groups);
    switch (a.page_size) {
        case 16: return launch_with_events(mla_decode_mx_kernel<DC, 16, false>, grid, stream, ev_start, ev_stop, a);
        case 32: return launch_with_events(mla_decode_mx_kernel<DC, 32, false>, grid, stream, ev_start, ev_stop, a);
        case 64: return launch_with_events(mla_decode_mx_kernel<DC, 64, false>, grid, stream, ev_start, ev_stop, a);
        case 128: return launch_with_events(mla_decode_mx_kernel<DC, 128, false>, grid, stream, ev_start, ev_stop, a);
        case 256: return launch_with_events(mla_decode_mx_kernel<DC, 256, false>, grid, stream, ev_start, ev_stop, a);
        default: return hipErrorInvalidValue;
    }
}

template <int DC>
hipError_t launch_decode_fp8_mx_sparse_dc(const DecodeArgs& a, int row_groups, hipStream_t stream,
                                          hipEvent_t ev_start, hipEvent_t ev_stop, bool window) {
    // rows are gathered one by one: the page-block size enters only as a shift
    const dim3 grid(a.num_workers * row_groups);
    return window ? launch_with_events(mla_decode_mx_kernel<DC, 64, true, true>, grid, stream, ev_start, ev_stop, a)
                  : launch_with_events(mla_decode_mx_kernel<DC, 64, true, false>, grid, stream, ev_start, ev_stop, a);
}

}  // namespace

hipError_t launch_quantize_q_mx(const DecodeArgs& a, hipStream_t stream) {
    switch (a.d_c) {
        case kDc: return launch_quantize_q_mx_dc<kDc>(a, stream);
        case kDcNarrow: return launch_quantize_q_mx_dc<kDcNarrow>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_fp8_mx(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                hipEvent_t ev_stop) {
    switch (a.d_c) {
        case kDc: return launch_decode_fp8_mx_dc<kDc>(a, row_groups, stream, ev_start, ev_stop);
        case kDcNarrow: return launch_decode_fp8_mx_dc<kDcNarrow>(a, row_groups, stream, ev_start, ev_stop);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_fp8_mx_sparse(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                       hipEvent_t ev_stop, bool window) {
    switch (a.d_c) {
        case kDc: return launch_decode_fp8_mx_sparse_dc<kDc>(a, row_groups, stream, ev_start, ev_stop, window);
        case kDcNarrow:
            return launch_decode_fp8_mx_sparse_dc<kDcNarrow>(a, row_groups, stream, ev_start, ev_stop, window);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mla
