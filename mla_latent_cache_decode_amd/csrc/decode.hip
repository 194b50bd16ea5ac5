// Split-KV MLA decode for an fp4 latent cache (e2m1 codes + one e8m0 scale
// per 16) on gfx950 (CDNA4).
//
// What one workgroup computes ("DeepSeek R1 Architecture & Deployment Guide",
// section 1.1): for 128 query rows (heads of one or more query positions) and
// a contiguous range of cache pages of one sequence,
//     S = K Q^T      over the 576-element shared row (latent c, then RoPE k_R),
//     online softmax of S over the tokens,
//     O = V^T P^T    with V = the first 512 elements (the latent c) of the
//                    same rows (the value up-projection is absorbed into the
//                    output projection downstream).
// A split's partial result (O / l, lse) goes to the workspace for the LSE
// combine; a sequence served by one worker is finished here directly.  The
// row format (two e2m1 codes per byte over every dimension, RoPE included,
// then one e8m0 scale per 16 values) is this build's reading of the
// "DeepSeek-R1" record's 288-byte fp4 variant in its engine constraint (2).
//
// Mapping onto CDNA4 (one workgroup of 4 waves per CU):
//  * 4 waves x 32 rows.  Each wave holds its 32 query rows as fp16 MFMA
//    B-operands (q_abs in VGPRs, q_R in LDS) and its O^T accumulator (512 x
//    32 fp32, 256 AGPRs).  Heads are the MFMA N dimension in both products,
//    so a head's softmax statistics live in one lane pair (l, l^32) and the
//    S^T accumulator is directly the B-operand of the PV product.
//  * One 64-token page is one tile.  Page p + 1 streams through VGPRs while
//    tile p is computed: buffer loads of codes and their scale bytes,
//    dequantised in registers (v_cvt_scalef32_pk_f16_fp4) and stored into
//    the idle fp16 LDS tile by hooks placed between the MFMA steps; one
//    barrier per tile.  Rows past the visible tokens are never fetched (the
//    descriptor size excludes them; the tile receives zeros).
//  * LDS tile layout: 9 column blocks of 64 dims; within a block, token t's
//    16-byte chunk c sits at slot t*8 + (c ^ sw(t)), conflict-free for the
//    row-wise Q.K^T reads, the dequantised stores and the transposed PV
//    reads (ds_read_b64_tr_b16).
//  * Both products run as fp16 MFMA with fp32 accumulation; queries are
//    prescaled per head by a power of two into [2^14, 2^15) before the fp16
//    conversion (exact) and the factor is folded into the softmax scale.
//  * Lazy rescaling: the running max m is only raised when a tile's max
//    exceeds it by more than 23 (log2 units), so O is rarely rescaled after
//    the first tile; the weights 2^(s - m - 8) stay <= 2^15, inside fp16.
#include "decode_rowsplit.h"

namespace mla {
namespace {

constexpr int kQkAhead = 2;                     // K fragment prefetch distance (k-steps)

constexpr int kLdsTiles = 2 * kTileBytes;       // 147456: two fp16 tiles
constexpr int kQRegSteps = kDc / 16;            // 32 k-steps (q_abs) whose Q fragments live in VGPRs
constexpr int kQLdsSteps = kKSteps - kQRegSteps; // 4 k-steps (q_R) whose fragments live in LDS
constexpr int kQLdsBytes = 4 * kQLdsSteps * 1024;  // 16384: 4 waves x 4 fragments x 64 lanes x 16 B
constexpr int kLdsBytes = kLdsTiles + kQLdsBytes;  // 163840 = all of a CU's LDS

// ---------------------------------------------------------------------------
// page pieces: HBM -> VGPRs -> dequantise -> fp16 LDS tile
// ---------------------------------------------------------------------------
//
// A page is moved by the four waves in pieces of one vector load per lane
// (16 fp4 values, plus their scale byte).  A piece is issued into registers well ahead of its use and
// stored into the tile that the next tile step reads; both halves of the
// work are spread over the MFMA steps of the current tile, so the memory
// path, the conversion and the matrix cores overlap.
//
// Every piece load goes through one buffer descriptor per page whose size
// is n_valid rows: lanes whose row lies past the visible tokens read zeros
// (the rows are never fetched) and the tile receives finite zeros.  The
// whole offset of a lane is in the VGPR offset, so the range check sees it.

// fp4 rows (D/2 bytes of e2m1 codes, element 2i in the low nibble of byte i,
// then one e8m0 scale per 16 values, 16-byte stride).  Wave w moves tokens
// 16w .. 16w + 15 in pieces k < 9: lane i carries one of them (see the
// constructor), the 16 values of group
// j = 4k + (i >> 4) -- 8 code bytes -- and their own scale byte j; they
// dequantise to tile chunks 2j and 2j + 1 of that token.
struct Fp4Pieces {
    static constexpr int kPieces = 9;
    static constexpr int kBatches = 3;
    static constexpr int kStage = 3;
    __device__ static constexpr int first(int b) { return 3 * b; }
    static constexpr int kHookPv[3] = {0, 0, 1};
    static constexpr int kHookAt[3] = {2, 22, 12};
    static constexpr int kHookStride[3] = {5, 5, 10};
    struct Stage {
        u32x2 codes;
        uint32_t scale;
    };
    // the fp4 scales travel with each piece
    struct PageScales {};

    int src_lane;       // (token - tok0) * 336 + 8 * (i >> 4), inside the wave's page
    int dst_lane;       // tile_off(token, 2 * (i >> 4)) without the column block
    __amdgpu_buffer_rsrc_t win;   // the declared cache window (sparse gather)

    // spread: lane i carries token 16w + store_token(i & 15) (conflict-free
    // tile stores); the sparse gather keeps token 16w + (i & 15), whose row
    // address the lane swaps deliver
    __device__ __forceinline__ Fp4Pieces(int lane, int wave, int tok0, __amdgpu_buffer_rsrc_t w, bool spread) : win(w) {
        const int t = wave * 16 + (spread ? store_token(lane & 15) : (lane & 15));
        src_lane = (t - tok0) * kFp4RowBytes + ((lane >> 4) << 3);
        dst_lane = tile_off(t, 2 * (lane >> 4));
    }
    __device__ __forceinline__ void issue(Stage& s, __amdgpu_buffer_rsrc_t r, int, int k) const {
        s.codes = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, pinned(src_lane) + k * 32, 0, 0));
        const int l = opaque_lane();
        const int scl = pinned(src_lane) - ((l >> 4) << 3) + kD / 2 + (l >> 4);
        s.scale = __builtin_amdgcn_raw_buffer_load_b8(r, scl + k * 4, 0, 0);
    }
    // sparse gather: the lane's token row starts at `row`
    __device__ __forceinline__ void issue(Stage& s, const uint8_t* row, int, int k) const {
        const int l = opaque_lane();
        s.codes = *(const u32x2*)(row + ((l >> 4) << 3) + k * 32);
        s.scale = row[kD / 2 + (l >> 4) + k * 4];
    }
    __device__ __forceinline__ void issue(Stage& s, uint32_t row, int, int k) const {
        const int l = opaque_lane();
        s.codes = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(win, (int)(row + ((l >> 4) << 3) + k * 32), 0, 0));
        s.scale = __builtin_amdgcn_raw_buffer_load_b8(win, (int)(row + kD / 2 + (l >> 4) + k * 4), 0, 0);
    }
    __device__ __forceinline__ void load_scales(PageScales&, __amdgpu_buffer_rsrc_t) const {}
    __device__ __forceinline__ void load_scales(PageScales&, const uint8_t*) const {}
    __device__ __forceinline__ void load_scales(PageScales&, uint32_t) const {}
    __device__ __forceinline__ void store(const Stage& s, const PageScales&, LDS_AS uint8_t* tile, int, int k) const {
        // the e8m0 scale as fp32 bits e << 23; e = 255 (NaN) also sets the top
        // mantissa bit, making a quiet NaN; e = 0 gives 0 rather than 2^-127,
        // which every e2m1 value times 2^-127 rounds to in fp16 anyway
        const uint32_t e = s.scale & 0xFF;
        const float scale = __builtin_bit_cast(float, (((e + 1) >> 8) << 22) | (e << 23));
        LDS_AS uint8_t* d = tile + k * 8192;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // 8 codes: byte b holds elements 2b (low nibble) and 2b + 1
            const u32x4 h = {
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.codes[c], scale, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.codes[c], scale, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.codes[c], scale, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(s.codes[c], scale, 3))};
            *(LDS_AS u32x4*)(d + (dst_lane ^ (c << 4))) = h;
        }
    }
};

// ---------------------------------------------------------------------------
// per-tile compute of one wave: 32 heads x 64 tokens
// ---------------------------------------------------------------------------
// One tile step of one wave: Q.K^T on the fp16 tile, then the shared
// softmax and P.V.  qk_hook(ks) runs inside Q.K^T step ks and pv_hook(step)
// inside P.V step `step` (both compile-time); they carry the page
// pipeline's loads and LDS stores so that these issue between MFMAs.
template <bool kSparse, typename QkHook, typename PvHook>
__device__ __forceinline__ void compute_tile(const LDS_AS uint8_t* tile, const f16x8 (&qf)[kQRegSteps],
                                             const LDS_AS uint8_t* qr, WaveState<>& st, int n_valid, uint64_t mask,
                                             float scale_log2, QkHook&& qk_hook, PvHook&& pv_hook) {
    const int lane = opaque_lane();
    const int hi = lane >> 5;

    // ---- S^T = K Q^T : two 32-token blocks (two independent MFMA chains).
    // Fragment of k-step ks: token (lane & 31) [+32], chunk 2*ks + hi, i.e.
    // tile_off(lane & 31, 2*(ks & 3) + hi) + (ks >> 2) * 8192 [+ 4096].
    int k_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) k_off[k] = tile_off(lane & 31, 2 * k + hi);
    f32x16 s0 = {}, s1 = {};
    f16x8 kf[kQkAhead + 1][3];      // [2]: the q_R fragment of the last k-steps
    auto read_k = [&](auto ks_c, f16x8 (&dst)[3]) {
        constexpr int ks = decltype(ks_c)::value;
        const LDS_AS uint8_t* base = tile + k_off[ks & 3] + (ks >> 2) * 8192;
        dst[0] = *(const LDS_AS f16x8*)(base);
        dst[1] = *(const LDS_AS f16x8*)(base + 4096);
        if constexpr (ks >= kQRegSteps) dst[2] = *(const LDS_AS f16x8*)(qr + (ks - kQRegSteps) * 1024);
    };
    static_for<0, kQkAhead>([&](auto i) { read_k(i, kf[decltype(i)::value]); });
    static_for<0, kKSteps>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        if constexpr (ks + kQkAhead < kKSteps)
            read_k(std::integral_constant<int, ks + kQkAhead>{}, kf[(ks + kQkAhead) % (kQkAhead + 1)]);
        f16x8 qb;
        if constexpr (ks < kQRegSteps) qb = qf[ks];
        else qb = kf[ks % (kQkAhead + 1)][2];
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks % (kQkAhead + 1)][0], qb, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks % (kQkAhead + 1)][1], qb, s1, 0, 0, 0);
        // the hook's VALU and memory work issues while the two MFMAs run
        qk_hook(ks_c);
        __builtin_amdgcn_sched_barrier(0);
    });
    // the scores feed VALU work (softmax): keep them in arch VGPRs
    asm volatile("" : "+v"(s0), "+v"(s1));
    softmax_pv<kSparse>(tile, st, s0, s1, n_valid, mask, scale_log2, lane, pv_hook);
}

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------
// kSparse: the top-k decode ("DeepSeek-V3.2" record): a unit (one query
// position, n_h rows) attends to the rows its index list selects, 64
// entries a tile.  Lane l loads entry l of the tile; a ballot of its
// validity (0 <= t < the query's causal context) gives the mask that takes
// the place of the length mask, and lane l of wave w gathers the row of
// entry 16w + (l & 15), moved to it by two lane swaps (entries that do not
// take part read a row of zeros).  The list is turned into rows in the
// page pipeline: during tile p the entries of tile p + 4 are loaded and
// those of tile p + 3 (loaded a tile earlier) issue their block-table
// loads, whose results give tile p + 3's rows one tile later.
__device__ __attribute__((aligned(256))) uint8_t g_sparse_zero_row[kSparseZeroRowBytes] = {};

// kWin (sparse only): the caller has declared that the whole cache lies in
// the first kGatherWindow bytes from its base; rows are then gathered with
// 32-bit buffer offsets.
template <int PS, bool kSparse, bool kWin = false>
__global__ __launch_bounds__(kDecodeThreads, 1) void mla_decode_kernel(DecodeArgs a) {
    typedef Fp4Pieces Pieces;
    typedef PageGeom<PS> Geom;
    constexpr int kPieces = Pieces::kPieces;
    constexpr int kRowBytes = kFp4RowBytes;
    static_assert(Geom::kRangeTok % 16 == 0, "a wave's 16 tokens lie in one page");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
    int* sbuf = (int*)smem;                 // planner scratch; dead before the first tile store

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.num_workers;
    int worker, rg;
    block_role(G, worker, rg);
    const int M = a.s_q * a.n_h;
    const int row0 = rg * kRowsPerGroup + wave * kRowsPerWave;
    const bool active = row0 < M;
    const int j_wave = (active ? row0 : M - 1) / a.n_h;
    const int j_last = min(rg * kRowsPerGroup + kRowsPerGroup - 1, M - 1) / a.n_h;

    const WorkerStart start = plan_worker(a, worker, rg == 0, sbuf, tid);
    if (start.b >= a.batch) return;
    const int64_t Q = start.quota;
    const int64_t w_lo = (int64_t)worker * Q, w_hi = w_lo + Q;

    LDS_AS uint8_t* const tiles[2] = {lds, lds + kTileBytes};
    // first token (within a tile) of the page this wave loads from
    const int tok0 = Geom::tok0(wave);
    // this wave's q_R fragments, lane-major: fragment f of lane l at f*1024 + l*16
    LDS_AS uint8_t* const qr_lds = lds + kLdsTiles + wave * (kQLdsSteps * 1024) + (tid & 63) * 16;

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

        const int n_vis = L - a.s_q + 1 + j_wave;           // tokens this wave may see
        const int n_load = L - a.s_q + 1 + j_last;          // tokens the workgroup loads

        // Block-table entries are read with vector loads (ordered with the
        // page loads on vmcnt; a scalar load would share lgkmcnt with the
        // LDS traffic and make every LDS wait a full drain).  Entries of
        // pages at or past p_hi read 0 and are not used.
        // The entry read for tile p is that of the page holding token tok0
        // of the tile (the wave's page); an entry past the sequence's last
        // page may be read but is not used (its rows are past n_load).
        // sparse: unit b is query position j of sequence b_seq, whose block
        // table bt covers; its causal context is n_ctx tokens
        const int sq = kSparse ? a.sparse_sq : 1;
        const int b_seq = b / sq;
        const int n_ctx = kSparse ? ld_const(a.seq_lens + b_seq) - sq + 1 + (b - b_seq * sq) : 0;
        const __amdgpu_buffer_rsrc_t bt =
            kSparse ? make_rsrc((const uint8_t*)(a.block_table + (int64_t)b_seq * a.max_blocks), a.max_blocks * 4)
                    : make_rsrc((const uint8_t*)(a.block_table + (int64_t)b * a.max_blocks),
                                (PS < kPage ? min(Geom::entries(p_hi), a.max_blocks) : Geom::entries(p_hi)) * 4);
        // dense: the block-table entry of tile p's page for this wave
        auto load_phys = [&](int p) -> int {
            return __builtin_amdgcn_raw_buffer_load_b32(bt, Geom::entry(p, tok0) * 4, 0, 0);
        };
        // sparse: entry l of tile p's list for lane l (entries past topk
        // read 0 and are masked)
        const __amdgpu_buffer_rsrc_t r_idx =
            make_rsrc((const uint8_t*)(a.sparse_indices + (kSparse ? (int64_t)b * L : 0)), kSparse ? L * 4 : 0);
        const int e_tok = wave * 16 + (tid & 15);
        const int pshift = __builtin_ctz((unsigned)a.page_size);
        auto load_idx = [&](int p) -> int {
            return __builtin_amdgcn_raw_buffer_load_b32(r_idx, (p * kPage + pinned(tid & 63)) * 4, 0, 0);
        };
        auto takes_part = [&](int p, int e, int t) { return p < p_hi && p * kPage + e < L && t >= 0 && t < n_ctx; };
        // x of lane 16 * wave + (l & 15), for every lane l: permlane16_swap
        // of x with itself yields rows (0, 0, 2, 2) and (1, 1, 3, 3) of x,
        // permlane32_swap of a value with itself its lower and its upper half
        // in both halves
        auto quarter_bcast = [&](int x) -> int {
            const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
            const unsigned y = (wave & 1) ? r16[1] : r16[0];
            const auto r32 = __builtin_amdgcn_permlane32_swap(y, y, false, false);
            return (int)((wave & 2) ? r32[1] : r32[0]);
        };
        // sparse: tile p's entries (lane l: entry l) -> the tile's mask, and
        // the lane's token's block-table entry in flight and its slot in the
        // page (-1: no token)
        struct SparsePend {
            int e, slot;
        };
        auto expand = [&](int p, int iv, uint64_t& mask) -> SparsePend {
            mask = __builtin_amdgcn_ballot_w64(takes_part(p, tid & 63, iv));
            const int t = quarter_bcast(iv);
            const bool v = takes_part(p, e_tok, t);
            SparsePend r;
            r.e = __builtin_amdgcn_raw_buffer_load_b32(bt, (v ? t >> pshift : 0) * 4, 0, 0);
            r.slot = v ? t & (a.page_size - 1) : -1;
            return r;
        };
        // sparse: the row id (page * block + slot) of a landed entry
        auto row_of = [&](const SparsePend& q) -> int {
            return q.slot < 0 ? (int)kNoRow : (q.e << pshift) + q.slot;
        };
        // dense: descriptor over the rows of tile p in the wave's page
        // (physical page phys) that the workgroup loads, size 0 past p_hi;
        // sparse: the lane's row (row id phys), or the zero row
        auto page_rsrc = [&](int p, int phys) {
            if constexpr (kSparse && kWin) {
                // the row's byte offset in the window; kGatherWindow (past it,
                // and past it still after a piece's offset is added) reads zeros
                constexpr uint32_t kRowMax = (kGatherWindow - kRowBytes) / kRowBytes;
                const bool live = p < p_hi && (uint32_t)phys != kNoRow && (uint32_t)phys <= kRowMax;
                return live ? (uint32_t)phys * (uint32_t)kRowBytes : kGatherWindow;
            } else if constexpr (kSparse) {
                const bool live = p < p_hi && (uint32_t)phys != kNoRow;
                return live ? a.kv + (uint64_t)(uint32_t)phys * kRowBytes : (const uint8_t*)g_sparse_zero_row;
            } else {
                const int nv = p < p_hi ? min(max(n_load - p * kPage - tok0, 0), Geom::kRangeTok) : 0;
                return make_rsrc(a.kv + (int64_t)__builtin_amdgcn_readfirstlane(phys) * a.page_bytes +
                                     Geom::row_in_page(p, tok0) * kRowBytes,
                                 nv * kRowBytes);
            }
        };
        typedef decltype(page_rsrc(0, 0)) Src;

        // this wave's 32 query rows as MFMA B operands (q_abs || q_R): bf16
        // loaded, scaled per head by 2^-sh so the head's max |q| lands in
        // [2^14, 2^15), converted to fp16 (exact up to fp16 subnormals); the
        // head's softmax scale absorbs 2^sh
        f16x8 qf[kKSteps];      // the q_R part moves to LDS after the conversion
        float scale_lane;
        WaveState<> st;
        const int lane0 = tid & 63;
        // segment prologue, ordered for overlap: the first block-table
        // entries, then the first page as soon as its entry lands, then the
        // queries; the page is stored while the queries are still arriving
        // (loads complete in issue order), and the queries are converted after
        int phys0, phys1;
        SparsePend pend;        // sparse: tile p + 2's rows in flight (tile p_lo + 2 in the prologue)
        int iv_next = 0;        // sparse: the lane's entry of tile p + 3
        // sparse: masks of tiles p .. p + 3 (wave-uniform)
        uint64_t mask_cur = ~0ull, mask1 = 0, mask2 = 0, mask3 = 0;
        if constexpr (kSparse) {
            const int iv0 = load_idx(p_lo), iv1 = load_idx(p_lo + 1), iv2 = load_idx(p_lo + 2);
            iv_next = load_idx(p_lo + 3);
            const SparsePend pend0 = expand(p_lo, iv0, mask_cur);
            const SparsePend pend1 = expand(p_lo + 1, iv1, mask1);
            pend = expand(p_lo + 2, iv2, mask2);
            phys0 = row_of(pend0);
            phys1 = row_of(pend1);
        } else {
            phys0 = load_phys(p_lo);
            phys1 = load_phys(p_lo + 1);
        }

        // scale each head's query by 2^-sh so its max |q| lands in [2^14, 2^15)
        // and convert to fp16 (exact up to fp16 subnormals); the q_R part
        // moves to LDS
        auto convert_q = [&]() {
            float qmax = 0.f;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                const bf16x8 qb = __builtin_bit_cast(bf16x8, qf[ks]);
#pragma unroll
                for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf((float)qb[e]));
            }
            qmax = pair_max(qmax);
            // exponent of qmax (the bf16 widening keeps fp32's exponent range;
            // a bf16 subnormal reads as exponent -127, zero is taken as 14).
            // sh >= -100 keeps both factors normal floats: a head whose max
            // |q| lies below 2^-86 is scaled by 2^100 only, and its scores,
            // below 2^-60 in magnitude, give a flat softmax either way
            const int ex = qmax > 0.f ? (int)((__builtin_bit_cast(uint32_t, qmax) >> 23) & 0xFF) - 127 : 14;
            const int sh = max(ex - 14, -100);
            const float down = __builtin_bit_cast(float, (uint32_t)(127 - sh) << 23);   // 2^-sh
            const float up = __builtin_bit_cast(float, (uint32_t)(127 + sh) << 23);     // 2^sh
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                const bf16x8 qb = __builtin_bit_cast(bf16x8, qf[ks]);
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[ks][e] = (_Float16)((float)qb[e] * down);
            }
            scale_lane = a.scale_log2 * up;
            // the previous segment's last tile has retired its q_R reads (barrier)
#pragma unroll
            for (int ks = kQRegSteps; ks < kKSteps; ++ks)
                *(LDS_AS f16x8*)(qr_lds + (ks - kQRegSteps) * 1024) = qf[ks];
        };
        const f16x8(&qreg)[kQRegSteps] = *reinterpret_cast<const f16x8(*)[kQRegSteps]>(&qf[0]);
        const Pieces pc(opaque_lane(), wave, tok0, make_rsrc(a.kv, kWin ? (int)kGatherWindow : 0), !kSparse);

        // ---- Page pipeline, one barrier per tile.  Pieces stream through
        // VGPRs (converted or dequantised in registers) into the idle
        // tile: page p + 1 moves during tile p in three or four batches
        // through one set of staging registers; each hook stores a batch
        // (the first was issued during the previous tile) and issues the
        // next; the last hook issues batch 0 of page p + 2.  Block-table
        // entries are loaded a tile before their use.
        typedef typename Pieces::Stage Stage;
        constexpr int kNB = Pieces::kBatches;
        constexpr int kS = Pieces::kStage;
        static_assert(Pieces::first(kNB) == kPieces, "batches cover the page");
        // the last hook issues page p + 2, whose descriptor exists after Q.K^T
        static_assert(Pieces::kHookPv[kNB - 1] == 1, "the last hook must sit in P.V");
        // slot k of hook h runs at step at(h) + k * stride(h) of its phase;
        // hooks of one phase must not overlap and must fit their loop
        static_for<0, kNB>([&](auto h_c) {
            constexpr int h = decltype(h_c)::value;
            constexpr int last = Pieces::kHookAt[h] + (kS - 1) * Pieces::kHookStride[h];
            static_assert(last < (Pieces::kHookPv[h] ? kPvSteps : kKSteps), "hook must fit its loop");
            if constexpr (h + 1 < kNB && Pieces::kHookPv[h + 1] == Pieces::kHookPv[h])
                static_assert(last < Pieces::kHookAt[h + 1], "hooks of a phase must not overlap");
        });

        const Src r0 = page_rsrc(p_lo, phys0);
        Stage stg[kS], s0p[kPieces];
        // the scales of the page whose pieces are stored next
        typename Pieces::PageScales sc;
        pc.load_scales(sc, r0);
        static_for<0, kPieces>([&](auto k) { pc.issue(s0p[k], r0, wave, k); });
        {
            const int row = active ? row0 + (lane0 & 31) : 0;
            const uint16_t* qrow = a.q + ((int64_t)b * M + row) * kD + (lane0 >> 5) * 8;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = __builtin_bit_cast(f16x8, *(const bf16x8*)(qrow + ks * 16));
        }
        Src r_next = page_rsrc(p_lo + 1, phys1);
        int phys2 = kSparse ? 0 : load_phys(p_lo + 2);
        st.m = -__builtin_inff();
        st.l = 0.f;
        st.o_zero = true;
#pragma unroll
        for (int md = 0; md < kMdBlocks; ++md) st.o[md] = f32x16{};
        static_for<0, kPieces>([&](auto k) {
            pc.store(s0p[k], sc, tiles[0], wave, k);
            if constexpr (k < Pieces::first(1)) pc.issue(stg[k], r_next, wave, k);   // batch 0 of page p_lo + 1
        });
        pc.load_scales(sc, r_next);
        convert_q();
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();

        for (int p = p_lo; p < p_hi; ++p) {
            const LDS_AS uint8_t* tile = tiles[(p - p_lo) & 1];
            LDS_AS uint8_t* tnext = tiles[(p - p_lo + 1) & 1];
            const int phys_next = kSparse ? 0 : load_phys(p + 3);
            Src r2;
            // hook h, slot k: store piece k of batch h (page p + 1) and load
            // piece k of the next batch into the freed slot; the last batch
            // is followed by batch 0 of page p + 2
            auto move_piece = [&](auto h_c, auto k_c) {
                constexpr int h = decltype(h_c)::value, k = decltype(k_c)::value;
                constexpr int n = Pieces::first(h) + k;
                if constexpr (n < Pieces::first(h + 1)) pc.store(stg[k], sc, tnext, wave, n);
                // page p + 1 is stored: the scales of page p + 2 follow
                if constexpr (n == kPieces - 1) pc.load_scales(sc, r2);
                if constexpr (h + 1 < kNB) {
                    constexpr int n2 = Pieces::first(h + 1) + k;
                    if constexpr (n2 < Pieces::first(h + 2)) pc.issue(stg[k], r_next, wave, n2);
                } else {
                    if constexpr (k < Pieces::first(1)) pc.issue(stg[k], r2, wave, k);
                }
            };
            auto qk_hook = [&](auto ks_c) {
                constexpr int ks = decltype(ks_c)::value;
                static_for<0, kNB>([&](auto h_c) {
                    constexpr int h = decltype(h_c)::value, at = Pieces::kHookAt[h];
                    constexpr int sd = Pieces::kHookStride[h];
                    if constexpr (!Pieces::kHookPv[h] && ks >= at && (ks - at) % sd == 0 && (ks - at) / sd < kS)
                        move_piece(h_c, std::integral_constant<int, (ks - at) / sd>{});
                });
                if constexpr (ks == kKSteps - 1) {
                    if constexpr (kSparse) {
                        // tile p + 2's rows have landed; tile p + 3's entries
                        // (loaded a tile ago) go out for theirs; tile p + 4's
                        // entries are loaded
                        r2 = page_rsrc(p + 2, row_of(pend));
                        pend = expand(p + 3, iv_next, mask3);
                        iv_next = load_idx(p + 4);
                    } else {
                        r2 = page_rsrc(p + 2, phys2);
                    }
                }
            };
            auto pv_hook = [&](auto step_c) {
                constexpr int step = decltype(step_c)::value;
                static_for<0, kNB>([&](auto h_c) {
                    constexpr int h = decltype(h_c)::value, at = Pieces::kHookAt[h];
                    constexpr int sd = Pieces::kHookStride[h];
                    if constexpr (Pieces::kHookPv[h] && step >= at && (step - at) % sd == 0 && (step - at) / sd < kS)
                        move_piece(h_c, std::integral_constant<int, (step - at) / sd>{});
                });
            };
            compute_tile<kSparse>(tile, qreg, qr_lds, st, min(max(n_vis - p * kPage, 0), kPage), mask_cur, scale_lane,
                                  qk_hook, pv_hook);
            r_next = r2;
            phys2 = phys_next;
            if constexpr (kSparse) {
                mask_cur = mask1;
                mask1 = mask2;
                mask2 = mask3;
            }
            __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);       // tile stores and reads retired
            wg_barrier();
        }
        // the last tile issued loads of pages past p_hi: zero-size
        // descriptors, nothing is fetched, and they are never waited for

        rowsplit_epilogue(a, st, lds + wave * (kRowsPerWave * 1024), b, M, row0, slot, active);
        // the next segment's first page and q_R fragments land in these bytes
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();
    }
}

}  // namespace

hipError_t launch_decode_fp4(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    const dim3 grid(a.num_workers * row_groups);
    switch (a.page_size) {
        case 16: return launch_with_events(mla_decode_kernel<16, false>, grid, stream, ev_start, ev_stop, a);
        case 32: return launch_with_events(mla_decode_kernel<32, false>, grid, stream, ev_start, ev_stop, a);
        case 64: return launch_with_events(mla_decode_kernel<64, false>, grid, stream, ev_start, ev_stop, a);
        case 128: return launch_with_events(mla_decode_kernel<128, false>, grid, stream, ev_start, ev_stop, a);
        case 256: return launch_with_events(mla_decode_kernel<256, false>, grid, stream, ev_start, ev_stop, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_fp4_sparse(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                    hipEvent_t ev_stop, bool window) {
    const dim3 grid(a.num_workers * row_groups);
    return window ? launch_with_events(mla_decode_kernel<64, true, true>, grid, stream, ev_start, ev_stop, a)
                  : launch_with_events(mla_decode_kernel<64, true>, grid, stream, ev_start, ev_stop, a);
}

}  // namespace mla
