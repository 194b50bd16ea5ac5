// Split-KV MLA decode for a bf16 latent cache on gfx950 (CDNA4).
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
// combine; a sequence served by one worker is finished here directly.
//
// Mapping onto CDNA4 (one workgroup of 4 waves per CU, all 160 KiB of LDS):
//  * Pages move HBM -> LDS with direct-to-LDS buffer loads (no VGPRs, no
//    LDS store instructions), one 64-token page per tile, double buffered:
//    page p + 1 is fetched while tile p is computed.  Rows past the visible
//    tokens are never fetched (the descriptor size excludes them; LDS gets
//    zeros).  Each lane fetches the 16-byte chunk that the swizzled tile
//    layout puts at its LDS slot, so the 1 KiB written by one load is
//    contiguous in LDS and the tile is read without bank conflicts.
//  * Q.K^T: wave w owns query rows 32w .. 32w + 31 and holds them in VGPRs
//    as bf16 MFMA B-operands (36 k-steps); the bf16 page is the A-operand
//    straight from LDS (v_mfma_f32_32x32x16_bf16: products exact, fp32
//    accumulation).  The 64 tokens are two 32-token blocks computed one
//    after the other, so the softmax of the first block runs on the VALU
//    while the matrix core works on the second.
//  * Online softmax per 32-token block with a lazy running max m: a row's
//    first block sets m, and the weights p = 2^(s - m) are rounded to fp16
//    (8x finer than bf16).  O is never rescaled in registers: a block whose
//    max exceeds m by more than 15 (log2 units; its weights would leave the
//    fp16 range) marks the segment, which is then computed once more with m
//    fixed at the first pass's final value.
//  * P.V is split by output dims: wave w accumulates O^T for dims
//    128w .. 128w + 127 of all 128 rows (4 x 4 blocks of 32 x 32, 256
//    AGPRs).  Each wave publishes its rows' P^T fragments in LDS; the V^T
//    fragments come from the tile through transposed reads
//    (ds_read_b64_tr_b16) and are converted bf16 -> fp16 in registers, so
//    every cache element is read from LDS once per P.V and converted once.
//  * Three workgroup barriers per tile: after the first block's weights are
//    published, after the second's, and at the end (page p + 1 landed,
//    tile p and the weights no longer read).
//  * Epilogue: the normalised rows are staged row-major in the idle tile
//    LDS and written as whole rows (fp16 for a split's partial).
#include "decode_common.h"

namespace mla {
namespace {

constexpr int kPFragBytes = 1024;                   // one P^T fragment: 64 lanes x 8 fp16
constexpr int kPBytes = 4 * 4 * kPFragBytes;        // 16384: 4 row blocks x 4 token steps
constexpr int kLdsBf16 = 2 * kTileBytes + kPBytes;  // 163840 = all of a CU's LDS
constexpr int kDmaPerWave = 18;                     // 1 KiB direct-to-LDS loads per wave per page
constexpr int kAhead = 2;                           // K fragment prefetch distance (MFMA steps)
constexpr float kTau = 15.0f;                       // lazy-rescale threshold (log2 units)
constexpr int kQkSteps = 2 * kKSteps;               // 72: two 32-token blocks x 36 k-steps

static_assert(4 * kDmaPerWave * 1024 == kTileBytes, "four waves move a page");

// The same 1 KiB direct-to-LDS load with a 64-bit address per lane (the
// sparse gather: every token row can sit anywhere in the cache).  No
// instruction offset: it would move the LDS destination as well.
__device__ __forceinline__ void dma16_gather(uint64_t addr, uint32_t dst) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(addr), "{m0}"(dst) : "memory");
}

// S^T += K Q^T on one k-step, with the accumulator in arch VGPRs.  Issued as
// asm: the builtin takes the accumulator form that O (in AGPRs) needs, and
// 32 more AGPRs for S would push O out.  The hardware orders dependent
// MFMAs; VALU readers of S wait for the last MFMA with s_nop (score_ready).
__device__ __forceinline__ void mfma_qk(f32x16& s, const bf16x8& k, const bf16x8& q) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void score_ready(f32x16& s) {
    // an XDL result needs 11 (8 passes) or 19 (16 passes) wait states before a VALU read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// Running softmax state of the lane's row (both lanes of a pair agree on m).
struct RowState {
    float m;    // running max in log2 units (softmax scale applied)
    float l;    // sum of weights over this lane's half of the tokens
};

// Lazy raise of the running max m by a block's max mx (both in log2 units).
// A row's first block sets m; a later block whose max exceeds m by more than kTau (its weights would
// leave the fp16 range) raises m to that max and returns true: O was
// accumulated against the old m, so the segment is computed again with m
// fixed at the end-of-pass value, which no block exceeds by more than kTau.
__device__ __forceinline__ bool raise_max(float mx, RowState& rs) {
    const bool need = mx > rs.m + kTau;
    const bool fresh = rs.m == -__builtin_inff();
    rs.m = need ? mx : rs.m;
    return need && !fresh;
}

// kSparse: the top-k decode ("DeepSeek-V3.2" record).  A unit (one query
// position of one sequence, n_h rows) attends to the topk rows its index
// list selects; tile p holds entries 64p .. 64p + 63, gathered row by row
// (wave w loads tokens 16w .. 16w + 15).  The kernel turns the list into
// rows itself, in its page pipeline: the entries of tile p + 3 are loaded
// during tile p; those of tile p + 2 become the tile's mask (a ballot of
// 0 <= t < the query's causal context) and, for each lane's two tokens,
// block-table loads; tile p + 1's rows (page * block + slot) feed its
// gathers.  The mask takes the place of the length mask.  Entries that do
// not take part are fetched from a row of zeros (their weights are 0;
// zeros keep 0 x V finite).
__device__ __attribute__((aligned(256))) uint8_t g_sparse_zero_row[kSparseZeroRowBytes] = {};

// kWin (sparse only): the caller has declared that the whole cache lies in
// the first kGatherWindow bytes from its base; rows are then gathered with
// 32-bit buffer offsets.
template <int PS, bool kSparse, bool kWin = false>
__global__ __launch_bounds__(kDecodeThreads, 1) void mla_decode_bf16_kernel(DecodeArgs a) {
    typedef PageGeom<kSparse ? 16 : PS> Geom;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBf16];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
    int* sbuf = (int*)smem;                 // planner scratch; dead before the first page lands

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int worker, rg;
    block_role(a.num_workers, worker, rg);
    const int M = a.s_q * a.n_h;
    const int row_base = rg * kRowsPerGroup;
    const int row0 = row_base + wave * kRowsPerWave;
    const bool active = row0 < M;
    const int j_wave = (active ? row0 : M - 1) / a.n_h;
    const int j_last = min(row_base + kRowsPerGroup - 1, M - 1) / a.n_h;
    const int n_blocks = min((M - row_base + kRowsPerWave - 1) / kRowsPerWave, 4);   // active row blocks

    const WorkerStart start = plan_worker(a, worker, rg == 0, sbuf, tid);
    if (start.b >= a.batch) return;
    const int64_t Q = start.quota;
    const int64_t w_lo = (int64_t)worker * Q, w_hi = w_lo + Q;

    LDS_AS uint8_t* const tiles[2] = {lds, lds + kTileBytes};
    LDS_AS uint8_t* const pbuf = lds + 2 * kTileBytes;
    const int lane0 = tid & 63;
    // first token (within a tile) of the page this wave loads from
    const int tok0 = Geom::tok0(wave);
    // direct-to-LDS source offset of this lane inside a page piece: token
    // i >> 3 of the piece, the chunk whose swizzled slot is i & 7 (pieces
    // of odd row blocks flip the slot's low bit: address ^ 16)
    const int dma_lane = (lane0 >> 3) * kBf16RowBytes + (((lane0 & 7) ^ sw(lane0 >> 3)) << 4);

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

        const int n_vis = active ? L - a.s_q + 1 + j_wave : 0;     // tokens this wave's rows see
        const int n_load = L - a.s_q + 1 + j_last;                  // tokens the workgroup loads

        // block-table entries by vector loads, a tile ahead of their use:
        // the entry of the page holding token tok0 of tile p.  Entries the
        // segment cannot touch read 0; an entry past the sequence's last
        // page is read but not used (its rows are past n_load)
        const __amdgpu_buffer_rsrc_t bt = make_rsrc((const uint8_t*)(a.block_table + (int64_t)b * a.max_blocks),
                                                    (PS < kPage ? min(Geom::entries(p_hi), a.max_blocks)
                                                                : Geom::entries(p_hi)) * 4);
        auto load_phys = [&](int p) -> int {
            return __builtin_amdgcn_raw_buffer_load_b32(bt, Geom::entry(p, tok0) * 4, 0, 0);
        };
        // the same by a scalar load, for the segment prologue: its wait
        // (lgkmcnt) does not queue behind the direct-to-LDS query loads
        const int n_entries = PS < kPage ? min(Geom::entries(p_hi), a.max_blocks) : Geom::entries(p_hi);
        auto load_phys_s = [&](int p) -> int {
            const int e = __builtin_amdgcn_readfirstlane(Geom::entry(p, tok0));
            const bool in = e < n_entries;
            const int v = ld_const(a.block_table + (int64_t)b * a.max_blocks + (in ? e : 0));
            return in ? v : 0;
        };
        // rows of tile p this wave's page holds for the workgroup (0 past p_hi); uniform
        auto page_rows = [&](int p) {
            return __builtin_amdgcn_readfirstlane(
                p < p_hi ? min(max(n_load - p * kPage - tok0, 0), Geom::kRangeTok) : 0);
        };
        // descriptor over those rows of physical page phys
        auto rsrc_of = [&](int p, int phys, int rows) {
            return make_rsrc(a.kv + (int64_t)__builtin_amdgcn_readfirstlane(phys) * a.page_bytes +
                                 Geom::row_in_page(p, tok0) * kBf16RowBytes,
                             rows * kBf16RowBytes);
        };
        auto page_rsrc = [&](int p, int phys) { return rsrc_of(p, phys, page_rows(p)); };
        // piece k of this wave: 1 KiB = 8 rows (token group g) of one 64-dim
        // column block cb, from the wave's page; it lands at LDS piece
        // cb * 8 + g of the tile.  g and k agree in their low bit (the
        // swizzle's slot flip).
        auto dma_piece = [&](__amdgpu_buffer_rsrc_t r, LDS_AS uint8_t* tile, int k) {
            if constexpr (Geom::kRanges == 1) {
                const int pn = wave * kDmaPerWave + k;
                const int off = (pn & 7) * 8 * kBf16RowBytes + ((pn >> 3) << 7);
                dma16(r, (pinned(dma_lane) ^ ((k & 1) << 4)) + off, (uint32_t)(uintptr_t)(tile + pn * 1024));
            } else {
                constexpr int kGroups = 8 / Geom::kRanges;        // token groups of 8 in one page
                const int i = (wave % Geom::kWavesPerRange) * kDmaPerWave + k;
                const int gl = i % kGroups, cb = i / kGroups;
                const int pn = cb * 8 + tok0 / 8 + gl;
                const int off = gl * 8 * kBf16RowBytes + (cb << 7);
                dma16(r, (pinned(dma_lane) ^ ((k & 1) << 4)) + off, (uint32_t)(uintptr_t)(tile + pn * 1024));
            }
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
        auto expand = [&](int iv, int p, uint32_t& m_lo, uint32_t& m_hi) -> SparsePend {
            const int l = pinned(lane0);
            const bool valid = p < p_hi && p * kPage + l < L && iv >= 0 && iv < n_ctx;
            const uint64_t m = __builtin_amdgcn_ballot_w64(valid);
            m_lo = (uint32_t)m;
            m_hi = (uint32_t)(m >> 32);
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
        // kWin: one buffer descriptor over the window; a 32-bit offset per
        // lane issues faster than a 64-bit address (-4.7 % on the sparse
        // step, same box).  An entry that does not take part -- or a row past
        // the window, should the caller's declaration be wrong -- gets an
        // offset past the window, which the range check turns into zeros.
        // Otherwise 64-bit addresses; entries that do not take part read a
        // row of zeros.  Zeros weigh 0 and keep 0 x V finite.
        const __amdgpu_buffer_rsrc_t r_win = make_rsrc(a.kv, (int)kGatherWindow);
        const uint8_t* const zero_row = g_sparse_zero_row;
        // piece k of tile p (row ids rw): token 16w + 8(k & 1) + x, column
        // block k >> 1, landing at LDS piece (k >> 1) * 8 + 2w + (k & 1)
        auto dma_sparse = [&](const u32x2& rw, int p, LDS_AS uint8_t* tile, auto k_c) {
            constexpr int k = decltype(k_c)::value, gl = k & 1, cb = k >> 1;
            const uint32_t row = rw[gl];
            const bool live = p < p_hi && row != kNoRow;
            const int l = pinned(lane0);
            const int chunk = ((((l & 7) ^ sw(l >> 3)) << 4) ^ (gl << 4)) + cb * 128;
            const uint32_t dst = (uint32_t)(uintptr_t)(tile + (cb * 8 + 2 * wave + gl) * 1024);
            if constexpr (kWin) {
                const bool in = live && row <= kGatherRowMax;
                dma16(r_win, (int)(in ? row * (uint32_t)kBf16RowBytes + chunk : kGatherNone), dst);
            } else {
                const uint8_t* base = live ? a.kv + (uint64_t)row * kBf16RowBytes : zero_row;
                dma16_gather((uint64_t)(base + chunk), dst);
            }
        };

        const float scale_log2 = a.scale_log2;
        RowState rs;
        rs.m = -__builtin_inff();
        // a second pass runs only if a block overflowed the first pass's m
        for (int pass = 0;; ++pass) {
        // segment prologue: the first half of the queries, the first
        // block-table entries (or index-list entries), the first page, the
        // second half of the queries.  The queries go first: the compiler's
        // waits for the entries count only its own loads, so a wait for an
        // entry also waits for every direct-to-LDS load issued before it.
        // this wave's 32 query rows as bf16 B-operands: lane i holds row
        // i & 31, elements 8 (i >> 5) .. + 7 of each 16-element k-step.
        // Loaded per pass (from L2 on a second pass) so that they are not
        // live across the epilogue.  The rows (36 KiB, contiguous) come in
        // two halves of 18 k-steps through this wave's quarter of tiles[1],
        // which is free until the loop loads page p_lo + 1: direct-to-LDS
        // loads of whole 1 KiB runs, then fragment reads.  A load of lanes
        // reading 32 rows each would touch 32 lines per instruction; these
        // touch 9 to 11.  16-byte chunk m = 36 r + k of a half (row r, byte
        // 16 k of the row's half) sits at LDS chunk m ^ ((m >> 4) & 3), so
        // each load still covers one contiguous KiB (in permuted order) and
        // the 16 rows one fragment read serves per pass hit 16 distinct bank
        // groups.
        bf16x8 qf[kKSteps];
        LDS_AS uint8_t* const qst = tiles[1] + wave * (kTileBytes / 4);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint8_t*)(a.q + ((int64_t)b * M + (active ? row0 : 0)) * kD),
                                                    kRowsPerWave * kD * 2);
        auto q_half_load = [&](int h) {
            const int l = opaque_lane();
            const int pl = l ^ ((l >> 4) & 3);
#pragma unroll
            for (int c = 0; c < kKSteps / 2; ++c) {
                const int m = 64 * c + pl, r = m / 36, k = m - 36 * r;
                dma16_shared(rq, r * (kD * 2) + h * kD + 16 * k, (uint32_t)(uintptr_t)(qst + c * 1024));
            }
        };
        auto q_half_read = [&](int h) {
            const int l = opaque_lane();
            const int m0 = (l & 31) * 36 + (l >> 5);
#pragma unroll
            for (int j = 0; j < kKSteps / 2; ++j) {
                const int m = m0 + 2 * j;
                qf[h * (kKSteps / 2) + j] = *(const LDS_AS bf16x8*)(qst + ((m ^ ((m >> 4) & 3)) << 4));
            }
        };
        q_half_load(0);
        int phys0 = 0, phys_next = 0, rows0 = 0;
        uint32_t mk_lo = ~0u, mk_hi = ~0u;       // sparse: mask of the current tile
        uint32_t mk_next_lo = ~0u, mk_next_hi = ~0u;
        SparsePend pend0, pend;                  // sparse: tiles p_lo and p_lo + 1, then p + 1
        int iv = 0;                              // sparse: the lane's entry of tile p + 2
        if constexpr (kSparse) {
            const int iv0 = load_idx(p_lo), iv1 = load_idx(p_lo + 1);
            iv = load_idx(p_lo + 2);
            pend0 = expand(iv0, p_lo, mk_lo, mk_hi);
            pend = expand(iv1, p_lo + 1, mk_next_lo, mk_next_hi);
        } else {
            phys0 = load_phys_s(p_lo);
            phys_next = load_phys_s(p_lo + 1);
            // computed here from an opaque copy of n_load, and held in an SGPR:
            // a copy hoisted out of the pass loop would be spilled, and its
            // reload would wait for every load in flight
            int nl = n_load;
            asm volatile("" : "+s"(nl));
            rows0 = __builtin_amdgcn_readfirstlane(
                p_lo < p_hi ? min(max(nl - p_lo * kPage - tok0, 0), Geom::kRangeTok) : 0);
            asm volatile("" : "+s"(rows0));
        }
        if constexpr (kSparse) {
            const u32x2 rw0 = rows_of(pend0);
            static_for<0, kDmaPerWave>([&](auto k) { dma_sparse(rw0, p_lo, tiles[0], k); });
        } else {
            const __amdgpu_buffer_rsrc_t r0 = rsrc_of(p_lo, phys0, rows0);
#pragma unroll
            for (int k = 0; k < kDmaPerWave; ++k) dma_piece(r0, tiles[0], k);
        }
        // the first half landed (only the page's loads may still be in
        // flight); its reads complete before the second half overwrites it
        __builtin_amdgcn_s_waitcnt(VMCNT_IMM(kDmaPerWave));
        q_half_read(0);
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        q_half_load(1);
        rs.l = 0.f;
        bool overflow = false;
        f32x16 o[4][4];                   // O^T blocks [dim block][row block]
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) o[db][hb] = f32x16{};
        __builtin_amdgcn_s_waitcnt(VMCNT0_IMM);
        q_half_read(1);
        // every wave's reads of tiles[1] complete before any wave loads
        // page p_lo + 1 into it
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();

        for (int p = p_lo; p < p_hi; ++p) {
            const LDS_AS uint8_t* tile = tiles[(p - p_lo) & 1];
            LDS_AS uint8_t* const tnext = tiles[(p - p_lo + 1) & 1];
            __amdgpu_buffer_rsrc_t r_next;
            int phys_after = 0;
            u32x2 rw_next;
            uint32_t mk_after_lo = ~0u, mk_after_hi = ~0u;
            if constexpr (kSparse) {
                // tile p + 1's rows (its block-table entries landed during
                // tile p - 1), tile p + 2's mask and entries, tile p + 3's list
                rw_next = rows_of(pend);
                pend = expand(iv, p + 2, mk_after_lo, mk_after_hi);
                iv = load_idx(p + 3);
            } else {
                r_next = page_rsrc(p + 1, phys_next);
                phys_after = load_phys(p + 2);
            }
            const int n_valid = min(max(n_vis - p * kPage, 0), kPage);

            const int lane = opaque_lane();
            const int hi = lane >> 5;
            int k_off[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) k_off[k] = tile_off(lane & 31, 2 * k + hi);
            // V^T fragment pointers (see read_v)
            const LDS_AS uint8_t* vp[2][2];
            {
                const int g = lane >> 4, li = lane & 15;
                const int tok = ((g >> 1) << 2) + (li >> 2);
                const int dim = ((g & 1) << 4) + ((li & 3) << 2);
                const LDS_AS uint8_t* tw = tile + wave * 2 * 8192;     // this wave's 128 dims
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int off = tile_off(tok, (m * 32 + dim) >> 3) + (dim & 7) * 2;
                    vp[m][0] = tw + off;
                    vp[m][1] = tw + (off ^ 16) + 8 * 128;
                }
            }
            const LDS_AS uint8_t* const pown = pbuf + wave * 4 * kPFragBytes + lane * 16;
            const LDS_AS uint8_t* const pall = pbuf + lane * 16;

            f32x16 sblk[2] = {f32x16{}, f32x16{}};
            bf16x8 kf[kAhead + 1];
            auto read_k = [&](auto g_c) {
                constexpr int g = decltype(g_c)::value, blk = g / kKSteps, ks = g % kKSteps;
                kf[g % (kAhead + 1)] =
                    *(const LDS_AS bf16x8*)(tile + k_off[ks & 3] + (ks >> 2) * 8192 + blk * 4096);
            };
            // V^T fragment (dim block db of this wave, token step ts): two
            // transposed reads (tokens 16 ts + 8 e + token_lane, dims
            // 128 wave + 32 db + dim_lane), converted to fp16
            u32x4 vf[2][4];       // raw bf16 pairs after the read, fp16 pairs after conv_v
            auto read_v = [&](auto ts_c, auto db_c) {
                constexpr int ts = decltype(ts_c)::value, db = decltype(db_c)::value;
                constexpr int off = (db >> 1) * 8192 + ts * 16 * 128;
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp[db & 1][0] + off));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp[db & 1][1] + off));
                vf[ts & 1][db] =
                    __builtin_bit_cast(u32x4, i16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
            };
            auto conv_v = [&](auto ts_c, auto db_c, auto half_c) {
                constexpr int ts = decltype(ts_c)::value, db = decltype(db_c)::value, h = decltype(half_c)::value;
#pragma unroll
                for (int e = 2 * h; e < 2 * h + 2; ++e) vf[ts & 1][db][e] = bf16x2_to_f16x2(vf[ts & 1][db][e]);
            };
            u32x4 pf[2][4];
            auto read_p = [&](auto ts_c) {
                constexpr int ts = decltype(ts_c)::value;
#pragma unroll
                for (int hb = 0; hb < 4; ++hb)
                    pf[ts & 1][hb] = *(const LDS_AS u32x4*)(pall + (hb * 4 + ts) * kPFragBytes);
            };

            // softmax of one 32-token block (this wave's rows): statistics,
            // then the two fp16 fragments published in LDS
            // softmax of one 32-token block (this wave's rows) in small
            // stages that issue between MFMAs: three for the statistics,
            // one per weight, one per published fragment
            float neg_m = 0.f, lsum = 0.f, mx0 = 0.f, mx1 = 0.f;
            float ya[4], xa[4];
            u32x4 pk[2];
            auto sm_max = [&](auto blk_c, auto part_c) {
                constexpr int blk = decltype(blk_c)::value, part = decltype(part_c)::value;
                f32x16& sv = sblk[blk];
                if constexpr (part == 0) {
                    score_ready(sv);
                    if constexpr (kSparse) {
                        // the lane's token c_r + 4 hi of the block takes part iff its mask bit is set
                        const uint32_t mb = blk == 0 ? mk_lo : mk_hi;
                        if (mb != ~0u) {
                            const uint32_t ml = mb >> (4 * hi);
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int c_r = ((r >> 2) << 3) + (r & 3);
                                sv[r] = (ml >> c_r) & 1 ? sv[r] : -__builtin_inff();
                            }
                        }
                    } else if (n_valid < 32 * (blk + 1)) {
                        const int nv_lane = n_valid - 32 * blk - 4 * hi;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int c_r = ((r >> 2) << 3) + (r & 3);
                            sv[r] = c_r < nv_lane ? sv[r] : -__builtin_inff();
                        }
                    }
                    mx0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
                    mx1 = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
                } else if constexpr (part == 1) {
                    mx0 = fmaxf(fmaxf(mx0, sv[6]), sv[7]);
                    mx1 = fmaxf(fmaxf(mx1, sv[8]), sv[9]);
                } else if constexpr (part == 2) {
                    mx0 = fmaxf(fmaxf(mx0, sv[10]), sv[11]);
                    mx1 = fmaxf(fmaxf(mx1, sv[12]), sv[13]);
                } else if constexpr (part == 3) {
                    mx0 = fmaxf(fmaxf(mx0, sv[14]), sv[15]);
                    mx0 = pair_max(fmaxf(mx0, mx1)) * scale_log2;
                } else {
                    // weights published so far are relative to the current m
                    rs.l += lsum;
                    lsum = 0.f;
                    overflow |= raise_max(mx0, rs);
                    // a row with nothing visible yet keeps m = -inf; its
                    // scores are -inf too and their weights 0
                    neg_m = rs.m == -__builtin_inff() ? 0.f : -rs.m;
                }
            };
            // weight e in three dependent parts, one MFMA step apart
            auto sm_exp = [&](auto blk_c, auto e_c, auto part_c) {
                constexpr int blk = decltype(blk_c)::value, e = decltype(e_c)::value, part = decltype(part_c)::value;
                if constexpr (part == 0) {
                    ya[e % 4] = fmaf(sblk[blk][e], scale_log2, neg_m);
                } else if constexpr (part == 1) {
                    xa[e % 4] = fast_exp2(ya[e % 4]);
                } else {
                    lsum += xa[e % 4];
                    if constexpr (e % 2 == 1)
                        pk[e / 8][(e % 8) / 2] =
                            __builtin_bit_cast(uint32_t, f16x2{(_Float16)xa[(e - 1) % 4], (_Float16)xa[e % 4]});
                }
            };
            auto sm_write = [&](auto blk_c, auto f_c) {
                constexpr int blk = decltype(blk_c)::value, f = decltype(f_c)::value;
                *(LDS_AS u32x4*)(pown + (2 * blk + f) * kPFragBytes) = pk[f];
            };
            // stage schedule of a block's softmax, by MFMA step k counted from
            // the step its scores are complete: max parts at 2..6, weight e
            // over 7 + e .. 9 + e, fragment f published after its eighth weight
            auto softmax_step = [&](auto blk_c, auto k_c) {
                constexpr int k = decltype(k_c)::value;
                if constexpr (k >= 2 && k <= 6) sm_max(blk_c, std::integral_constant<int, k - 2>{});
                static_for<0, 3>([&](auto part_c) {
                    constexpr int e = k - 7 - decltype(part_c)::value;
                    if constexpr (e >= 0 && e < 16) sm_exp(blk_c, std::integral_constant<int, e>{}, part_c);
                });
                if constexpr (k == 17) sm_write(blk_c, std::integral_constant<int, 0>{});
                if constexpr (k == 25) sm_write(blk_c, std::integral_constant<int, 1>{});
            };

            // ---- Q.K^T, block 0 then block 1.  Hooks: direct-to-LDS loads of
            // page p + 1 (block 0), V^T fragments of token steps 0 and 1, the
            // softmax of block 0 (block 1), first barrier.
            static_for<0, kAhead>([&](auto i) { read_k(i); });
            static_for<0, kQkSteps>([&](auto g_c) {
                constexpr int g = decltype(g_c)::value, blk = g / kKSteps, ks = g % kKSteps;
                if constexpr (g + kAhead < kQkSteps) read_k(std::integral_constant<int, g + kAhead>{});
                mfma_qk(sblk[blk], kf[g % (kAhead + 1)], qf[ks]);
                // page p + 1: one direct-to-LDS load every fourth MFMA.  The
                // sparse gather issues one per MFMA over the first 18 steps:
                // rows scattered over the cache take longer to arrive, and the
                // early start measured -15 % on its step (the dense page is
                // no faster that way: +3 % on the long-context workload).
                if constexpr (kSparse) {
                    if constexpr (g < kDmaPerWave)
                        dma_sparse(rw_next, p + 1, tnext, std::integral_constant<int, g>{});
                } else if constexpr (g % 4 == 0 && g / 4 < kDmaPerWave) {
                    dma_piece(r_next, tnext, g / 4);
                }
                if constexpr (blk == 0) {
                    // V^T of token step 0
                    if constexpr (ks >= 6 && ks < 30 && (ks - 6) % 6 == 0)
                        read_v(std::integral_constant<int, 0>{}, std::integral_constant<int, (ks - 6) / 6>{});
                    if constexpr (ks >= 9 && ks < 33 && (ks - 9) % 6 < 2)
                        conv_v(std::integral_constant<int, 0>{}, std::integral_constant<int, (ks - 9) / 6>{},
                               std::integral_constant<int, (ks - 9) % 6>{});
                } else {
                    softmax_step(std::integral_constant<int, 0>{}, std::integral_constant<int, ks>{});
                    if constexpr (ks == 28) {
                        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
                        wg_barrier();
                    }
                    if constexpr (ks == 33) read_p(std::integral_constant<int, 0>{});
                    // V^T of token step 1, once block 0's scores are dead
                    if constexpr (ks >= 22 && ks < 34 && (ks - 22) % 3 == 0)
                        read_v(std::integral_constant<int, 1>{}, std::integral_constant<int, (ks - 22) / 3>{});
                    if constexpr (ks >= 24 && ks < 36 && (ks - 24) % 3 < 2)
                        conv_v(std::integral_constant<int, 1>{}, std::integral_constant<int, (ks - 24) / 3>{},
                               std::integral_constant<int, (ks - 24) % 3>{});
                }
                __builtin_amdgcn_sched_barrier(0);
            });

            // ---- O^T += V^T P^T over token steps 0..3.  Hooks: softmax of
            // block 1 (step 0), second barrier (step 1), fragments of the
            // following token steps.
            static_for<0, 64>([&](auto st_c) {
                constexpr int st = decltype(st_c)::value, ts = st / 16, i = st % 16, db = i / 4, hb = i % 4;
                o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vf[ts & 1][db]),
                                                                  __builtin_bit_cast(f16x8, pf[ts & 1][hb]),
                                                                  o[db][hb], 0, 0, 0);
                if constexpr (st < 26) softmax_step(std::integral_constant<int, 1>{}, std::integral_constant<int, st>{});
                if constexpr (st == 8) read_p(std::integral_constant<int, 1>{});
                if constexpr (st == 27) {
                    __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
                    wg_barrier();
                }
                if constexpr (st == 28) read_p(std::integral_constant<int, 2>{});
                if constexpr (st == 34) read_p(std::integral_constant<int, 3>{});
                // V^T of token step 2 into the registers of step 0 once its
                // dim block is issued, converted after the weights are done;
                // step 3 likewise during step 2
                if constexpr (st >= 4 && st <= 16 && st % 4 == 0)
                    read_v(std::integral_constant<int, 2>{}, std::integral_constant<int, st / 4 - 1>{});
                if constexpr (st >= 24 && st < 32)
                    conv_v(std::integral_constant<int, 2>{}, std::integral_constant<int, (st - 24) / 2>{},
                           std::integral_constant<int, (st - 24) % 2>{});
                if constexpr (st >= 36 && st <= 48 && st % 4 == 0)
                    read_v(std::integral_constant<int, 3>{}, std::integral_constant<int, st / 4 - 9>{});
                if constexpr (st >= 38 && st < 52 && (st - 38) % 4 < 2)
                    conv_v(std::integral_constant<int, 3>{}, std::integral_constant<int, (st - 38) / 4>{},
                           std::integral_constant<int, (st - 38) % 4>{});
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) asm volatile("" : "+a"(o[db][hb]));
            rs.l += lsum;
            if constexpr (kSparse) {
                mk_lo = mk_next_lo;
                mk_hi = mk_next_hi;
                mk_next_lo = mk_after_lo;
                mk_next_hi = mk_after_hi;
            } else {
                phys_next = phys_after;
            }
            // page p + 1 landed, tile p and the weights are no longer read
            __builtin_amdgcn_s_waitcnt(VMCNT0_IMM);
            __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
            wg_barrier();
        }
        // the last tile fetched page p_hi through a zero-size descriptor:
        // nothing was read and its zeros are never used

        // epilogue: each wave owns the l of its rows; publish 1/l and the
        // overflow flag, then every wave normalises its dims of all rows
        const int lane = tid & 63;
        const float l_tot = pair_sum(rs.l);
        float* const inv_l = (float*)(smem + 2 * kTileBytes);
        int* const flags = (int*)(smem + 2 * kTileBytes + 4 * kRowsPerWave * 4);
        const bool wave_overflow = __builtin_amdgcn_ballot_w64(overflow) != 0;
        if (lane < 32) inv_l[wave * 32 + lane] = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        if (lane == 0) flags[wave] = wave_overflow;
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();
        const bool again = pass == 0 && (flags[0] | flags[1] | flags[2] | flags[3]);
        if (!again) {
            // lane-derived offsets come from opaque_lane() so that they are
            // computed here, not hoisted out of the page loop into registers
            const int lane_e = opaque_lane();
            if (lane_e < 32 && active) {
                const float lse_v = l_tot > 0.f ? (rs.m + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                                : -__builtin_inff();
                const int row = row0 + lane_e;
                if (slot < 0) {
                    if (a.lse) a.lse[(int64_t)b * M + row] = lse_v;
                } else {
                    a.plan.part_lse[(int64_t)row * a.plan.slots + slot] = lse_v;
                }
            }
            // O^T lives in MFMA layout (lane = row), so direct stores would
            // scatter 8-16 bytes over 32 rows per instruction.  The rows go
            // through LDS (the tile buffers are free) and leave as whole rows.
            const int hi = lane_e >> 5;
            float inv[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) inv[hb] = inv_l[hb * 32 + (lane_e & 31)];
            auto norm4 = [&](int db, int hb, int r4) {
                return f32x4{o[db][hb][r4 * 4 + 0] * inv[hb], o[db][hb][r4 * 4 + 1] * inv[hb],
                             o[db][hb][r4 * 4 + 2] * inv[hb], o[db][hb][r4 * 4 + 3] * inv[hb]};
            };
            const int n_rows = n_blocks * kRowsPerWave;
            if (slot >= 0) {
                // fp16 partial rows of 1 KiB; 8-byte slot s of row r sits at
                // slot s ^ (r & 31), so the 32 rows one write touches hit
                // distinct banks
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) {
                    if (hb < n_blocks) {
                        const int r = hb * 32 + (lane_e & 31);
#pragma unroll
                        for (int db = 0; db < 4; ++db)
#pragma unroll
                            for (int r4 = 0; r4 < 4; ++r4) {
                                const f32x4 v = norm4(db, hb, r4);
                                const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                                const int sl = wave * 32 + db * 8 + r4 * 2 + hi;
                                *(LDS_AS u32x2*)(lds + r * 1024 + ((sl ^ (r & 31)) << 3)) = __builtin_bit_cast(u32x2, h);
                                // one accumulator block at a time
                                __builtin_amdgcn_sched_barrier(0);
                            }
                    }
                }
                __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
                wg_barrier();
                // wave w stores rows 32w .. 32w + 31, lane l the 16 bytes of
                // logical slots 2l, 2l + 1
                uint16_t* const pbase = a.plan.part_o + ((int64_t)slot * M + row_base) * kDc + lane_e * 8;
                for (int j = 0; j < kRowsPerWave; ++j) {
                    const int r = wave * kRowsPerWave + j;
                    if (r >= n_rows) break;
                    u32x4 v = *(const LDS_AS u32x4*)(lds + r * 1024 + (((2 * lane_e) ^ (r & 30)) << 3));
                    if (r & 1) v = u32x4{v[2], v[3], v[0], v[1]};
                    *(u32x4*)(pbase + r * kDc) = v;
                }
            } else {
                // fp32 output rows of 2 KiB, 64 rows at a time; 16-byte
                // granule g of row r sits at granule g ^ (r & 15)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int hb = 2 * half + hh;
                        if (hb < n_blocks) {
                            const int r = hh * 32 + (lane_e & 31);
#pragma unroll
                            for (int db = 0; db < 4; ++db)
#pragma unroll
                                for (int r4 = 0; r4 < 4; ++r4) {
                                    const int g = wave * 32 + db * 8 + r4 * 2 + hi;
                                    *(LDS_AS f32x4*)(lds + r * 2048 + ((g ^ (r & 15)) << 4)) = norm4(db, hb, r4);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                        }
                    }
                    __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
                    wg_barrier();
                    // wave w stores rows 16w .. 16w + 15 of the half, two
                    // instructions of 1 KiB per row
                    float* const obase = a.out + ((int64_t)b * M + row_base + half * 64) * kDc + lane_e * 4;
                    for (int j = 0; j < 16; ++j) {
                        const int r = wave * 16 + j;
                        if (half * 64 + r >= n_rows) break;
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int g = k * 64 + lane_e;
                            const f32x4 v = *(const LDS_AS f32x4*)(lds + r * 2048 + ((g ^ (r & 15)) << 4));
                            *(f32x4*)(obase + r * kDc + k * 256) = v;
                        }
                    }
                    if (half == 0) {
                        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
                        wg_barrier();
                    }
                }
            }
        }
        // the next pass or segment overwrites inv_l and the flags
        __builtin_amdgcn_s_waitcnt(LGKMCNT0_IMM);
        wg_barrier();
        if (!again) break;
        }
    }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                              hipEvent_t ev_stop) {
    const dim3 grid(a.num_workers * row_groups);
    switch (a.page_size) {
        case 16: return launch_with_events(mla_decode_bf16_kernel<16, false>, grid, stream, ev_start, ev_stop, a);
        case 32: return launch_with_events(mla_decode_bf16_kernel<32, false>, grid, stream, ev_start, ev_stop, a);
        case 64: return launch_with_events(mla_decode_bf16_kernel<64, false>, grid, stream, ev_start, ev_stop, a);
        case 128: return launch_with_events(mla_decode_bf16_kernel<128, false>, grid, stream, ev_start, ev_stop, a);
        case 256: return launch_with_events(mla_decode_bf16_kernel<256, false>, grid, stream, ev_start, ev_stop, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_bf16_sparse(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                     hipEvent_t ev_stop, bool window) {
    // rows are gathered one by one: the page-block size enters only as a shift
    const dim3 grid(a.num_workers * row_groups);
    return window ? launch_with_events(mla_decode_bf16_kernel<64, true, true>, grid, stream, ev_start, ev_stop, a)
                  : launch_with_events(mla_decode_bf16_kernel<64, true, false>, grid, stream, ev_start, ev_stop, a);
}

}  // namespace mla
