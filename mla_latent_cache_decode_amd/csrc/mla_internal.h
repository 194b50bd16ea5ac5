// Internal interface between the C-ABI host code (api.cpp) and the kernel
// translation units.  Not installed; the public ABI is include/mla_decode.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Shapes this build instantiates (guide section 1.1: 512 latent + 64 RoPE).
// The decode works on tiles of 64 tokens whatever the page-block size
// ("DeepSeek-R1" record, constraint (1): decode kernels are instantiated per
// page-block size; 64 is the usual one, 32 that of a compressed layer).
constexpr int kPage = 64;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;                 // 576 elements per cached row
constexpr int kBf16RowBytes = 2 * kD;         // 1152
constexpr int kFp8Payload = kD + kD / 32;     // 594
constexpr int kFp8RowBytes = (kFp8Payload + 15) / 16 * 16;  // 608
// fp4 row (a reading of the same record's 288-byte fp4 variant at 512 dims):
// D/2 bytes of e2m1 codes, two per byte, then one e8m0 scale per 16 values
constexpr int kFp4Payload = kD / 2 + kD / 16;                // 324
constexpr int kFp4RowBytes = (kFp4Payload + 15) / 16 * 16;  // 336
// the fp8 decode's query rows: two terms (q_hi, q_lo), each in the fp8 row format
constexpr int kMxQxRowBytes = 2 * kFp8RowBytes;             // 1216
// The fp8 cache also serves a latent width of 448 (D = 512): the "DeepSeek-R1"
// record's constraint (2) row, 512 e4m3 codes and 16 e8m0 scales = 528 bytes
// with no padding.  Per latent width DC: the row, its stride, the 32-dim
// output blocks, the two-term query row.
constexpr int kDcNarrow = 448;
template <int DC>
struct Fp8Dims {
    static constexpr int kDc = DC;
    static constexpr int kD = DC + kDr;                             // 576 / 512
    static constexpr int kRowBytes = (kD + kD / 32 + 15) / 16 * 16;  // 608 / 528
    static constexpr int kMdBlocks = DC / 32;                        // 16 / 14
    static constexpr int kQxRowBytes = 2 * kRowBytes;
};
static_assert(Fp8Dims<kDc>::kRowBytes == kFp8RowBytes && Fp8Dims<kDcNarrow>::kRowBytes == 528, "fp8 rows");
constexpr int kRowsPerGroup = 128;            // query rows one workgroup serves
constexpr int kRowsPerWave = 32;
constexpr int kDecodeThreads = 256;           // 4 waves of 64

constexpr int kMaxWorkers = 4096;             // bound on context-split workers
constexpr int kMaxSplits = kMaxWorkers;       // a sequence has at most one split per worker

// Per-call scratch in the workspace.  The decode kernel writes, per
// sequence, its number of splits and first partial slot; split partials
// (O/l and lse) live in slots [slot, slot + nsplit).
struct PlanView {
    int32_t* seq_nsplit;        // [batch]
    int32_t* seq_slot;          // [batch]
    float* part_lse;            // [M][slots]: one row's split LSEs are contiguous
    uint16_t* part_o;           // fp16 [slots][M][d_c]: a split's O / l
    int32_t slots;              // partial slot capacity (row stride of part_lse)
};

struct DecodeArgs {
    const uint16_t* q;          // bf16 [B][s_q][n_h][kD]
    const uint8_t* kv;          // pages
    const int32_t* block_table; // [B][max_blocks]
    const int32_t* seq_lens;    // [B]
    float* out;                 // [B][M][d_c]
    float* lse;                 // [B][M] or null
    PlanView plan;
    uint8_t* qx;                // fp8 cache: the two-term query rows [B][M][2 fp8 rows] (workspace)
    int64_t page_bytes;         // bytes per page
    int32_t page_size;          // tokens per page block (16 .. 256, a power of two)
    int32_t batch;
    int32_t s_q;
    int32_t n_h;
    int32_t max_blocks;
    int32_t num_workers;
    int32_t overhead_units;     // per-segment fixed cost on the cost axis, in pages
    int32_t min_quota;          // lower bound on cost units per worker
    float scale_log2;           // softmax_scale * log2(e)
    // sparse (top-k) decode: batch counts (sequence, query position) units of
    // n_h rows each (s_q = 1 here), every unit topk entries long; the
    // kernels read each unit's index list and turn its valid entries into
    // cache rows through the block table of its sequence.  sparse_topk = 0:
    // the dense decode.
    int32_t sparse_topk;
    const int32_t* sparse_indices;  // [units][topk] token positions
    int32_t sparse_sq;              // query positions per sequence (unit u = b * sparse_sq + j)
    int32_t d_c;                    // latent width: kDc, or kDcNarrow (fp8 cache only)
};

// A sparse entry that does not take part has no row (row ids are
// page * page_size + slot); it is gathered from a row of zeros of
// kSparseZeroRowBytes that each kernel keeps in device memory.
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
// With MLA_FLAG_KV_WITHIN_4GIB the sparse gathers address rows inside
// the first kGatherWindow bytes of the cache with 32-bit buffer offsets (rows
// up to kGatherRowMax); kGatherNone lies past the window, so a load there
// returns zeros.
constexpr uint32_t kGatherWindow = 0xFFFFF000u;
constexpr uint32_t kGatherRowMax = (kGatherWindow - 2 * 576) / (2 * 576);
constexpr uint32_t kGatherNone = 0xFFFFFFF0u;
static_assert((uint64_t)kGatherRowMax * 1152 + 1152 <= kGatherWindow, "a window row ends inside the window");
static_assert(kGatherNone >= kGatherWindow, "the no-row offset lies past the window");
constexpr int kSparseZeroRowBytes = 2048;      // >= one bf16 row (1152 B)

struct CombineArgs {
    PlanView plan;
    float* out;
    float* lse;                 // may be null
    int32_t batch;
    int32_t rows;               // M = s_q * n_h
    int32_t d_c;                // latent width of a row (a multiple of 8, at most kDc)
};

// Launchers: enqueue on `stream`, return hipGetLastError() of the launch.
// ev_start / ev_stop (may be null): events that take the decode kernel's own
// start and end timestamps (recorded with its dispatch, not as separate
// stream packets).
hipError_t launch_decode_bf16(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                              hipEvent_t ev_stop);
// the fp4 cache (e2m1 codes, e8m0 per 16): dequantised into an fp16 tile
hipError_t launch_decode_fp4(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop);
// the fp8 cache's dense decode: quantise the queries into a.qx (two e4m3
// terms with e8m0 scales per 32), then the block-scaled decode
hipError_t launch_quantize_q_mx(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_fp8_mx(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                hipEvent_t ev_stop);
hipError_t launch_decode_fp8_mx_sparse(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                       hipEvent_t ev_stop, bool window);
// window: the cache lies in the first kGatherWindow bytes (MLA_FLAG_KV_WITHIN_4GIB)
hipError_t launch_decode_bf16_sparse(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                     hipEvent_t ev_stop, bool window);
hipError_t launch_decode_fp4_sparse(const DecodeArgs& a, int row_groups, hipStream_t stream, hipEvent_t ev_start,
                                    hipEvent_t ev_stop, bool window);
// max_splits: an upper bound on the splits of one sequence (the worker
// count); it sizes the combine's LDS and picks its shape.
hipError_t launch_combine(const CombineArgs& a, int max_splits, hipStream_t stream);

// Bytes of the per-device scratch that mla_decode_run_noalloc uses as its
// workspace (MLA_NOALLOC_SCRATCH_BYTES in the public header).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
// The device address of `device`'s copy of that scratch; `device` must be
// current.  Taken with hipGetSymbolAddress on the first call per device and
// kept; later calls return the kept address.  Thread-safe.
hipError_t scratch_address(int device, void** out);

}  // namespace mla
