// C ABI of the MLA decode library (declared in include/mla_decode.h).
//
// Host responsibilities: validate every argument before touching HIP, query
// the device once at init, size the workspace, and enqueue decode -> combine
// on the caller's stream without synchronising (the work plan is derived
// from seq_lens on the device, inside the decode kernel).  All device memory
// is the caller's.
#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "mla_internal.h"

struct mla_decode_handle {
    mla_decode_params_t p;
    int device;
    int compute_units;
    int num_workers;
    int row_groups;
    int rows;                  // M = s_q * n_h
    int partial_slots;         // upper bound on partial results
    hipEvent_t ev_start;
    hipEvent_t ev_stop;
    void* scratch;             // this device's copy of the no-alloc scratch (a device address)
};

namespace {

static_assert(MLA_NOALLOC_SCRATCH_BYTES == mla::kNoAllocScratchBytes, "the header states the scratch size");

constexpr size_t kAlign = 256;
constexpr int kOverheadUnits = 3;    // per-segment cost (query load, first page, epilogue), in pages: measured ~2.2 tiles of prologue plus the partial write
constexpr int kMinQuota = 1;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// bytes of one query row's two e4m3 terms (the fp8 cache's decode)
size_t qx_row_bytes(const mla_decode_handle* h) {
    return 2 * mla_kv_row_stride(MLA_KV_FP8_E4M3_E8M0, h->p.d_c, h->p.d_r);
}

struct WsLayout {
    size_t seq_nsplit, seq_slot, part_lse, part_o, qx, total;
};

WsLayout layout(const mla_decode_handle* h, int32_t batch) {
    WsLayout l{};
    const size_t nb = (size_t)(batch > 0 ? batch : 1);
    size_t off = 0;
    l.seq_nsplit = off;    off += align_up(nb * sizeof(int32_t));
    l.seq_slot = off;      off += align_up(nb * sizeof(int32_t));
    l.part_lse = off;      off += align_up((size_t)h->partial_slots * h->rows * sizeof(float));
    l.part_o = off;        off += align_up((size_t)h->partial_slots * h->rows * h->p.d_c * sizeof(uint16_t));
    // fp8 cache: the queries as two e4m3 terms, written by the decode's first kernel
    l.qx = off;
    if (h->p.kv_dtype == MLA_KV_FP8_E4M3_E8M0) off += align_up(nb * (size_t)h->rows * qx_row_bytes(h));
    l.total = off;
    return l;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int32_t kMaxTopk = 1 << 20;

// Workspace of a sparse run: the plan and partials of batch * s_q units of
// n_h rows.
struct SparseLayout {
    size_t seq_nsplit, seq_slot, part_lse, part_o, qx, total;
    int units, tiles, row_groups, workers, slots;
};

SparseLayout sparse_layout(const mla_decode_handle* h, int32_t batch, int32_t topk) {
    SparseLayout l{};
    l.units = (batch > 0 ? batch : 1) * h->p.s_q;
    l.tiles = (topk + mla::kPage - 1) / mla::kPage;
    l.row_groups = (h->p.n_h + mla::kRowsPerGroup - 1) / mla::kRowsPerGroup;
    // as many workgroups as the dense decode of this handle launches
    if (h->p.num_workers > 0) {
        l.workers = h->p.num_workers;
    } else {
        int w = h->num_workers * h->row_groups / l.row_groups;
        if (w >= 8) w = w / 8 * 8;
        l.workers = w < 1 ? 1 : (w > mla::kMaxWorkers ? mla::kMaxWorkers : w);
    }
    l.slots = l.workers > 1 ? 2 * (l.workers - 1) : 1;
    const size_t nu = (size_t)l.units;
    size_t off = 0;
    l.seq_nsplit = off;  off += align_up(nu * sizeof(int32_t));
    l.seq_slot = off;    off += align_up(nu * sizeof(int32_t));
    l.part_lse = off;    off += align_up((size_t)l.slots * h->p.n_h * sizeof(float));
    l.part_o = off;      off += align_up((size_t)l.slots * h->p.n_h * h->p.d_c * sizeof(uint16_t));
    l.qx = off;
    if (h->p.kv_dtype == MLA_KV_FP8_E4M3_E8M0) off += align_up(nu * (size_t)h->p.n_h * qx_row_bytes(h));
    l.total = off;
    return l;
}

mla_status_t check_run_pointers(const void* q, const void* kv_pages, const int32_t* block_table,
                                const int32_t* seq_lens, const float* out, const float* lse, const void* workspace) {
    if (!q || !kv_pages || !block_table || !seq_lens || !out || !workspace) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(kv_pages, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, kAlign)) return MLA_ERR_INVALID_ARGUMENT;
    return MLA_OK;
}

// The decode arguments a dense and a sparse run share.
mla::DecodeArgs decode_args(const mla_decode_handle* h, const void* q, const void* kv_pages,
                            const int32_t* block_table, const int32_t* seq_lens, float* out, float* lse,
                            const mla::PlanView& plan) {
    mla::DecodeArgs da{};
    da.q = (const uint16_t*)q;
    da.kv = (const uint8_t*)kv_pages;
    da.block_table = block_table;
    da.seq_lens = seq_lens;
    da.out = out;
    da.lse = lse;
    da.plan = plan;
    da.qx = nullptr;
    da.page_bytes = (int64_t)h->p.block_size * (int64_t)mla_kv_row_stride(h->p.kv_dtype, h->p.d_c, h->p.d_r);
    da.page_size = h->p.block_size;
    da.n_h = h->p.n_h;
    da.d_c = h->p.d_c;
    da.max_blocks = h->p.max_blocks_per_seq;
    da.overhead_units = kOverheadUnits;
    da.min_quota = kMinQuota;
    da.scale_log2 = h->p.softmax_scale * 1.4426950408889634f;
    da.sparse_topk = 0;
    da.sparse_indices = nullptr;
    da.sparse_sq = 1;
    return da;
}

mla_status_t validate_params(const mla_decode_params_t* p) {
    if (p->struct_size != (int32_t)sizeof(mla_decode_params_t)) return MLA_ERR_INVALID_ARGUMENT;
    if (p->max_batch < 1 || p->max_batch > (1 << 20)) return MLA_ERR_INVALID_ARGUMENT;
    if (p->s_q < 1 || p->s_q > 8) return MLA_ERR_INVALID_ARGUMENT;
    if (p->n_h < 32 || p->n_h > 1024 || p->n_h % 32 != 0) return MLA_ERR_INVALID_ARGUMENT;
    if (p->d_c <= 0 || p->d_r < 0 || p->block_size <= 0) return MLA_ERR_INVALID_ARGUMENT;
    if (p->max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARGUMENT;
    if ((int64_t)p->max_blocks_per_seq * p->block_size > (int64_t)1 << 30) return MLA_ERR_INVALID_ARGUMENT;
    if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3_E8M0 && p->kv_dtype != MLA_KV_FP4_E2M1_E8M0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
    if (p->num_workers < 0 || p->num_workers > mla::kMaxWorkers) return MLA_ERR_INVALID_ARGUMENT;
    if ((p->flags & ~MLA_FLAG_KV_WITHIN_4GIB) != 0) return MLA_ERR_INVALID_ARGUMENT;
    if ((p->d_c + p->d_r) % 32 != 0 && p->kv_dtype != MLA_KV_BF16) return MLA_ERR_INVALID_ARGUMENT;
    // valid requests outside what this build instantiates: d_r = 64 and
    // d_c = 512, or d_c = 448 with the fp8 cache (the record's 528-byte row)
    if (p->d_r != mla::kDr) return MLA_ERR_UNSUPPORTED;
    if (p->d_c != mla::kDc && !(p->d_c == mla::kDcNarrow && p->kv_dtype == MLA_KV_FP8_E4M3_E8M0))
        return MLA_ERR_UNSUPPORTED;
    if (p->block_size < 16 || p->block_size > 256 || (p->block_size & (p->block_size - 1)) != 0)
        return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_decode_abi_version(void) { return MLA_DECODE_ABI_VERSION; }

const char* mla_status_string(mla_status_t s) {
    switch (s) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
        case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
        case MLA_ERR_HIP: return "MLA_ERR_HIP";
        case MLA_ERR_OUT_OF_MEMORY: return "MLA_ERR_OUT_OF_MEMORY";
    }
    return "MLA_ERR_UNKNOWN";
}

size_t mla_kv_row_bytes(int32_t kv_dtype, int32_t d_c, int32_t d_r) {
    if (d_c <= 0 || d_r < 0) return 0;
    const size_t d = (size_t)d_c + (size_t)d_r;
    if (kv_dtype == MLA_KV_BF16) return 2 * d;
    if (kv_dtype == MLA_KV_FP8_E4M3_E8M0) return d % 32 ? 0 : d + d / 32;
    if (kv_dtype == MLA_KV_FP4_E2M1_E8M0) return d % 32 ? 0 : d / 2 + d / 16;
    return 0;
}

size_t mla_kv_row_stride(int32_t kv_dtype, int32_t d_c, int32_t d_r) {
    const size_t b = mla_kv_row_bytes(kv_dtype, d_c, d_r);
    return (b + 15) / 16 * 16;
}

mla_status_t mla_decode_init(const mla_decode_params_t* params, mla_decode_handle_t* out) {
    if (out) *out = nullptr;
    if (!params || !out) return MLA_ERR_INVALID_ARGUMENT;
    const mla_status_t v = validate_params(params);
    if (v != MLA_OK) return v;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MLA_ERR_UNSUPPORTED;

    mla_decode_handle* h = new (std::nothrow) mla_decode_handle;
    if (!h) return MLA_ERR_OUT_OF_MEMORY;
    std::memset(h, 0, sizeof(*h));
    h->p = *params;
    h->device = dev;
    h->compute_units = prop.multiProcessorCount;
    h->rows = params->s_q * params->n_h;
    h->row_groups = (h->rows + mla::kRowsPerGroup - 1) / mla::kRowsPerGroup;
    if (params->num_workers > 0) {
        h->num_workers = params->num_workers;
    } else {
        // one workgroup per compute unit (the kernel holds a CU's LDS); keep the
        // row groups of one worker on one XCD by using a multiple of 8 workers
        int w = h->compute_units / h->row_groups;
        if (w >= 8) w = w / 8 * 8;
        h->num_workers = w < 1 ? 1 : (w > mla::kMaxWorkers ? mla::kMaxWorkers : w);
    }
    h->partial_slots = h->num_workers > 1 ? 2 * (h->num_workers - 1) : 1;
    // the device's no-alloc scratch: its address is taken here, once per
    // device, with the device current
    if (mla::scratch_address(dev, &h->scratch) != hipSuccess) {
        delete h;
        return MLA_ERR_HIP;
    }
    const char* log = std::getenv("MLA_DECODE_LOG");
    if (log && log[0] == '1') {
        std::fprintf(stderr, "[mla_decode] device %d (%s) CUs=%d rows=%d row_groups=%d workers=%d kv=%s\n",
                     dev, prop.gcnArchName, h->compute_units, h->rows, h->row_groups, h->num_workers,
                     params->kv_dtype == MLA_KV_BF16 ? "bf16" : params->kv_dtype == MLA_KV_FP8_E4M3_E8M0 ? "fp8" : "fp4");
    }
    *out = h;
    return MLA_OK;
}

mla_status_t mla_decode_workspace_size(mla_decode_handle_t h, int32_t batch, size_t* bytes) {
    if (!h || !bytes) return MLA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || batch > h->p.max_batch) return MLA_ERR_INVALID_ARGUMENT;
    *bytes = layout(h, batch).total;
    return MLA_OK;
}

mla_status_t mla_decode_set_profile_events(mla_decode_handle_t h, void* ev_start, void* ev_stop) {
    if (!h) return MLA_ERR_INVALID_ARGUMENT;
    if ((ev_start == nullptr) != (ev_stop == nullptr)) return MLA_ERR_INVALID_ARGUMENT;
    h->ev_start = (hipEvent_t)ev_start;
    h->ev_stop = (hipEvent_t)ev_stop;
    return MLA_OK;
}

mla_status_t mla_decode_get_info(mla_decode_handle_t h, int32_t* num_workers, int32_t* row_groups,
                                 int32_t* compute_units) {
    if (!h) return MLA_ERR_INVALID_ARGUMENT;
    if (num_workers) *num_workers = h->num_workers;
    if (row_groups) *row_groups = h->row_groups;
    if (compute_units) *compute_units = h->compute_units;
    return MLA_OK;
}

mla_status_t mla_decode_free(mla_decode_handle_t h) {
    delete h;
    return MLA_OK;
}

mla_status_t mla_decode_run(mla_decode_handle_t h, const void* q, const void* kv_pages,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* hip_stream) {
    if (!h) return MLA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || batch > h->p.max_batch) return MLA_ERR_INVALID_ARGUMENT;
    if (batch == 0) return MLA_OK;
    const mla_status_t v = check_run_pointers(q, kv_pages, block_table, seq_lens, out, lse, workspace);
    if (v != MLA_OK) return v;
    const WsLayout l = layout(h, batch);
    if (workspace_bytes < l.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    uint8_t* ws = (uint8_t*)workspace;
    mla::PlanView plan{};
    plan.seq_nsplit = (int32_t*)(ws + l.seq_nsplit);
    plan.seq_slot = (int32_t*)(ws + l.seq_slot);
    plan.part_lse = (float*)(ws + l.part_lse);
    plan.slots = h->partial_slots;
    plan.part_o = (uint16_t*)(ws + l.part_o);
    hipStream_t stream = (hipStream_t)hip_stream;

    mla::DecodeArgs da = decode_args(h, q, kv_pages, block_table, seq_lens, out, lse, plan);
    da.batch = batch;
    da.s_q = h->p.s_q;
    da.num_workers = h->num_workers;
    // profile events (both or neither) take the decode kernel's own timestamps
    const hipEvent_t e0 = h->ev_start && h->ev_stop ? h->ev_start : nullptr;
    const hipEvent_t e1 = e0 ? h->ev_stop : nullptr;
    hipError_t e = hipSuccess;
    if (h->p.kv_dtype == MLA_KV_BF16) {
        e = mla::launch_decode_bf16(da, h->row_groups, stream, e0, e1);
    } else if (h->p.kv_dtype == MLA_KV_FP8_E4M3_E8M0) {
        da.qx = ws + l.qx;
        e = mla::launch_quantize_q_mx(da, stream);
        if (e == hipSuccess) e = mla::launch_decode_fp8_mx(da, h->row_groups, stream, e0, e1);
    } else {
        e = mla::launch_decode_fp4(da, h->row_groups, stream, e0, e1);
    }
    if (e != hipSuccess) return MLA_ERR_HIP;

    mla::CombineArgs ca{};
    ca.plan = plan;
    ca.out = out;
    ca.lse = lse;
    ca.batch = batch;
    ca.rows = h->rows;
    ca.d_c = h->p.d_c;
    if (mla::launch_combine(ca, h->num_workers, stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

mla_status_t mla_decode_run_noalloc(mla_decode_handle_t h, const void* q, const void* kv_pages,
                                    const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                    float* out, float* lse, void* hip_stream) {
    if (!h) return MLA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || batch > h->p.max_batch) return MLA_ERR_INVALID_ARGUMENT;
    if (!h->scratch) return MLA_ERR_HIP;
    // the plan and partials of this handle and batch must fit the scratch
    if (layout(h, batch).total > mla::kNoAllocScratchBytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
    // the scratch's device address (taken at init), never the array's name;
    // nothing in it needs clearing: the decode writes every plan record and
    // partial before the combine reads it
    return mla_decode_run(h, q, kv_pages, block_table, seq_lens, batch, out, lse, h->scratch,
                          mla::kNoAllocScratchBytes, hip_stream);
}

mla_status_t mla_decode_sparse_workspace_size(mla_decode_handle_t h, int32_t batch, int32_t topk, size_t* bytes) {
    if (!h || !bytes) return MLA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || batch > h->p.max_batch) return MLA_ERR_INVALID_ARGUMENT;
    if (topk < 1 || topk > kMaxTopk) return MLA_ERR_INVALID_ARGUMENT;
    *bytes = sparse_layout(h, batch, topk).total;
    return MLA_OK;
}

mla_status_t mla_decode_sparse_run(mla_decode_handle_t h, const void* q, const void* kv_pages,
                                   const int32_t* block_table, const int32_t* seq_lens, const int32_t* indices,
                                   int32_t topk, int32_t batch, float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
    if (!h) return MLA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || batch > h->p.max_batch) return MLA_ERR_INVALID_ARGUMENT;
    if (topk < 1 || topk > kMaxTopk) return MLA_ERR_INVALID_ARGUMENT;
    if (batch == 0) return MLA_OK;
    const mla_status_t v = check_run_pointers(q, kv_pages, block_table, seq_lens, out, lse, workspace);
    if (v != MLA_OK) return v;
    if (!indices || !aligned(indices, 4)) return MLA_ERR_INVALID_ARGUMENT;
    const SparseLayout l = sparse_layout(h, batch, topk);
    if (workspace_bytes < l.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    uint8_t* ws = (uint8_t*)workspace;
    mla::PlanView plan{};
    plan.seq_nsplit = (int32_t*)(ws + l.seq_nsplit);
    plan.seq_slot = (int32_t*)(ws + l.seq_slot);
    plan.part_lse = (float*)(ws + l.part_lse);
    plan.slots = l.slots;
    plan.part_o = (uint16_t*)(ws + l.part_o);
    hipStream_t stream = (hipStream_t)hip_stream;
    // every (sequence, query position) is a unit of n_h rows attending to its own tokens
    mla::DecodeArgs da = decode_args(h, q, kv_pages, block_table, seq_lens, out, lse, plan);
    da.batch = l.units;
    da.s_q = 1;
    da.num_workers = l.workers;
    da.sparse_topk = topk;
    da.sparse_indices = indices;
    da.sparse_sq = h->p.s_q;
    const hipEvent_t e0 = h->ev_start && h->ev_stop ? h->ev_start : nullptr;
    const hipEvent_t e1 = e0 ? h->ev_stop : nullptr;
    const bool window = (h->p.flags & MLA_FLAG_KV_WITHIN_4GIB) != 0;
    hipError_t e = hipSuccess;
    if (h->p.kv_dtype == MLA_KV_BF16) {
        e = mla::launch_decode_bf16_sparse(da, l.row_groups, stream, e0, e1, window);
    } else if (h->p.kv_dtype == MLA_KV_FP8_E4M3_E8M0) {
        da.qx = ws + l.qx;
        e = mla::launch_quantize_q_mx(da, stream);
        if (e == hipSuccess) e = mla::launch_decode_fp8_mx_sparse(da, l.row_groups, stream, e0, e1, window);
    } else {
        e = mla::launch_decode_fp4_sparse(da, l.row_groups, stream, e0, e1, window);
    }
    if (e != hipSuccess) return MLA_ERR_HIP;

    mla::CombineArgs ca{};
    ca.plan = plan;
    ca.out = out;
    ca.lse = lse;
    ca.batch = l.units;
    ca.rows = h->p.n_h;
    ca.d_c = h->p.d_c;
    if (mla::launch_combine(ca, l.workers, stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

}  // extern "C"
