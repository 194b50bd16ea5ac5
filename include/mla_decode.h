/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) MLA latent-cache decode library.
 *
 * Operation ("DeepSeek R1 Architecture & Deployment Guide", section 1.1):
 * every cached token holds ONE row shared by all attention heads, the
 * concatenation of the compressed latent c (d_c values) and the decoupled,
 * already-rotated RoPE key k_R (d_r values).  With the key up-projection
 * absorbed into the query and the value up-projection absorbed into the
 * output projection (applied by the caller afterwards), head h of query j of
 * sequence b computes
 *
 *     s_t  = softmax_scale * ( q_abs . c_t + q_R . k_R_t )      for visible t
 *     out  = sum_t softmax(s)_t * c_t                            (d_c floats)
 *     lse  = ln sum_t exp(s_t)
 *
 * The cache is paged: the "DeepSeek-R1" record, engine kernel constraint (1),
 * instantiates MLA decode per page-block size and names 64; constraint (2)
 * gives the FP8 row (e4m3 codes over every dimension, RoPE included, plus one
 * e8m0 scale per 32 codes).
 *
 * Conventions shared by every entry point:
 *   - All device pointers are plain device addresses owned by the caller
 *     (this library allocates no device memory).  Host pointers are marked.
 *   - No entry point aborts, prints or throws; every failure is a status.
 *   - Entry points that launch work are asynchronous on the caller's HIP
 *     stream (passed as void*, NULL = the default stream) and never
 *     synchronise; a device fault surfaces at the caller's next sync.
 *   - The library is silent; MLA_DECODE_LOG=1 in the environment makes
 *     mla_decode_init print the chosen plan to stderr.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_DECODE_ABI_VERSION 1

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARGUMENT = 1,    /* null/misaligned pointer, bad size or field */
    MLA_ERR_UNSUPPORTED = 2,         /* valid request this build does not implement */
    MLA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < mla_decode_workspace_size */
    MLA_ERR_HIP = 4,                 /* a HIP runtime call failed (incl. no device) */
    MLA_ERR_OUT_OF_MEMORY = 5        /* host allocation of the handle failed */
} mla_status_t;

/* Cache row formats.
 * MLA_KV_BF16: a row is d_c + d_r bf16 values, c first then k_R
 *   (guide section 1.1 concat order); row stride 2*(d_c+d_r) bytes.
 * MLA_KV_FP8_E4M3_E8M0: a row is D = d_c + d_r e4m3fn codes (c then k_R),
 *   then D/32 e8m0 scale bytes, scale g multiplying codes 32g..32g+31
 *   ("DeepSeek-R1" record, constraint (2)); value = e4m3(code) * 2^(e-127);
 *   the row is padded to a 16-byte stride (608 bytes at D = 576; 528 bytes,
 *   no padding, at D = 512).  Padding bytes are never read. */
typedef enum mla_kv_dtype {
    MLA_KV_BF16 = 0,
    MLA_KV_FP8_E4M3_E8M0 = 1,   /* D e4m3 codes, then one e8m0 scale per 32 ("DeepSeek-R1"
                                   record, engine kernel constraint (2))                   */
    MLA_KV_FP4_E2M1_E8M0 = 2    /* D/2 bytes of e2m1 codes (element 2i in the low nibble of
                                   byte i), then one e8m0 scale per 16: a reading of the
                                   same constraint's 288-byte fp4 row at 512 dims          */
} mla_kv_dtype_t;

/* Flags for mla_decode_params_t.flags */
#define MLA_FLAG_NONE 0
/* The caller guarantees that every page it will pass lies within the first
 * 0xFFFFF000 bytes (4 GiB - 4 KiB) from the kv_pages pointer of each run
 * call.  The sparse decode then gathers rows with 32-bit offsets, which
 * issue faster; without the flag it uses 64-bit addresses.  A row past that
 * window under the flag reads as zeros (a wrong result, never an access
 * outside the window).  The dense decode is not affected. */
#define MLA_FLAG_KV_WITHIN_4GIB 1

typedef struct mla_decode_params {
    int32_t struct_size;        /* = sizeof(mla_decode_params_t); guards ABI evolution     */
    int32_t max_batch;          /* upper bound on the run-time batch, >= 1                  */
    int32_t s_q;                /* queries per sequence (1 = plain decode, 2 = MTP), 1..8   */
    int32_t n_h;                /* heads, a multiple of 32, <= 1024                         */
    int32_t d_c;                /* latent width; this build: 512, or 448 with the FP8 cache
                                   (D = 512: the record's own 528-byte row, constraint (2));
                                   other widths give MLA_ERR_UNSUPPORTED                   */
    int32_t d_r;                /* RoPE key width; this build: 64                           */
    int32_t block_size;         /* tokens per page block: a power of two, 16..256 (64 is the
                                   usual size, 32 that of a ratio-2 compressed layer:
                                   "DeepSeek-R1" record, engine kernel constraint (1));
                                   other sizes give MLA_ERR_UNSUPPORTED                    */
    int32_t max_blocks_per_seq; /* row stride (in entries) of block_table, >= 1             */
    int32_t kv_dtype;           /* an mla_kv_dtype_t                                        */
    float   softmax_scale;      /* multiplies q.row; finite and > 0 (e.g. 1/sqrt(192))      */
    int32_t num_workers;        /* 0 = one worker per compute unit (chosen at init);
                                   > 0 forces that many context-split workers (tests,
                                   sweeps); at most 4096                                   */
    int32_t flags;              /* MLA_FLAG_*                                               */
} mla_decode_params_t;

typedef struct mla_decode_handle* mla_decode_handle_t;

/* mla_decode_init -- validate params, query the current HIP device, choose the
 * kernel instance and the split plan bounds.
 *   params : host pointer, read only during the call.
 *   out    : host pointer; receives a host-only handle (immutable except
 *            through mla_decode_set_profile_events) on MLA_OK, NULL otherwise.
 * Every field is validated on the host BEFORE any HIP call
 * (MLA_ERR_INVALID_ARGUMENT / MLA_ERR_UNSUPPORTED).  Then the current device
 * must be a gfx950; otherwise MLA_ERR_UNSUPPORTED, and MLA_ERR_HIP if no
 * device can be queried.  The handle is bound to the device current at init. */
mla_status_t mla_decode_init(const mla_decode_params_t* params, mla_decode_handle_t* out);

/* mla_decode_workspace_size -- device workspace bytes that mla_decode_run needs
 * for `batch` sequences (0 <= batch <= max_batch).  `bytes` is a host pointer.
 * The workspace holds the per-call work plan and the split-KV partial results
 * (fp16 normalised outputs and fp32 LSEs of every context split); for the FP8
 * cache also the queries as two e4m3 terms (two cache rows per query row:
 * 1216 bytes at d_c = 512, 1056 at d_c = 448). */
mla_status_t mla_decode_workspace_size(mla_decode_handle_t h, int32_t batch, size_t* bytes);

/* mla_decode_run -- one decode step for `batch` sequences, all heads, all queries.
 *   q           : device, bf16 [batch][s_q][n_h][d_c + d_r], each row q_abs then q_R
 *                 (scale not applied), 16-byte aligned.
 *   kv_pages    : device, [num_pages][block_size][row_stride] in kv_dtype's row
 *                 format (see mla_kv_row_stride), 16-byte aligned.
 *   block_table : device, int32 [batch][max_blocks_per_seq]; entry [b][p] is the
 *                 physical page of logical page p of sequence b.  Entries
 *                 p < ceil(seq_lens[b] / block_size) must be valid page indices
 *                 (precondition, not checked on the device).  The decode works
 *                 on 64-token tiles: with block_size < 64 it may also read the
 *                 entries up to the end of the sequence's last tile (within
 *                 max_blocks_per_seq), but never dereferences them.
 *   seq_lens    : device, int32 [batch]; L_b counts every cached token including
 *                 the s_q new ones.  Query j of sequence b sees tokens
 *                 0 .. L_b - s_q + j (causal over the last s_q positions).
 *                 Precondition 0 <= L_b <= block_size * max_blocks_per_seq; a
 *                 query that sees no token gets out = 0 and lse = -inf.
 *   batch       : 0 <= batch <= max_batch; 0 is a no-op.
 *   out         : device, fp32 [batch][s_q][n_h][d_c], 16-byte aligned.
 *   lse         : device, fp32 [batch][s_q][n_h] natural-log LSE, or NULL.
 *   workspace   : device, >= mla_decode_workspace_size(batch) bytes, 256-byte
 *                 aligned; contents need not be initialised and are scratch
 *                 after the call.  Concurrent runs need distinct workspaces.
 *   hip_stream  : hipStream_t as void*, NULL = default stream.
 * Tail slots after a sequence's last token, unused pages and row padding are
 * never read, whatever they hold.
 *
 * Value range (precondition).  The products run on matrix cores with fp32
 * accumulation.  BF16 cache: Q.K^T takes the values as they are (bf16 MFMA).
 * FP8 cache: Q.K^T multiplies the cache's own e4m3 codes and e8m0 scales by
 * the query split into two e4m3 terms with one e8m0 scale per 32
 * (q ~ q_hi + q_lo, q_lo encoding the residual; block-scaled fp8 MFMA).
 * FP4 cache: Q.K^T takes the dequantised values converted to fp16.  P.V takes
 * the dequantised (bf16: the raw) values converted to fp16 for every format.
 * Every decoded cache element x of a visible token must therefore satisfy
 * |x| < 65520 (every finite bf16 value up to 65280 in magnitude; an fp8 code
 * times its scale up to 61440); a larger one becomes infinite and the output
 * of its rows NaN.  Magnitudes below 2^-14 keep fewer significant bits, and
 * those below 2^-25 become zero; both are far below the output tolerance
 * whenever the values that dominate a row are of ordinary size.  The
 * softmax weights that P.V takes are fp16 as well, relative to a running
 * maximum of the row's scores that is raised only when a score exceeds it
 * by a large margin: a token whose weight is below 2^-17 (FP8 and FP4
 * caches) or 2^-25 (BF16) of the weight at that maximum contributes nothing.
 *
 * Split-KV: the context of a sequence is split across workers, and each
 * split's normalised partial output is stored as fp16 (relative rounding
 * 2^-11) before the fp32 log-sum-exp merge, so results depend on the split
 * count (the handle's worker count) at that level, far inside the stated
 * tolerance.  Repeated calls with the same inputs and handle are bitwise
 * identical. */
mla_status_t mla_decode_run(mla_decode_handle_t h,
                            const void* q,
                            const void* kv_pages,
                            const int32_t* block_table,
                            const int32_t* seq_lens,
                            int32_t batch,
                            float* out,
                            float* lse,
                            void* workspace,
                            size_t workspace_bytes,
                            void* hip_stream);

/* mla_decode_run_noalloc -- mla_decode_run without a caller workspace, for
 * callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * kernels, same arguments and results as mla_decode_run, minus workspace and
 * workspace_bytes: the plan and split partials go to a scratch array that the
 * library keeps in device memory, MLA_NOALLOC_SCRATCH_BYTES per GPU (each GPU
 * it runs on holds its own copy from the first init on that GPU until the
 * process ends).  Nothing is allocated per call.
 *   Returns MLA_ERR_WORKSPACE_TOO_SMALL when mla_decode_workspace_size(h,
 *   batch) exceeds MLA_NOALLOC_SCRATCH_BYTES.  With the default worker count
 *   on a 256-CU device the plan and partials take under 68 MB for every
 *   n_h * s_q, so bf16 and fp4 calls always fit; the FP8 cache adds its
 *   two-term query rows (batch * s_q * n_h * 1216 bytes), which fit up to
 *   about 400 sequences at n_h = 128, s_q = 1.  Large forced worker counts
 *   may not fit.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (other streams, other threads) race and give wrong
 *   results; calls ordered on one stream are safe. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
mla_status_t mla_decode_run_noalloc(mla_decode_handle_t h,
                                    const void* q,
                                    const void* kv_pages,
                                    const int32_t* block_table,
                                    const int32_t* seq_lens,
                                    int32_t batch,
                                    float* out,
                                    float* lse,
                                    void* hip_stream);

/* mla_decode_sparse_workspace_size -- device workspace bytes that
 * mla_decode_sparse_run needs for `batch` sequences (0 <= batch <= max_batch)
 * and index lists of `topk` entries (1 <= topk <= 2^20).  `bytes` is a host
 * pointer.  The workspace holds the work plan and split partials of
 * batch * s_q query units (and, for the FP8 cache, their two-term query
 * rows); its size does not depend on topk (the decode reads the index lists
 * itself, nothing per entry is stored). */
mla_status_t mla_decode_sparse_workspace_size(mla_decode_handle_t h, int32_t batch, int32_t topk,
                                              size_t* bytes);

/* mla_decode_sparse_run -- one sparse (top-k) decode step: the "DeepSeek-V3.2"
 * model record keeps the latent cache of the dense decode but has a top-k
 * selector (index_topk = 2048) choose, for every query token, the tokens it
 * attends over.  Query j of sequence b computes the dense decode's result
 * over the tokens listed in indices[b][j] only.
 *   indices     : device, int32 [batch][s_q][topk], 4-byte aligned: logical
 *                 token positions of sequence b.  An entry takes part iff
 *                 0 <= t < L_b - s_q + 1 + j (the query's causal context);
 *                 padding such as -1, and any other value, is ignored.
 *                 Entries count as listed: a selector returns distinct
 *                 positions (a repeated one would count twice).  A query
 *                 with no valid entry gets out = 0 and lse = -inf.
 *   topk        : entries per list, 1 .. 2^20.
 *   every other argument as for mla_decode_run (the handle's s_q, n_h,
 *   block_size and softmax scale apply); workspace >=
 *   mla_decode_sparse_workspace_size(batch, topk) bytes.
 * Every cache format is served.  Two kernels are enqueued on the stream:
 * the decode, which reads the index lists and the block table itself and
 * gathers the rows, and the split combine.  Only the listed rows are read;
 * the block-table entries of listed valid tokens must be valid pages. */
mla_status_t mla_decode_sparse_run(mla_decode_handle_t h,
                                   const void* q,
                                   const void* kv_pages,
                                   const int32_t* block_table,
                                   const int32_t* seq_lens,
                                   const int32_t* indices,
                                   int32_t topk,
                                   int32_t batch,
                                   float* out,
                                   float* lse,
                                   void* workspace,
                                   size_t workspace_bytes,
                                   void* hip_stream);

/* mla_decode_set_profile_events -- measurement hook.  When both are non-NULL,
 * later runs have ev_start and ev_stop take the start and end timestamps of
 * the split-KV decode kernel's own dispatch (not the combine) on the run's
 * stream, so their elapsed time is that kernel's duration.
 * Both are hipEvent_t passed as void*, owned by the caller.  NULL, NULL turns
 * the hook off.  Not thread-safe with concurrent runs on the same handle. */
mla_status_t mla_decode_set_profile_events(mla_decode_handle_t h, void* ev_start, void* ev_stop);

/* mla_decode_get_info -- host copies of the plan bounds chosen at init.
 * Any output pointer may be NULL. */
mla_status_t mla_decode_get_info(mla_decode_handle_t h, int32_t* num_workers,
                                 int32_t* row_groups, int32_t* compute_units);

/* mla_decode_free -- release the host handle (no device memory is held).
 * NULL is accepted. */
mla_status_t mla_decode_free(mla_decode_handle_t h);

/* mla_kv_row_bytes -- payload bytes of one cached row: 2*(d_c+d_r) for bf16,
 * (d_c+d_r) + (d_c+d_r)/32 for FP8 (594 at 576 dims, 528 at 512 dims).
 * Returns 0 for an invalid combination. */
size_t mla_kv_row_bytes(int32_t kv_dtype, int32_t d_c, int32_t d_r);

/* mla_kv_row_stride -- row stride in a page: the payload rounded up to 16 bytes
 * (1152 bf16, 608 FP8 at 576 dims).  Returns 0 for an invalid combination. */
size_t mla_kv_row_stride(int32_t kv_dtype, int32_t d_c, int32_t d_r);

/* mla_status_string -- static, never NULL. */
const char* mla_status_string(mla_status_t s);

/* mla_decode_abi_version -- MLA_DECODE_ABI_VERSION of the built library. */
int32_t mla_decode_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H */
