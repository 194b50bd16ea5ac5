"""GPU parity: the HIP decode (through the C ABI) against the float64 oracle on
the same seeded bytes.  Element-by-element at reduced sizes that still span
several pages, splits and ragged tails; on sampled sequences at the full
workload sizes, in the launch configuration the bench times."""

import dataclasses

import numpy as np
import pytest
import torch

from mla_inputs import SPECS, WorkloadSpec, make_workload, to_torch
from gpu_helpers import run_gpu, oracle, assert_parity, make_decoder, say

pytestmark = pytest.mark.gpu

SMALL = ["single_1k_small", "paged_b32_small", "long_ctx_b4_small", "fp8_b64_small", "mtp2_b128_small",
         "fp4_b64_small", "fp8_b64_d512_small"]


@pytest.mark.parametrize("name", SMALL)
def test_parity_small_all_elements(name):
    w = make_workload(name)
    out, lse = run_gpu(w)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("workers", [1, 3, 16, 300])
def test_parity_small_any_split(name, workers):
    # forcing the number of context splits exercises the planner and combine
    w = make_workload(name)
    out, lse = run_gpu(w, num_workers=workers)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


FULL_SAMPLES = {
    "single_1k": None,
    "paged_b32": [0, 7, 31],
    "long_ctx_b4": [0, 2],
    "fp8_b64": [0, 33, 63],
    "mtp2_b128": [0, 64, 127],
    "fp4_b64": [0, 33, 63],
    "fp8_b64_d512": [0, 33, 63],
}


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_parity_full_size_sampled(name):
    w = make_workload(name)
    batches = FULL_SAMPLES[name]
    if batches is None:
        batches = list(range(w.spec.batch))
    # include the longest sequence
    batches = sorted(set(batches) | {int(np.argmax(w.seq_lens))})
    out, lse = run_gpu(w)
    ro, rl = oracle(w, batches=batches)
    assert_parity(w, out, lse, ro, rl, batches=batches)
    # every output of every sequence is finite and every lse is finite
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def _identity_layout(w):
    """Same logical cache, pages stored in logical order (identity block table)."""
    pages = (w.seq_lens.astype(np.int64) + 63) // 64
    rows = [w.block_table[b, :pages[b]] for b in range(w.spec.batch)]
    order = np.concatenate(rows)
    pool2 = w.pool[order].copy()
    bt2 = np.full_like(w.block_table, -1)
    off = 0
    for b in range(w.spec.batch):
        bt2[b, :pages[b]] = np.arange(off, off + pages[b])
        off += pages[b]
    return dataclasses.replace(w, pool=pool2, block_table=bt2)


@pytest.mark.parametrize("name", ["paged_b32_small", "fp8_b64_small", "mtp2_b128_small", "fp8_b64_d512_small"])
def test_paged_equals_identity_bitwise(name):
    w = make_workload(name)
    w2 = _identity_layout(w)
    o1, l1 = run_gpu(w, num_workers=7)
    o2, l2 = run_gpu(w2, num_workers=7)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def _repage(w, page: int, seed: int):
    """The same logical cache laid out in page blocks of `page` tokens: each
    sequence's rows copied in order into a seeded permutation of physical
    blocks, with NaN-poisoned tails and spare blocks.  The decode works on
    64-token tiles whatever the block size, so its output must not change by
    a single bit."""
    s = w.spec
    rng = np.random.default_rng(seed)
    lens = w.seq_lens.astype(np.int64)
    nb = (lens + page - 1) // page
    n_used = int(nb.sum())
    pool_pages = n_used + 3
    phys = rng.permutation(pool_pages)[:n_used]
    pool = np.empty((pool_pages, page) + w.pool.shape[2:], dtype=w.pool.dtype)
    if s.kv_dtype == "bf16":
        pool[...] = 0x7FC0
    elif s.kv_dtype == "fp8":
        pool[...] = 0xFF
        pool[..., :s.d] = 0x7F
    else:
        pool[...] = 0xFF
        pool[..., :s.d // 2] = 0x77
    bt = np.full((s.batch, max(int(nb.max()), 1)), -1, dtype=np.int32)
    off = 0
    for b in range(s.batch):
        n64 = (int(lens[b]) + 63) // 64
        rows = w.pool[w.block_table[b, :n64]].reshape((n64 * 64,) + w.pool.shape[2:])[:lens[b]]
        for k in range(int(nb[b])):
            seg = rows[k * page:(k + 1) * page]
            pool[phys[off + k], :len(seg)] = seg
            bt[b, k] = phys[off + k]
        off += int(nb[b])
    spec = dataclasses.replace(s, page=page, name=f"{s.name}_p{page}")
    return dataclasses.replace(w, spec=spec, pool=pool, block_table=bt)


@pytest.mark.parametrize("name", ["paged_b32_small", "fp8_b64_small", "mtp2_b128_small", "long_ctx_b4_small",
                                  "fp4_b64_small", "fp8_b64_d512_small"])
@pytest.mark.parametrize("page", [16, 32, 128, 256])
def test_page_block_sizes(name, page):
    # page blocks other than 64 ("DeepSeek-R1" record, constraint (1): 32 for
    # a compressed layer): bitwise the 64-token result, and the oracle's
    # result through its own gather at that block size
    w64 = make_workload(name)
    w = _repage(w64, page, seed=page)
    o64, l64 = run_gpu(w64, num_workers=7)
    o, l = run_gpu(w, num_workers=7)
    np.testing.assert_array_equal(o, o64)
    np.testing.assert_array_equal(l, l64)
    ro, rl = oracle(w)
    assert_parity(w, o, l, ro, rl)


@pytest.mark.parametrize("name,page", [("paged_b32", 32), ("fp8_b64", 128)])
def test_page_block_sizes_full_size_sampled(name, page):
    # a full-size workload generated at another block size, default plan
    w = make_workload(dataclasses.replace(SPECS[name], page=page, name=f"{name}_p{page}"))
    batches = sorted({0, w.spec.batch // 2, int(np.argmax(w.seq_lens))})
    out, lse = run_gpu(w)
    ro, rl = oracle(w, batches=batches)
    assert_parity(w, out, lse, ro, rl, batches=batches)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("name", ["long_ctx_b4_small", "fp8_b64_small"])
def test_repeat_runs_bitwise_identical(name):
    w = make_workload(name)
    t = to_torch(w, torch.device("cuda:0"))
    dec = make_decoder(w)
    o1, l1 = run_gpu(w, tensors=t, dec=dec)
    o2, l2 = run_gpu(w, tensors=t, dec=dec)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("name", ["paged_b32_small", "fp8_b64_small", "fp4_b64_small"])
def test_unread_bytes_do_not_matter(name):
    # rewrite every byte the decode must not read (tails, spare pages, padding)
    w = make_workload(name)
    pages = (w.seq_lens.astype(np.int64) + 63) // 64
    used = np.zeros(w.pool.shape[:2], dtype=bool)
    for b in range(w.spec.batch):
        for t in range(int(w.seq_lens[b])):
            used[w.block_table[b, t // 64], t % 64] = True
    pool2 = w.pool.copy()
    pool2[~used] = 0x5A5A if w.spec.kv_dtype == "bf16" else 0xFF
    if w.spec.kv_dtype == "fp8":
        pool2[:, :, 594:] = 0x7F
    if w.spec.kv_dtype == "fp4":
        pool2[:, :, 324:] = 0x7F                      # row padding
    w2 = dataclasses.replace(w, pool=pool2)
    o1, l1 = run_gpu(w, num_workers=5)
    o2, l2 = run_gpu(w2, num_workers=5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


EDGE = [
    # one token, a page multiple, one past a page, causal s_q=2 with L = 1 (query 0 sees nothing)
    WorkloadSpec("edge_lens", 6, ("fixed", (1, 64, 65, 128, 129, 3)), spare_pages=4, seed=11),
    WorkloadSpec("edge_mtp", 5, ("fixed", (1, 2, 64, 65, 200)), s_q=2, spare_pages=4, seed=12),
    WorkloadSpec("edge_fp8", 4, ("fixed", (1, 63, 64, 700)), kv_dtype="fp8", spare_pages=4, seed=13,
                 outlier_p=0.01, outlier_mult=20.0),
    WorkloadSpec("edge_heads32", 3, ("fixed", (100, 5, 300)), n_h=32, spare_pages=2, seed=14),
    WorkloadSpec("edge_heads64_mtp", 3, ("fixed", (100, 5, 300)), n_h=64, s_q=2, spare_pages=2, seed=15),
    WorkloadSpec("edge_heads256", 2, ("fixed", (129, 640)), n_h=256, spare_pages=2, seed=16),
    WorkloadSpec("edge_mtp4", 3, ("fixed", (3, 66, 257)), s_q=4, spare_pages=2, seed=17),
    WorkloadSpec("edge_empty_seq", 3, ("fixed", (0, 70, 0)), spare_pages=2, seed=18),
    # flat softmax (q = 0, or nearly): every visible token weighs the same, so
    # a token wrongly counted or dropped by a mask moves the output by about
    # 1/n, far past the tolerance
    WorkloadSpec("edge_flat_q0", 5, ("fixed", (1, 36, 100, 700, 1500)), q_scale=0.0, spare_pages=4, seed=19),
    WorkloadSpec("edge_flat_q0_fp8", 5, ("fixed", (1, 36, 100, 700, 1500)), q_scale=0.0, kv_dtype="fp8",
                 spare_pages=4, seed=20),
    WorkloadSpec("edge_flat_mtp", 4, ("fixed", (2, 37, 101, 701)), q_scale=0.02, s_q=2, spare_pages=4, seed=24),
    WorkloadSpec("edge_fp4", 4, ("fixed", (1, 63, 64, 700)), kv_dtype="fp4", spare_pages=4, seed=25,
                 outlier_p=0.01, outlier_mult=20.0),
    WorkloadSpec("edge_flat_q0_fp4", 5, ("fixed", (1, 36, 100, 700, 1500)), q_scale=0.0, kv_dtype="fp4",
                 spare_pages=4, seed=26),
]


@pytest.mark.parametrize("spec", EDGE, ids=[s.name for s in EDGE])
@pytest.mark.parametrize("workers", [0, 2])
def test_edge_cases(spec, workers):
    w = make_workload(spec)
    out, lse = run_gpu(w, num_workers=workers)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


def test_without_lse_output():
    w = make_workload("paged_b32_small")
    out, _ = run_gpu(w, with_lse=False)
    ro, rl = oracle(w)
    assert_parity(w, out, None, ro, rl)


def test_batch_zero_is_a_noop_and_errors_are_reported():
    import mla_latent_cache_decode_amd as m
    w = make_workload("paged_b32_small")
    dec = make_decoder(w)
    t = to_torch(w, torch.device("cuda:0"))
    lib = m.load_library()
    ws = dec.alloc_workspace(w.spec.batch)
    out = torch.zeros((w.spec.batch, 1, 128, 512), dtype=torch.float32, device="cuda")
    say("error paths")
    assert lib.mla_decode_run(dec._h, t["q"].data_ptr(), t["kv"].data_ptr(), t["block_table"].data_ptr(),
                              t["seq_lens"].data_ptr(), 0, out.data_ptr(), None, ws.data_ptr(), 0, None) == 0
    # workspace too small
    assert lib.mla_decode_run(dec._h, t["q"].data_ptr(), t["kv"].data_ptr(), t["block_table"].data_ptr(),
                              t["seq_lens"].data_ptr(), w.spec.batch, out.data_ptr(), None, ws.data_ptr(),
                              16, None) == m.MLA_ERR_WORKSPACE_TOO_SMALL
    # misaligned output
    assert lib.mla_decode_run(dec._h, t["q"].data_ptr(), t["kv"].data_ptr(), t["block_table"].data_ptr(),
                              t["seq_lens"].data_ptr(), w.spec.batch, out.data_ptr() + 4, None, ws.data_ptr(),
                              ws.numel(), None) == m.MLA_ERR_INVALID_ARGUMENT
    # batch above max_batch
    assert lib.mla_decode_run(dec._h, t["q"].data_ptr(), t["kv"].data_ptr(), t["block_table"].data_ptr(),
                              t["seq_lens"].data_ptr(), w.spec.batch + 1, out.data_ptr(), None, ws.data_ptr(),
                              ws.numel(), None) == m.MLA_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def _scale_later_tokens(w, start: int, log2_factor: int):
    """Scale every cached element of logical tokens >= start by 2^log2_factor,
    exactly: bf16 exponent field + k, or each fp8 row's e8m0 scale bytes + k.
    Scores against those tokens grow by the same factor, so a later block's
    max exceeds the first block's by far more than the lazy-max threshold."""
    pool2 = w.pool.copy()
    for b in range(w.spec.batch):
        for t in range(start, int(w.seq_lens[b])):
            pg, r = w.block_table[b, t // 64], t % 64
            if w.spec.kv_dtype == "bf16":
                row = pool2[pg, r].astype(np.int32)
                e = (row >> 7) & 0xFF
                nz = e != 0
                row[nz] += log2_factor << 7
                pool2[pg, r] = row.astype(np.uint16)
            else:
                d = w.spec.d
                pool2[pg, r, d:d + d // 32] += np.uint8(log2_factor)
    return dataclasses.replace(w, pool=pool2)


RISING = [
    WorkloadSpec("rising_bf16", 3, ("fixed", (700, 2000, 4100)), spare_pages=4, seed=21),
    WorkloadSpec("rising_mtp", 2, ("fixed", (900, 3000)), s_q=2, spare_pages=4, seed=22),
    WorkloadSpec("rising_fp8", 3, ("fixed", (700, 2000, 4100)), kv_dtype="fp8", spare_pages=4, seed=23),
]


@pytest.mark.parametrize("spec", RISING, ids=[s.name for s in RISING])
@pytest.mark.parametrize("workers", [0, 1, 7])
def test_rising_scores(spec, workers):
    # the softmax max of a segment moves up by ~8x mid-way: the kernels'
    # lazily kept max must still give the oracle's result
    w = _scale_later_tokens(make_workload(spec), start=300, log2_factor=3)
    out, lse = run_gpu(w, num_workers=workers)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)
