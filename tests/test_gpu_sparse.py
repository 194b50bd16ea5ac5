"""GPU parity of the sparse (top-k) decode ("DeepSeek-V3.2" record: a top-k
selector, index_topk 2048, picks each query's tokens) through the C ABI,
against the float64 sparse oracle on the same seeded bytes."""

import dataclasses

import numpy as np
import pytest
import torch

from mla_inputs import SPECS, WorkloadSpec, make_workload, to_torch
from oracle import mla_sparse_decode_ref
from gpu_helpers import assert_parity, make_decoder, run_gpu, say

pytestmark = pytest.mark.gpu


def run_sparse(w, num_workers=0, indices=None, with_lse=True, dec=None, tensors=None, flags=0):
    s = w.spec
    dev = torch.device("cuda:0")
    t = tensors if tensors is not None else to_torch(w, dev)
    idx = t["indices"] if indices is None else torch.from_numpy(np.ascontiguousarray(indices)).to(dev)
    dec = dec or make_decoder(w, num_workers, flags=flags)
    say(f"sparse decode {s.name} B={s.batch} s_q={s.s_q} n_h={s.n_h} topk={idx.shape[2]} page={s.page} "
        f"workers={dec.info()['num_workers']} flags={flags} seed={s.seed}")
    out = torch.full((s.batch, s.s_q, s.n_h, s.d_c), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((s.batch, s.s_q, s.n_h), float("nan"), dtype=torch.float32, device=dev) if with_lse else None
    dec.run_sparse(t["q"], t["kv"], t["block_table"], t["seq_lens"], idx, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def sparse_oracle(w, indices=None, batches=None):
    s = w.spec
    return mla_sparse_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens,
                                 w.indices if indices is None else indices, kv_dtype=s.kv_dtype, d_c=s.d_c,
                                 d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale, batches=batches)


SMALL = SPECS["sparse_topk2048_b64_small"]
VARIANTS = [
    SMALL,
    dataclasses.replace(SMALL, name="sparse_mtp2_small", s_q=2, seed=41),
    dataclasses.replace(SMALL, name="sparse_heads64_small", n_h=64, seed=42),
    dataclasses.replace(SMALL, name="sparse_heads256_small", n_h=256, batch=3, seed=43),
    dataclasses.replace(SMALL, name="sparse_page32_small", page=32, seed=44),
    dataclasses.replace(SMALL, name="sparse_topk64_small", topk=64, seed=45),
    dataclasses.replace(SMALL, name="sparse_topk1_small", topk=1, seed=46),
    SPECS["sparse_fp8_topk2048_b64_small"],
    dataclasses.replace(SPECS["sparse_fp8_topk2048_b64_small"], name="sparse_fp8_mtp2_small", s_q=2, seed=50),
    dataclasses.replace(SPECS["sparse_fp8_topk2048_b64_small"], name="sparse_fp8_page32_small", page=32, seed=51),
    dataclasses.replace(SPECS["sparse_fp8_topk2048_b64_small"], name="sparse_fp4_small", kv_dtype="fp4", seed=54),
    # the record's 528-byte fp8 row (d_c = 448)
    SPECS["sparse_fp8_topk2048_b64_d512_small"],
    # flat softmax: a token wrongly counted or dropped by the tile mask moves
    # the output by about 1/n (the lists here are shorter than 64 tokens past
    # the last full tile, both tile halves partly valid)
    dataclasses.replace(SMALL, name="sparse_flat_q0", q_scale=0.0, seq_lens=("fixed", (100, 36, 700, 2000, 1)),
                        topk=700, seed=52),
    dataclasses.replace(SPECS["sparse_fp8_topk2048_b64_small"], name="sparse_fp8_flat_q0", q_scale=0.0,
                        seq_lens=("fixed", (100, 36, 700, 2000, 1)), topk=700, seed=53),
]


WINDOW = 1   # MLA_FLAG_KV_WITHIN_4GIB: these caches are far smaller


@pytest.mark.parametrize("spec", VARIANTS, ids=[s.name for s in VARIANTS])
@pytest.mark.parametrize("workers", [0, 1, 3, 300])
@pytest.mark.parametrize("flags", [0, WINDOW], ids=["addr64", "window"])
def test_sparse_parity_small(spec, workers, flags):
    w = make_workload(spec)
    out, lse = run_sparse(w, num_workers=workers, flags=flags)
    ro, rl = sparse_oracle(w)
    assert_parity(w, out, lse, ro, rl)


@pytest.mark.parametrize("name", ["sparse_topk2048_b64", "sparse_fp8_topk2048_b64"])
@pytest.mark.parametrize("flags", [0, WINDOW], ids=["addr64", "window"])
def test_sparse_full_size_sampled(name, flags):
    w = make_workload(name)
    batches = sorted({0, 31, 63, int(np.argmax(w.seq_lens))})
    out, lse = run_sparse(w, flags=flags)
    ro, rl = sparse_oracle(w, batches=batches)
    assert_parity(w, out, lse, ro, rl, batches=batches)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_sparse_ignores_entries_outside_the_context():
    # entries past the causal limit, past the sequence, huge and negative
    w = make_workload(dataclasses.replace(SMALL, name="sparse_bad_entries", s_q=2, seed=47))
    rng = np.random.default_rng(5)
    idx = w.indices.copy()
    for b in range(w.spec.batch):
        L = int(w.seq_lens[b])
        for j in range(w.spec.s_q):
            n_vis = L - w.spec.s_q + 1 + j
            pos = rng.choice(idx.shape[2], size=4, replace=False)
            idx[b, j, pos] = [n_vis, L + 3, 1 << 30, -5]
    out, lse = run_sparse(w, indices=idx, num_workers=5)
    ro, rl = sparse_oracle(w, indices=idx)
    assert_parity(w, out, lse, ro, rl)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_reads_only_selected_rows(kv_dtype):
    # every row no list selects is NaN-poisoned: bitwise the same result
    base = SMALL if kv_dtype == "bf16" else SPECS["sparse_fp8_topk2048_b64_small"]
    w = make_workload(dataclasses.replace(base, name=f"sparse_poison_{kv_dtype}", seed=48))
    o1, l1 = run_sparse(w, num_workers=7)
    used = np.zeros(w.pool.shape[:2], dtype=bool)
    for b in range(w.spec.batch):
        for t in w.indices[b, 0]:
            if 0 <= t < int(w.seq_lens[b]):
                used[w.block_table[b, t // 64], t % 64] = True
    pool = w.pool.copy()
    pool[~used] = 0x7FC0 if kv_dtype == "bf16" else 0x7F
    o2, l2 = run_sparse(dataclasses.replace(w, pool=pool), num_workers=7)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("kv_dtype,d_c", [("bf16", 512), ("fp8", 512), ("fp4", 512), ("fp8", 448)],
                         ids=["bf16", "fp8", "fp4", "fp8_d512"])
def test_sparse_over_whole_context_equals_dense_bitwise(kv_dtype, d_c):
    # index lists 0 .. L-1 in order (padded with -1) visit the dense decode's
    # tiles in the dense order; with one worker neither run splits, so the
    # two must agree bit for bit
    spec = WorkloadSpec(f"sparse_vs_dense_{kv_dtype}_{d_c}", 3, ("fixed", (700, 64, 1500)), topk=1500,
                        spare_pages=4, seed=49, kv_dtype=kv_dtype, outlier_p=0.01, outlier_mult=20.0, d_c=d_c)
    w = make_workload(spec)
    idx = np.full_like(w.indices, -1)
    for b in range(spec.batch):
        idx[b, 0, :w.seq_lens[b]] = np.arange(w.seq_lens[b])
    o_d, l_d = run_gpu(w, num_workers=1)
    for flags in (0, WINDOW):
        o_s, l_s = run_sparse(w, indices=idx, num_workers=1, flags=flags)
        np.testing.assert_array_equal(o_s, o_d)
        np.testing.assert_array_equal(l_s, l_d)


def test_sparse_repeat_bitwise_and_without_lse():
    w = make_workload(SMALL)
    t = to_torch(w, torch.device("cuda:0"))
    dec = make_decoder(w)
    o1, l1 = run_sparse(w, dec=dec, tensors=t)
    o2, l2 = run_sparse(w, dec=dec, tensors=t)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o3, _ = run_sparse(w, dec=dec, tensors=t, with_lse=False)
    np.testing.assert_array_equal(o1, o3)


def test_sparse_error_paths():
    import mla_latent_cache_decode_amd as m
    w = make_workload(SMALL)
    t = to_torch(w, torch.device("cuda:0"))
    lib = m.load_library()
    dec = make_decoder(w)
    B, k = w.spec.batch, w.spec.topk
    ws = dec.alloc_sparse_workspace(B, k)
    out = torch.zeros((B, 1, 128, 512), dtype=torch.float32, device="cuda")
    args = lambda topk, ws_bytes, idx_ptr: (dec._h, t["q"].data_ptr(), t["kv"].data_ptr(),  # noqa: E731
                                             t["block_table"].data_ptr(), t["seq_lens"].data_ptr(), idx_ptr,
                                             topk, B, out.data_ptr(), None, ws.data_ptr(), ws_bytes, None)
    say("sparse error paths")
    idx = t["indices"].data_ptr()
    assert lib.mla_decode_sparse_run(*args(0, ws.numel(), idx)) == m.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_decode_sparse_run(*args(k, ws.numel(), None)) == m.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_decode_sparse_run(*args(k, ws.numel(), idx + 2)) == m.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_decode_sparse_run(*args(k, 64, idx)) == m.MLA_ERR_WORKSPACE_TOO_SMALL
    # the decode keeps no per-entry table: topk does not change the size
    assert dec.sparse_workspace_size(B, 4 * k) == dec.sparse_workspace_size(B, k)
    assert lib.mla_decode_sparse_run(*args((1 << 20) + 1, ws.numel(), idx)) == m.MLA_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_rows_beyond_4gib(kv_dtype):
    # Without the window flag the gathers use 64-bit addresses: odd pages
    # move past 5 GiB into a cache whose other bytes are NaN, tiles mix near
    # and far rows, and the result must be bitwise the one from the compact
    # cache.
    base = SMALL if kv_dtype == "bf16" else SPECS["sparse_fp8_topk2048_b64_small"]
    w = make_workload(dataclasses.replace(base, name=f"sparse_far_{kv_dtype}", s_q=2, seed=55))
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    o1, l1 = run_sparse(w, num_workers=7, tensors=t)
    kv = t["kv"]
    n_pages, page_bytes = kv.shape[0], kv.shape[1] * kv.shape[2]
    high = (5 << 30) // page_bytes
    say(f"sparse far rows: {n_pages} pages, odd ones from page {high} ({high * page_bytes / 2**30:.2f} GiB) on")
    big = torch.full((high + n_pages,) + tuple(kv.shape[1:]), 0xFF, dtype=kv.dtype, device=dev)
    pages = torch.arange(n_pages, device=dev)
    new = torch.where(pages % 2 == 0, pages, pages + high)
    big[new] = kv
    bt = t["block_table"].clone()
    valid = bt >= 0
    bt[valid] = new[bt[valid].long()].to(bt.dtype)
    o2, l2 = run_sparse(w, num_workers=7, tensors=dict(t, kv=big, block_table=bt))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "fp4"])
def test_sparse_window_flag_never_reads_past_the_window(kv_dtype):
    # a caller that sets the 32-bit window flag for a cache larger than the
    # window gets zeros for the rows past it (odd pages here), not an access
    # outside it; rows inside keep their values
    base = SMALL if kv_dtype == "bf16" else SPECS["sparse_fp8_topk2048_b64_small"]
    w = make_workload(dataclasses.replace(base, name=f"sparse_window_broken_{kv_dtype}", kv_dtype=kv_dtype, seed=56))
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    kv = t["kv"]
    n_pages, page_bytes = kv.shape[0], kv.shape[1] * kv.shape[2]
    high = (5 << 30) // page_bytes
    big = torch.zeros((high + n_pages,) + tuple(kv.shape[1:]), dtype=kv.dtype, device=dev)
    pages = torch.arange(n_pages, device=dev)
    new = torch.where(pages % 2 == 0, pages, pages + high)
    big[new] = kv
    bt = t["block_table"].clone()
    valid = bt >= 0
    bt[valid] = new[bt[valid].long()].to(bt.dtype)
    say("sparse window flag with rows past the window")
    o, l_ = run_sparse(w, num_workers=7, tensors=dict(t, kv=big, block_table=bt), flags=WINDOW)
    assert np.isfinite(o).all() and np.isfinite(l_).all()
    # the oracle on a cache whose odd pages are zero
    pool = w.pool.copy()
    pool[1::2] = 0
    ro, rl = sparse_oracle(dataclasses.replace(w, pool=pool))
    assert_parity(w, o, l_, ro, rl)
    del big
    torch.cuda.empty_cache()
