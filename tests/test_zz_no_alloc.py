"""mla_decode_run_noalloc: the decode with the library's per-GPU scratch in
place of a caller workspace, through the C ABI, against mla_decode_run (same
kernels, so the results must be bitwise equal) on two calls in a row, the
second with a smaller input; and its size check."""

import numpy as np
import pytest
import torch

import mla_latent_cache_decode_amd as mla
from mla_inputs import WorkloadSpec, make_workload, to_torch
from gpu_helpers import make_decoder, say

pytestmark = pytest.mark.gpu


def _both(dec, w):
    s = w.spec
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    res = []
    for how in ("run", "noalloc"):
        out = torch.full((s.batch, s.s_q, s.n_h, s.d_c), float("nan"), dtype=torch.float32, device=dev)
        lse = torch.full((s.batch, s.s_q, s.n_h), float("nan"), dtype=torch.float32, device=dev)
        if how == "run":
            dec.run(t["q"], t["kv"], t["block_table"], t["seq_lens"], out, lse)
        else:
            dec.run_noalloc(t["q"], t["kv"], t["block_table"], t["seq_lens"], out, lse)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


CASES = [
    # (first call, second smaller call), same handle
    (WorkloadSpec("na_big", 6, ("fixed", (9000, 30, 4100, 0, 1500, 2222)), spare_pages=4, seed=81),
     WorkloadSpec("na_small", 3, ("fixed", (700, 64, 1)), spare_pages=2, seed=82)),
    (WorkloadSpec("na_big_fp8", 5, ("fixed", (6000, 3000, 129, 2000, 64)), kv_dtype="fp8", spare_pages=4,
                  seed=83, outlier_p=0.01, outlier_mult=20.0),
     WorkloadSpec("na_small_fp8", 2, ("fixed", (300, 65)), kv_dtype="fp8", spare_pages=2, seed=84)),
    (WorkloadSpec("na_big_mtp", 4, ("fixed", (5000, 2, 3000, 900)), s_q=2, spare_pages=4, seed=85),
     WorkloadSpec("na_small_mtp", 2, ("fixed", (100, 40)), s_q=2, spare_pages=2, seed=86)),
    # the fp8 cache's 528-byte row (d_c = 448)
    (WorkloadSpec("na_big_fp8_d512", 4, ("fixed", (5000, 1, 2600, 700)), kv_dtype="fp8", d_c=448, spare_pages=4,
                  seed=87, outlier_p=0.01, outlier_mult=20.0),
     WorkloadSpec("na_small_fp8_d512", 2, ("fixed", (200, 64)), kv_dtype="fp8", d_c=448, spare_pages=2, seed=88)),
]


@pytest.mark.parametrize("big,small", CASES, ids=[c[0].name for c in CASES])
@pytest.mark.parametrize("workers", [0, 7])
def test_noalloc_matches_run(big, small, workers):
    w1, w2 = make_workload(big), make_workload(small)
    mb = max(w1.block_table.shape[1], w2.block_table.shape[1])
    # one handle for both calls: pad the smaller block table to the same row stride
    def pad(w):
        bt = np.full((w.spec.batch, mb), -1, dtype=np.int32)
        bt[:, :w.block_table.shape[1]] = w.block_table
        import dataclasses
        return dataclasses.replace(w, block_table=bt)
    w1, w2 = pad(w1), pad(w2)
    dec = make_decoder(w1, num_workers=workers, max_batch=big.batch)
    assert dec.workspace_size(big.batch) <= mla.NOALLOC_SCRATCH_BYTES
    for w in (w1, w2):
        say(f"noalloc {w.spec.name} B={w.spec.batch} workers={dec.info()['num_workers']}")
        (o_run, l_run), (o_na, l_na) = _both(dec, w)
        assert np.isfinite(o_run).all()
        np.testing.assert_array_equal(o_na, o_run)
        np.testing.assert_array_equal(l_na, l_run)


def test_noalloc_default_plan_fits_the_scratch():
    # every n_h * s_q of the default plan fits (256-CU device)
    for s_q, n_h in [(1, 128), (2, 128), (4, 128), (8, 128), (1, 1024), (1, 32)]:
        dec = mla.MlaDecode(max_batch=1024, s_q=s_q, n_h=n_h, max_blocks_per_seq=64,
                            softmax_scale=0.072)
        assert dec.workspace_size(1024) <= mla.NOALLOC_SCRATCH_BYTES, (s_q, n_h)
    # the fp8 cache adds its two-term query rows (1216 bytes each): 400
    # sequences of 128 heads still fit
    dec = mla.MlaDecode(max_batch=400, n_h=128, max_blocks_per_seq=64, kv_dtype="fp8", softmax_scale=0.072)
    assert dec.workspace_size(400) <= mla.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    w = make_workload(WorkloadSpec("na_reject", 2, ("fixed", (100, 200)), spare_pages=1, seed=87))
    dec = make_decoder(w, num_workers=4096)
    assert dec.workspace_size(2) > mla.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    out = torch.zeros((2, 1, 128, 512), dtype=torch.float32, device=dev)
    with pytest.raises(mla.MlaError) as e:
        dec.run_noalloc(t["q"], t["kv"], t["block_table"], t["seq_lens"], out)
    assert e.value.status == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
