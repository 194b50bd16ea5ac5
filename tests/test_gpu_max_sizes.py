"""Large and maximum shapes through the C ABI against the float64 oracles:
batches past one work-plan chunk (the planner scans lengths 256 sequences at
a time), the most rows one query position can have (n_h 1024; s_q 8 x 128
heads), and a single 1M-token context (1.2 GB of bf16 cache), checked on
sampled heads."""

import dataclasses

import numpy as np
import pytest
import torch

from mla_inputs import WorkloadSpec, make_workload, to_torch
from oracle import mla_decode_ref, mla_sparse_decode_ref
from gpu_helpers import assert_parity, make_decoder, run_gpu, say

pytestmark = pytest.mark.gpu

MANY = [
    WorkloadSpec("batch1000", 1000, ("uniform", 1, 300), spare_pages=16, seed=61),
    WorkloadSpec("batch1000_fp8_mtp2", 1000, ("uniform", 2, 300), s_q=2, kv_dtype="fp8", spare_pages=16, seed=62,
                 outlier_p=0.01, outlier_mult=20.0),
    WorkloadSpec("batch700_empty_and_long", 700, ("fixed", tuple([0, 1, 5000] + [37] * 697)), spare_pages=16, seed=63),
]


@pytest.mark.parametrize("spec", MANY, ids=[s.name for s in MANY])
@pytest.mark.parametrize("workers", [0, 300])
def test_many_sequences(spec, workers):
    w = make_workload(spec)
    out, lse = run_gpu(w, num_workers=workers)
    ro, rl = mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=spec.kv_dtype, d_c=spec.d_c,
                            d_r=spec.d_r, page=spec.page, softmax_scale=spec.softmax_scale)
    assert_parity(w, out, lse, ro, rl)


def test_many_sparse_units():
    spec = WorkloadSpec("sparse_batch600_mtp2", 600, ("uniform", 2, 500), s_q=2, topk=128, spare_pages=16, seed=64)
    w = make_workload(spec)
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    dec = make_decoder(w)
    say(f"sparse {spec.name}")
    out = torch.full((spec.batch, 2, 128, 512), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((spec.batch, 2, 128), float("nan"), dtype=torch.float32, device=dev)
    dec.run_sparse(t["q"], t["kv"], t["block_table"], t["seq_lens"], t["indices"], out, lse)
    torch.cuda.synchronize()
    ro, rl = mla_sparse_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, w.indices, kv_dtype="bf16",
                                   d_c=512, d_r=64, page=64, softmax_scale=spec.softmax_scale)
    assert_parity(w, out.cpu().numpy(), lse.cpu().numpy(), ro, rl)


WIDE = [
    WorkloadSpec("heads1024", 2, ("fixed", (700, 129)), n_h=1024, spare_pages=4, seed=65),
    WorkloadSpec("mtp8_heads128", 3, ("fixed", (8, 300, 1000)), s_q=8, spare_pages=4, seed=66),
    WorkloadSpec("mtp8_heads128_fp8", 2, ("fixed", (9, 1000)), s_q=8, kv_dtype="fp8", spare_pages=4, seed=67),
]


@pytest.mark.parametrize("spec", WIDE, ids=[s.name for s in WIDE])
def test_most_rows(spec):
    w = make_workload(spec)
    out, lse = run_gpu(w)
    ro, rl = mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=spec.kv_dtype, d_c=spec.d_c,
                            d_r=spec.d_r, page=spec.page, softmax_scale=spec.softmax_scale)
    assert_parity(w, out, lse, ro, rl)


def test_one_million_token_context():
    spec = WorkloadSpec("ctx1m", 1, ("fixed", (1 << 20,)), spare_pages=2, seed=68, q_scale=0.5)
    w = make_workload(spec)
    heads = [0, 77, 127]
    out, lse = run_gpu(w)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ro, rl = mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype="bf16", d_c=512, d_r=64,
                            page=64, softmax_scale=spec.softmax_scale, heads=heads)
    assert_parity(w, out, lse, ro, rl, heads=heads)


@pytest.mark.parametrize("kv_dtype,page", [("bf16", 64), ("fp8", 256)])
def test_sparse_one_million_token_context(kv_dtype, page):
    # index lists spread over a 1M-token context: page ids up to 16K (4K at
    # block 256) pass through the kernels' own list-to-row translation
    spec = WorkloadSpec(f"sparse_ctx1m_{kv_dtype}", 1, ("fixed", (1 << 20,)), s_q=2, topk=2048, page=page,
                        kv_dtype=kv_dtype, spare_pages=2, seed=69, q_scale=0.5,
                        outlier_p=0.01 if kv_dtype == "fp8" else 0.0, outlier_mult=20.0)
    w = make_workload(spec)
    assert int(w.indices.max()) > (1 << 20) - 4096
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    dec = make_decoder(w)
    say(f"sparse {spec.name} page={page}")
    out = torch.full((1, 2, 128, 512), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((1, 2, 128), float("nan"), dtype=torch.float32, device=dev)
    dec.run_sparse(t["q"], t["kv"], t["block_table"], t["seq_lens"], t["indices"], out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    heads = [0, 77, 127]
    ro, rl = mla_sparse_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, w.indices, kv_dtype=kv_dtype,
                                   d_c=512, d_r=64, page=page, softmax_scale=spec.softmax_scale, heads=heads)
    assert_parity(w, out, lse, ro, rl, heads=heads)
