"""Value ranges and plan records through the C ABI, against the float64 oracle.

* Large cache values: the products take the cache through fp16 (P.V for the
  bf16 cache; both products for the quantised formats), so the header states
  |x| < 65520 as a precondition.  Cases with values of several 10^4 and at
  the documented edge (the largest bf16 value below it, 65280, and the
  largest fp8 code times scale below it, 240 * 2^8 = 61440) must match the
  oracle element by element.
* Tiny queries: the fp8 / fp4 kernels prescale each head's query by a power
  of two; heads of about 1e-36 and bf16-subnormal heads give a flat softmax.
* Plan records: with a batch past one 256-sequence planner chunk, trailing
  empty sequences whose cost position equals the last worker's quota end
  must still get their split record (out = 0, lse = -inf), even when the
  workspace holds stale records from an earlier call.
"""

import dataclasses

import numpy as np
import pytest
import torch

from mla_inputs import WorkloadSpec, make_workload, to_torch
from gpu_helpers import assert_parity, make_decoder, oracle, run_gpu, say

pytestmark = pytest.mark.gpu

BF16_EDGE = 0x477F          # 65280, the largest bf16 value below 65520
FP8_CODE_240 = 0x77         # e4m3fn 0.1110.111 = 1.875 * 2^7 = 240
FP8_EDGE_SCALE = 127 + 8    # 240 * 2^8 = 61440


def _decoded_max(w):
    from oracle.formats import decode_bf16_rows, decode_fp8_rows, decode_fp4_rows
    s = w.spec
    mx = 0.0
    for b in range(s.batch):
        L = int(w.seq_lens[b])
        if L == 0:
            continue
        pages = w.block_table[b, :(L + s.page - 1) // s.page]
        raw = w.pool[pages].reshape((-1,) + w.pool.shape[2:])[:L]
        dec = {"bf16": decode_bf16_rows, "fp8": decode_fp8_rows, "fp4": decode_fp4_rows}[s.kv_dtype](raw, s.d)
        mx = max(mx, float(np.abs(dec).max()))
    return mx


LARGE = [
    # N(0,1) x 8000: values of several 10^4 (max ~5e4), queries scaled so the
    # scores stay of order one
    WorkloadSpec("large_bf16", 4, ("fixed", (70, 700, 1500, 2100)), kv_scale=8000.0, q_scale=1.0 / 8000.0,
                 spare_pages=4, seed=31),
    WorkloadSpec("large_fp8", 4, ("fixed", (70, 700, 1500, 2100)), kv_dtype="fp8", kv_scale=8000.0,
                 q_scale=1.0 / 8000.0, spare_pages=4, seed=32),
    WorkloadSpec("large_fp4", 4, ("fixed", (70, 700, 1500, 2100)), kv_dtype="fp4", kv_scale=8000.0,
                 q_scale=1.0 / 8000.0, spare_pages=4, seed=33),
    WorkloadSpec("large_mtp2", 3, ("fixed", (65, 900, 2000)), s_q=2, kv_scale=8000.0, q_scale=1.0 / 8000.0,
                 spare_pages=4, seed=34),
]


@pytest.mark.parametrize("spec", LARGE, ids=[s.name for s in LARGE])
@pytest.mark.parametrize("workers", [0, 5])
def test_large_cache_values(spec, workers):
    w = make_workload(spec)
    mx = _decoded_max(w)
    say(f"{spec.name}: max |decoded cache value| = {mx:.1f}")
    assert 3e4 <= mx < 65520
    out, lse = run_gpu(w, num_workers=workers)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


def _plant_edge_values(w, seed):
    """Put the documented edge values into visible tokens: in the latent part
    (which P.V reads) and in the RoPE part, with both signs."""
    s = w.spec
    rng = np.random.default_rng(seed)
    pool = w.pool.copy()
    for b in range(s.batch):
        L = int(w.seq_lens[b])
        for t in rng.choice(L, size=min(L, 6), replace=False):
            pg, r = w.block_table[b, t // s.page], t % s.page
            if s.kv_dtype == "bf16":
                for dim in rng.choice(s.d, size=4, replace=False):
                    pool[pg, r, dim] = BF16_EDGE | (0x8000 if rng.random() < 0.5 else 0)
            else:
                # one 32-code group gets scale 2^8 and codes of magnitude <= 240;
                # one code is exactly 240, so the group decodes up to 61440
                g = int(rng.integers(0, s.d // 32))
                codes = pool[pg, r, 32 * g:32 * g + 32].astype(np.int32)
                mag = np.minimum(codes & 0x7F, FP8_CODE_240)
                codes = (codes & 0x80) | mag
                codes[int(rng.integers(0, 32))] = FP8_CODE_240 | (0x80 if rng.random() < 0.5 else 0)
                pool[pg, r, 32 * g:32 * g + 32] = codes.astype(np.uint8)
                pool[pg, r, s.d + g] = FP8_EDGE_SCALE
    return dataclasses.replace(w, pool=pool)


EDGE_VALUES = [
    WorkloadSpec("edge65280_bf16", 3, ("fixed", (50, 640, 1300)), q_scale=1.0 / 2000.0, spare_pages=4, seed=35),
    WorkloadSpec("edge61440_fp8", 3, ("fixed", (50, 640, 1300)), kv_dtype="fp8", q_scale=1.0 / 2000.0,
                 spare_pages=4, seed=36),
]


@pytest.mark.parametrize("spec", EDGE_VALUES, ids=[s.name for s in EDGE_VALUES])
@pytest.mark.parametrize("workers", [0, 3])
def test_documented_edge_values(spec, workers):
    w = _plant_edge_values(make_workload(spec), seed=spec.seed)
    mx = _decoded_max(w)
    say(f"{spec.name}: max |decoded cache value| = {mx:.1f}")
    assert mx == (65280.0 if spec.kv_dtype == "bf16" else 61440.0)
    out, lse = run_gpu(w, num_workers=workers)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


TINY_Q = [
    # heads of about 1e-36 (bf16 normal) and about 1e-39 (bf16 subnormal):
    # every score is ~0, the softmax is flat and the output the mean row
    WorkloadSpec("tiny_q_fp8", 4, ("fixed", (1, 40, 300, 1200)), kv_dtype="fp8", q_scale=1e-36, spare_pages=4,
                 seed=37),
    WorkloadSpec("subnormal_q_fp8", 4, ("fixed", (1, 40, 300, 1200)), kv_dtype="fp8", q_scale=1e-39,
                 spare_pages=4, seed=38),
    WorkloadSpec("tiny_q_fp4", 4, ("fixed", (1, 40, 300, 1200)), kv_dtype="fp4", q_scale=1e-36, spare_pages=4,
                 seed=39),
    WorkloadSpec("subnormal_q_fp4", 4, ("fixed", (1, 40, 300, 1200)), kv_dtype="fp4", q_scale=1e-39,
                 spare_pages=4, seed=40),
    WorkloadSpec("subnormal_q_bf16", 4, ("fixed", (1, 40, 300, 1200)), q_scale=1e-39, spare_pages=4, seed=41),
]


@pytest.mark.parametrize("spec", TINY_Q, ids=[s.name for s in TINY_Q])
def test_tiny_queries(spec):
    w = make_workload(spec)
    qf = w.q_bits.astype(np.uint32) << 16
    q = qf.view(np.float32)
    assert np.abs(q).max() > 0
    if spec.q_scale < 1e-38:
        assert np.abs(q).max() < 2.0 ** -126          # every query element is a bf16 subnormal
    out, lse = run_gpu(w)
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


def _run_on(dec, w, ws):
    s = w.spec
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    out = torch.full((s.batch, s.s_q, s.n_h, s.d_c), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((s.batch, s.s_q, s.n_h), float("nan"), dtype=torch.float32, device=dev)
    dec.run(t["q"], t["kv"], t["block_table"], t["seq_lens"], out, lse, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _trailing_empty_case(lens_full, lens_empty_tail, workers, seed):
    """Run lens_full first (every record says 'one split'), then, on the same
    handle and workspace, lens_empty_tail, whose trailing empty sequences
    must be recorded by the planner's last worker."""
    B = len(lens_full)
    w_full = make_workload(WorkloadSpec("plan_full", B, ("fixed", tuple(lens_full)), spare_pages=2, seed=seed))
    w = make_workload(WorkloadSpec("plan_tail", B, ("fixed", tuple(lens_empty_tail)), spare_pages=2, seed=seed + 1))
    assert w.block_table.shape[1] == w_full.block_table.shape[1]
    dec = make_decoder(w, num_workers=workers, max_batch=B)
    ws = dec.alloc_workspace(B)
    say(f"plan records: B={B} workers={dec.info()['num_workers']} stale run first")
    _run_on(dec, w_full, ws)
    out, lse = _run_on(dec, w, ws)
    empty = np.asarray(lens_empty_tail) == 0
    assert np.all(out[empty] == 0.0), "an empty sequence's output was not written"
    assert np.all(lse[empty] == -np.inf), "an empty sequence's lse was not written"
    ro, rl = oracle(w)
    assert_parity(w, out, lse, ro, rl)


def test_trailing_empty_sequences_one_worker():
    # total cost = 250 x (2 pages + 3) = the single worker's quota end
    _trailing_empty_case([100] * 300, [100] * 250 + [0] * 50, workers=1, seed=42)


def test_trailing_empty_sequences_default_workers():
    # one page (cost 4) per non-empty sequence and G of them: the total cost
    # 4G is a multiple of the default worker count G
    import mla_latent_cache_decode_amd as m
    probe = make_decoder(make_workload(WorkloadSpec("probe", 1, ("fixed", (64,)), spare_pages=0, seed=43)))
    G = probe.info()["num_workers"]
    _trailing_empty_case([64] * (G + 44), [64] * G + [0] * 44, workers=0, seed=44)


def test_trailing_empty_sequences_forced_workers():
    # G = 250 forced, 250 non-empty sequences of cost 4 -> total = 4G
    _trailing_empty_case([64] * 300, [64] * 250 + [0] * 50, workers=250, seed=45)
