"""A seeded sweep of small random shapes through every decode path, against
the float64 oracles: dense and sparse, bf16, fp8 (also at the 448-d latent's
528-byte row) and fp4 caches, page blocks
16..256, 1..4 queries per sequence, 32..256 heads, forced worker counts,
lengths on and off tile edges, and some flat-softmax queries (q = 0 or
nearly), where a token wrongly masked in or out moves the output by about
1/n.  The cases are fixed by their seeds; each one prints its parameters
before it runs."""

import dataclasses

import numpy as np
import pytest

from mla_inputs import WorkloadSpec, make_workload
from oracle import mla_decode_ref, mla_sparse_decode_ref
from gpu_helpers import assert_parity, run_gpu, say

pytestmark = pytest.mark.gpu

N_CASES = 24
N_CASES_D512 = 8     # the fp8 cache's 528-byte row (d_c = 448)
N_CASES_LIN = 8      # the fp8 dense decode with page blocks of 64 and up (its linear page layout), both row widths


def _case(seed: int, d512: bool = False, lin: bool = False):
    if lin:
        d512 = seed % 2 == 1
    rng = np.random.default_rng(1000 + seed + (500 if d512 else 0) + (900 if lin else 0))
    kv = "fp8" if d512 or lin else ("bf16", "fp8", "bf16", "fp4")[seed % 4]
    sparse = False if lin else (seed % 2 == 1 if d512 else seed % 8 >= 4)
    page = int(rng.choice([64, 128, 256] if lin else [16, 32, 64, 64, 128, 256]))
    s_q = int(rng.choice([1, 1, 2, 3, 4]))
    n_h = int(rng.choice([32, 64, 128, 128, 256]))
    batch = int(rng.integers(1, 6))
    # lengths on tile edges, one past them, and anywhere
    pool = [1, 2, 63, 64, 65, 127, 128, 129, 191, 320, 1000, 1500, 2047]
    lens = tuple(int(rng.choice(pool)) if rng.random() < 0.6 else int(rng.integers(s_q, 2400))
                 for _ in range(batch))
    lens = tuple(max(L, s_q) for L in lens)
    q_scale = float(rng.choice([1.0, 1.0, 0.5, 0.02, 0.0]))
    topk = int(rng.choice([1, 40, 64, 100, 500, 2048])) if sparse else 0
    workers = int(rng.choice([0, 0, 1, 5, 37, 300]))
    spec = WorkloadSpec(f"rand{seed}" + ("_lin" if lin else "") + ("_d512" if d512 else ""), batch, ("fixed", lens),
                        kv_dtype=kv, s_q=s_q, n_h=n_h, page=page, q_scale=q_scale, spare_pages=3, topk=topk,
                        seed=2000 + seed + (500 if d512 else 0) + (900 if lin else 0), d_c=448 if d512 else 512,
                        outlier_p=0.01 if kv != "bf16" else 0.0, outlier_mult=20.0)
    return spec, workers


@pytest.mark.parametrize("seed,d512,lin", [(s, False, False) for s in range(N_CASES)]
                         + [(s, True, False) for s in range(N_CASES_D512)]
                         + [(s, False, True) for s in range(N_CASES_LIN)],
                         ids=[f"{s}" for s in range(N_CASES)] + [f"d512_{s}" for s in range(N_CASES_D512)]
                         + [f"lin_{s}" for s in range(N_CASES_LIN)])
def test_random_shape(seed, d512, lin):
    import torch
    spec, workers = _case(seed, d512, lin)
    say(f"case {seed}: {spec} workers={workers}")
    w = make_workload(spec)
    s = w.spec
    if s.topk:
        from gpu_helpers import make_decoder
        dev = torch.device("cuda:0")
        from mla_inputs import to_torch
        t = to_torch(w, dev)
        dec = make_decoder(w, workers)
        out = torch.full((s.batch, s.s_q, s.n_h, s.d_c), float("nan"), dtype=torch.float32, device=dev)
        lse = torch.full((s.batch, s.s_q, s.n_h), float("nan"), dtype=torch.float32, device=dev)
        dec.run_sparse(t["q"], t["kv"], t["block_table"], t["seq_lens"], t["indices"], out, lse)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        ro, rl = mla_sparse_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, w.indices, kv_dtype=s.kv_dtype,
                                       d_c=s.d_c, d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale)
    else:
        out, lse = run_gpu(w, num_workers=workers)
        ro, rl = mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=s.kv_dtype, d_c=s.d_c,
                                d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale)
    assert_parity(w, out, lse, ro, rl)
