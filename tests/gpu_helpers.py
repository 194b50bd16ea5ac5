"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the float64 oracle on the same seeded bytes."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from mla_inputs import make_workload, to_torch, Workload
from oracle import mla_decode_ref

# max|err| <= TOL * RMS(out): the stated bounds (bf16 2e-2, quantised fp8
# cache 4e-2); the fp4 cache, decoded from identical bytes by the oracle,
# is held to the fp8 bound
TOL = {"bf16": 2e-2, "fp8": 4e-2, "fp4": 4e-2}


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def make_decoder(w: Workload, num_workers: int = 0, max_batch=None, flags: int = 0):
    from mla_latent_cache_decode_amd import MlaDecode
    s = w.spec
    return MlaDecode(max_batch=max_batch or max(s.batch, 1), s_q=s.s_q, n_h=s.n_h, d_c=s.d_c, d_r=s.d_r,
                     block_size=s.page, max_blocks_per_seq=w.block_table.shape[1], kv_dtype=s.kv_dtype,
                     softmax_scale=s.softmax_scale, num_workers=num_workers, flags=flags)


def run_gpu(w: Workload, num_workers: int = 0, with_lse: bool = True, tensors=None, dec=None):
    s = w.spec
    dev = torch.device("cuda:0")
    t = tensors if tensors is not None else to_torch(w, dev)
    dec = dec or make_decoder(w, num_workers)
    say(f"decode {s.name} B={s.batch} s_q={s.s_q} n_h={s.n_h} kv={s.kv_dtype} "
        f"workers={dec.info()['num_workers']} seed={s.seed}")
    out = torch.full((s.batch, s.s_q, s.n_h, s.d_c), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((s.batch, s.s_q, s.n_h), float("nan"), dtype=torch.float32, device=dev) if with_lse else None
    dec.run(t["q"], t["kv"], t["block_table"], t["seq_lens"], out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def oracle(w: Workload, batches=None, heads=None):
    s = w.spec
    return mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=s.kv_dtype, d_c=s.d_c,
                          d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale, batches=batches, heads=heads)


def assert_parity(w: Workload, out_gpu, lse_gpu, out_ref, lse_ref, batches=None, heads=None):
    """max|err| <= TOL * RMS(oracle out) over the evaluated elements; lse to 1e-3 (relative)."""
    bsel = np.arange(w.spec.batch) if batches is None else np.asarray(list(batches))
    hsel = np.arange(w.spec.n_h) if heads is None else np.asarray(list(heads))
    og = out_gpu[bsel][:, :, hsel]
    orf = out_ref[bsel][:, :, hsel]
    assert np.isfinite(og).all(), "GPU output has non-finite values"
    rms = math.sqrt(float(np.mean(orf ** 2)))
    err = float(np.max(np.abs(og.astype(np.float64) - orf)))
    tol = TOL[w.spec.kv_dtype] * rms
    say(f"  max|err| = {err:.3e}  RMS(out) = {rms:.3e}  err/RMS = {err / rms:.3e}  (bound {TOL[w.spec.kv_dtype]})")
    assert err <= tol, f"max|err| {err} > {tol} (= {TOL[w.spec.kv_dtype]} x RMS {rms})"
    if lse_gpu is not None:
        lg = lse_gpu[bsel][:, :, hsel].astype(np.float64)
        lr = lse_ref[bsel][:, :, hsel]
        fin = np.isfinite(lr)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.all(lg[~fin] == lr[~fin])
        if fin.any():
            lerr = np.max(np.abs(lg[fin] - lr[fin]) / np.maximum(1.0, np.abs(lr[fin])))
            assert lerr <= 1e-3, f"lse relative error {lerr}"
    return err / rms
