#!/usr/bin/env python3
"""MLA latent-cache decode throughput on one MI355X.

One step = one call of the whole hot path (split-KV decode with its fused
work plan, then the LSE combine) over one batch of the long-context
workload: batch 4, seq_lens
{32768, 65536, 131072, 131072}, n_h 128, d_c 512, d_R 64, bf16 paged cache
(block 64, permuted pages).  Inputs are seeded synthetic data already
resident in HBM before the timed region.  ``--workload`` picks another
recipe (a parity workload, or the sparse top-k one, whose step is the
gathering decode, which reads the index lists itself, and the combine).

Order of the run, all on one stream:
  1. W warm-up steps (--warmup).
  2. Cold steps (--cold-steps): before each, a flush writes 1 GiB and then
     reads another 1 GiB, so no byte of the step's inputs is left in the L2s
     or the 256 MB last-level cache and no dirty line is left to write back;
     each step is timed alone by events around it (the flush is outside).
  3. A pre-roll of untimed steps until at least --preroll-ms of GPU time has
     passed: after a pause the GPU needs 30-40 ms of load to return to its
     steady clock (kernels start ~20 % slower), so the pre-roll comes right
     before the timed region (reported as "preroll_steps").
  4. The timed region: exactly K steps (--steps) back to back, warm cache,
     bracketed by synchronisations: ``value`` and ``ms_per_step``.
  5. A sampling pass of 8 x --kernel-samples more steps, every 8th of whose
     decode kernels is timed by HIP events recorded with its own dispatch
     (these cost ~6 us a step, so the timed region runs without them): the
     dominant kernel's roofline.

Prints one JSON line: KV-read GB/s (whole job), TFLOP/s, the cold-cache
figures, the dominant kernel's roofline and the float64 CPU oracle timed on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
def flop_per_row_token(spec) -> int:
    """Q.K^T over the d_c + d_R wide row, P.V over its d_c latent dims (2176 at 512 + 64)."""
    return 2 * (spec.d_c + spec.d_r) + 2 * spec.d_c


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--preroll-ms", type=float, default=150.0,
                    help="after the warm-up, untimed steps until this much GPU time has passed (steady clock)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one by one after a cache flush (0: none)")
    ap.add_argument("--kernel-samples", type=int, default=20,
                    help="steps whose decode kernel is timed by dispatch events, after the timed region (>= 10)")
    ap.add_argument("--workload", default=None, help="workload name (default: the long-context one)")
    ap.add_argument("--num-workers", type=int, default=0)
    ap.add_argument("--cpu-budget-s", type=float, default=15.0, help="oracle sample budget (seconds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def flops_per_step(w) -> int:
    """2176 flop per (query row, token it attends to) at d_c = 512, d_R = 64."""
    s = w.spec
    if w.indices is not None:
        return w.selected_tokens * s.n_h * flop_per_row_token(s)
    tot = 0
    for L in w.seq_lens.tolist():
        for j in range(s.s_q):
            tot += max(L - s.s_q + 1 + j, 0)
    return tot * s.n_h * flop_per_row_token(s)


def cpu_baseline(w, budget_s: float) -> dict:
    """The float64 oracle as it stands, on the same workload: whole sequences in
    batch order, wrapping around to repeat the batch, until the time budget is
    used (always at least one sequence).  Rate = KV bytes of the sequences
    processed over the wall time."""
    import numpy as np
    from oracle import mla_decode_ref, mla_sparse_decode_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    s = w.spec
    row_bytes = {"bf16": 2 * s.d, "fp8": s.d + s.d // 32, "fp4": s.d // 2 + s.d // 16}[s.kv_dtype]
    n_seq, tokens, nbytes = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        b = n_seq % s.batch
        if w.indices is None:
            mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=s.kv_dtype, d_c=s.d_c,
                           d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale, batches=[b])
            n_tok = int(w.seq_lens[b])
        else:
            mla_sparse_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, w.indices, kv_dtype=s.kv_dtype,
                                  d_c=s.d_c, d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale, batches=[b])
            L = int(w.seq_lens[b])
            n_vis = L - s.s_q + 1 + np.arange(s.s_q)[:, None]
            n_tok = int(((w.indices[b] >= 0) & (w.indices[b] < n_vis)).sum())
        n_seq += 1
        tokens += n_tok
        nbytes += n_tok * row_bytes
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    what = "tokens" if w.indices is None else f"selected tokens of top-{s.topk} lists"
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_seq} sequences of {s.name} taken in batch order, repeating the batch "
                      f"({n_seq / s.batch:.2f} passes; {tokens} {what}, all {s.n_h} heads, s_q={s.s_q}), "
                      f"float64 numpy oracle, {dt:.2f} s wall"}


def measured_traffic(kernel: str, workload: str) -> dict | None:
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on this workload and on the kernel source as it is now."""
    from mla_latent_cache_decode_amd.rocprof_summary import kernel_source_hash, read_traffic
    t = read_traffic(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt"))
    if t is None or t["source_hash"] != kernel_source_hash(kernel):
        return None
    return t


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this decode runs on one GPU; multi-GPU runs are not part of this build "
              "(the batch would shard by sequence with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mla_inputs import SPECS, BENCH_SPEC, make_workload, to_torch
    import mla_latent_cache_decode_amd as mla

    name = args.workload or BENCH_SPEC
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    w = make_workload(name)
    s = w.spec
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    # the cache tensor is the whole page pool: declare when it fits the
    # 32-bit gather window (used by the sparse decode only)
    flags = mla.MLA_FLAG_KV_WITHIN_4GIB if t["kv"].numel() <= mla.KV_WINDOW_BYTES else 0
    dec = mla.MlaDecode(max_batch=s.batch, s_q=s.s_q, n_h=s.n_h, d_c=s.d_c, d_r=s.d_r, block_size=s.page,
                        max_blocks_per_seq=w.block_table.shape[1], kv_dtype=s.kv_dtype,
                        softmax_scale=s.softmax_scale, num_workers=args.num_workers, flags=flags)
    sparse = w.indices is not None
    ws = dec.alloc_sparse_workspace(s.batch, s.topk, device=dev) if sparse else dec.alloc_workspace(s.batch, device=dev)
    out = torch.empty((s.batch, s.s_q, s.n_h, s.d_c), dtype=torch.float32, device=dev)
    lse = torch.empty((s.batch, s.s_q, s.n_h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = mla.load_library()
    if sparse:
        entry = lib.mla_decode_sparse_run
        call = (dec._h, t["q"].data_ptr(), t["kv"].data_ptr(), t["block_table"].data_ptr(),
                t["seq_lens"].data_ptr(), t["indices"].data_ptr(), s.topk, s.batch, out.data_ptr(),
                lse.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream)
    else:
        entry = lib.mla_decode_run
        call = (dec._h, t["q"].data_ptr(), t["kv"].data_ptr(), t["block_table"].data_ptr(),
                t["seq_lens"].data_ptr(), s.batch, out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(),
                stream.cuda_stream)

    def step():
        st = entry(*call)
        if st != 0:
            raise mla.MlaError(st, entry.__name__)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # cold steps: flush (write 1 GiB, then read another 1 GiB), then one step
    # timed alone; its decode kernel by dispatch events
    cold = None
    if args.cold_steps > 0:
        print(f"[bench] cold {args.cold_steps}", file=sys.stderr, flush=True)
        flush_w = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        flush_r = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        c_step, c_kern = [], []
        for k in range(args.cold_steps):
            flush_w.fill_(k & 0xFF)
            torch.sum(flush_r, dim=0, out=sink)
            s0, s1, k0, k1 = ev(), ev(), ev(), ev()
            k0.record(stream)   # torch only reads events it has seen recorded
            k1.record(stream)
            lib.mla_decode_set_profile_events(dec._h, k0.cuda_event, k1.cuda_event)
            s0.record(stream)
            step()
            s1.record(stream)
            lib.mla_decode_set_profile_events(dec._h, None, None)
            torch.cuda.synchronize()
            c_step.append(s0.elapsed_time(s1))
            c_kern.append(k0.elapsed_time(k1))
        del flush_w, flush_r
        cold = (float(np.median(c_step)), float(np.median(c_kern)), len(c_step))

    # pre-roll: untimed steps until --preroll-ms of GPU time has passed; the
    # count comes from a first batch of 10, the rest is enqueued in one go
    pre_steps, pre_ms = 0, 0.0
    if args.preroll_ms > 0:
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(10):
            step()
        b.record(stream)
        b.synchronize()
        per = max(a.elapsed_time(b) / 10, 1e-3)
        more = int(math.ceil(max(args.preroll_ms - a.elapsed_time(b), 0.0) / per))
        c = ev()
        for _ in range(more):
            step()
        c.record(stream)
        c.synchronize()
        pre_steps, pre_ms = 10 + more, a.elapsed_time(c)
    print(f"[bench] pre-roll {pre_steps} steps, {pre_ms:.1f} ms", file=sys.stderr, flush=True)

    # the timed region: K bare steps back to back
    t_start, t_stop = ev(), ev()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_stop)
    ms_step = ms_total / args.steps

    # sampling pass: the decode kernel's own dispatch timestamps on every
    # 8th step (events on consecutive steps slow the steps down), bare steps
    # in between
    n_samp = max(args.kernel_samples, 10)
    samp = [(ev(), ev()) for _ in range(n_samp)]
    for a, b in samp:           # torch only reads events it has seen recorded
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for a, b in samp:
        lib.mla_decode_set_profile_events(dec._h, a.cuda_event, b.cuda_event)
        step()
        lib.mla_decode_set_profile_events(dec._h, None, None)
        for _ in range(7):
            step()
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in samp]
    kms = float(np.mean(kernel_ms))

    if args.copy_mb:
        n = args.copy_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    kv_bytes = w.kv_bytes_algorithmic
    gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    fl = flops_per_step(w)
    tflops = fl / (ms_step * 1e-3) / 1e12
    k_gbs = kv_bytes / (kms * 1e-3) / 1e9
    k_tflops = fl / (kms * 1e-3) / 1e12
    # the kernel's roofline: HBM below the balance point (2.5 PFLOP/s over
    # 8 TB/s = 312.5 flop/B), the matrix cores above it.  The 16-bit peak
    # applies to every cache format: P.V runs as 16-bit MFMA, and Q.K^T too
    # except on the fp8 cache, where it runs as two block-scaled fp8
    # products (q_hi, q_lo) at twice the rate, the time of one 16-bit product
    intensity = fl / kv_bytes
    if intensity <= BF16_MFMA_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        roof = {"bound": "hbm", "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(k_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(k_tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
    info = dec.info()
    from mla_latent_cache_decode_amd.rocprof_summary import kernel_for_dtype
    kernel = kernel_for_dtype(s.kv_dtype, sparse)
    traffic = measured_traffic(kernel, s.name)
    res = {
        "metric": "MLA decode KV-read GB/s (% of HBM peak) + TFLOP/s, n_h=128, 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3/e8m0 cache, fp8 (two-term query) + fp16 mfma",
                  "fp4": "fp4-e2m1/e8m0 cache, fp16 mfma"}[s.kv_dtype],
        "data": "synthetic (seeded N(0,1) cache and queries, DeepSeek-V3/R1 shapes)",
        "config": {"workload": s.name, "batch": s.batch, "s_q": s.s_q, "n_h": s.n_h, "d_c": s.d_c,
                   "d_r": s.d_r, "page": s.page, "kv_dtype": s.kv_dtype,
                   "seq_lens": w.seq_lens.tolist() if s.batch <= 8 else f"{s.seq_lens}",
                   "total_tokens": int(w.seq_lens.sum()), "kv_bytes": kv_bytes,
                   **({"topk": s.topk, "selected_tokens": w.selected_tokens} if sparse else {}),
                   "workers": info["num_workers"], "row_groups": info["row_groups"],
                   "compute_units": info["compute_units"]},
        "preroll_steps": pre_steps,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tflop_s": round(tflops, 2),
        "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "roofline": {**roof,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "kernel": kernel, "kernel_ms": round(kms, 5), "kernel_samples": len(kernel_ms),
                     "bytes_per_launch": kv_bytes, "flop_per_launch": fl,
                     "intensity_flop_per_byte": round(intensity, 1), "kernel_gbs": round(k_gbs, 2)},
    }
    if cold is not None:
        c_step, c_kern, n_cold = cold
        res["cold"] = {"what": "each step timed alone after a 1 GiB write + 1 GiB read flush (median)",
                       "steps": n_cold, "ms_per_step": round(c_step, 5),
                       "value": round(kv_bytes / (c_step * 1e-3) / 1e9, 2), "unit": "GB/s",
                       "kernel_ms": round(c_kern, 5),
                       "kernel_gbs": round(kv_bytes / (c_kern * 1e-3) / 1e9, 2),
                       "kernel_hbm_frac": round(kv_bytes / (c_kern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "kernel_tflop_s": round(fl / (c_kern * 1e-3) / 1e12, 2)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
