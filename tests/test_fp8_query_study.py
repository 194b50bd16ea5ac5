"""Error study behind a design decision (CPU only): can Q.K^T of the fp8 cache
run as a block-scaled fp8 MFMA?

That needs the query in the cache's own format, e4m3 codes with one e8m0
scale per 32 ("DeepSeek-R1" record, engine kernel constraint (2)).  Emulated
here against the float64 oracle on the fp8 recipe (1 % outliers x 20), with
the decode's other roundings (fp16 weights) kept: one e4m3 term misses the
4e-2 * RMS(out) bound by two orders of magnitude (the outliers multiply the
query's rounding error, and sharp rows follow one token's score), while a
two-term query q ~ q_hi + q_lo (each e4m3 with its own scales) is as
accurate as the exact one.  The fp8 decode kernel therefore carries two
query terms and issues two scaled MFMAs per 64-deep k-block: the same
matrix-core time as fp16 MFMAs would take, but on the raw cache codes and
scales, with no dequantisation of K.
"""

import math

import numpy as np
import torch

from mla_inputs import make_workload, quantize_fp8_rows
from oracle import formats, mla

BOUND = 4e-2


def _quantise_rows(x: np.ndarray, d: int) -> np.ndarray:
    """Rows rounded through the cache's e4m3 / e8m0-per-32 format."""
    enc = quantize_fp8_rows(torch.from_numpy(x.astype(np.float32)), d, d + d // 32)
    return formats.decode_fp8_rows(enc, d)


def _attend_fp16_weights(q_rows, kv_rows, d_c, scale):
    s = scale * (q_rows @ kv_rows.T)
    p = np.exp(s - s.max(axis=1, keepdims=True)).astype(np.float16).astype(np.float64)
    return (p @ kv_rows[:, :d_c]) / p.sum(axis=1)[:, None]


def test_single_fp8_query_term_breaks_the_bound_two_terms_meet_it():
    w = make_workload("fp8_b64_small")
    s = w.spec
    errs = {"exact": [], "one": [], "two": []}
    refs = []
    for b in range(s.batch):
        L = int(w.seq_lens[b])
        rows = mla.decode_rows(mla.gather_rows(w.pool, w.block_table[b], L, s.page), s.kv_dtype, s.d)
        q = formats.bf16_bits_to_f64(w.q_bits[b, 0])
        ref, _ = mla.attend_one_query(q, rows, s.d_c, s.softmax_scale)
        refs.append(ref)
        q_hi = _quantise_rows(q, s.d)
        q_lo = _quantise_rows(q - q_hi, s.d)
        for k, qq in (("exact", q), ("one", q_hi), ("two", q_hi + q_lo)):
            errs[k].append(np.abs(_attend_fp16_weights(qq, rows, s.d_c, s.softmax_scale) - ref).max())
    rms = math.sqrt(np.mean(np.concatenate([r.ravel() for r in refs]) ** 2))
    one, two, exact = max(errs["one"]) / rms, max(errs["two"]) / rms, max(errs["exact"]) / rms
    assert one > 10 * BOUND, one            # measured ~5.5
    assert two < BOUND / 4 and exact < BOUND / 4, (two, exact)   # both ~2e-3
