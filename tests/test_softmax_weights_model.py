"""The row-split decode's fp16 softmax weights, modelled on the CPU (a design
check, like the fp8 query study).

The fp8 and fp4 cache kernels keep a lazy running max m per query row and
store the weights of P.V as fp16 2^(s - m - kPOffset) (s the score in log2
units); m is raised only when a 64-token tile's max exceeds it by more than
kRescaleTau, which keeps every weight at most 2^(kRescaleTau - kPOffset)
inside fp16, and O and the row sum are then rescaled.  The two constants are
read from the kernel header; the model redoes that arithmetic tile by tile
(per row; the kernel decides per wave of 32 rows) on the fp8 recipe's scores
and compares the result with float64 attention ("DeepSeek R1 Architecture &
Deployment Guide", section 1.1: softmax over the context, then the weighted
sum of the latent rows).  The offset trades a little precision (weights far
below the running max become fp16 subnormals or zero) for far fewer
rescales of the 256-register O accumulator.
"""

import math
import os
import re

import numpy as np
import pytest

from mla_inputs import make_workload
from oracle import formats, mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "mla_latent_cache_decode_amd", "csrc", "decode_rowsplit.h")
BOUND = 4e-2                      # fp8 cache: max |err| <= 4e-2 * RMS(out)
FP16_MAX = 65504.0


def _constant(name):
    m = re.search(r"constexpr float " + name + r" = ([0-9.]+)f;", open(HEADER).read())
    assert m, f"{name} not found in {HEADER}"
    return float(m.group(1))


TAU = _constant("kRescaleTau")
OFFSET = _constant("kPOffset")


def _model(s_log2, v, tau, offset, rows_per_wave=32):
    """Lazy-max attention with fp16 weights: s_log2 [rows, tokens] scores in
    log2 units, v [tokens, d] values.  Returns (out [rows, d], wave-tiles that
    rescaled O)."""
    rows, n = s_log2.shape
    o = np.zeros((rows, v.shape[1]))
    l = np.zeros(rows)
    m = np.full(rows, -np.inf)
    rescales = 0
    for t0 in range(0, n, 64):
        st = s_log2[:, t0:t0 + 64]
        mx = st.max(axis=1)
        need = mx > m + tau
        for w0 in range(0, rows, rows_per_wave):
            nw = need[w0:w0 + rows_per_wave]
            if nw.any() and np.isfinite(m[w0:w0 + rows_per_wave]).any():
                rescales += 1
        m_new = np.where(need, mx, m)
        alpha = np.where(np.isfinite(m), np.exp2(m - m_new), 0.0)
        o *= alpha[:, None]
        l *= alpha
        m = m_new
        x = np.exp2(st - m[:, None] - offset)
        p = x.astype(np.float32).astype(np.float16).astype(np.float64)
        assert np.isfinite(p).all() and p.max() <= FP16_MAX
        l += x.astype(np.float32).astype(np.float64).sum(axis=1)   # the kernel sums the unrounded weights
        o += p @ v[t0:t0 + 64]
    return o / l[:, None], rescales


def _sequences(name):
    w = make_workload(name)
    s = w.spec
    for b in range(s.batch):
        L = int(w.seq_lens[b])
        rows = mla.decode_rows(mla.gather_rows(w.pool, w.block_table[b], L, s.page), s.kv_dtype, s.d)
        q = formats.bf16_bits_to_f64(w.q_bits[b, 0])
        ref, _ = mla.attend_one_query(q, rows, s.d_c, s.softmax_scale)
        yield (q @ rows.T) * (s.softmax_scale / math.log(2)), rows[:, :s.d_c], ref


def test_weights_stay_inside_fp16():
    # a tile whose max is m + tau (no rescale) weighs 2^(tau - offset) there
    assert TAU - OFFSET <= 15 and 2.0 ** (TAU - OFFSET) < FP16_MAX
    assert OFFSET >= 0


@pytest.fixture(scope="module")
def fp8_small():
    return list(_sequences("fp8_b64_small"))


def test_modelled_weights_meet_half_the_fp8_bound(fp8_small):
    errs, refs = [], []
    for s_log2, v, ref in fp8_small:
        out, _ = _model(s_log2, v, TAU, OFFSET)
        errs.append(np.abs(out - ref).max())
        refs.append(ref)
    rms = math.sqrt(np.mean(np.concatenate([r.ravel() for r in refs]) ** 2))
    assert max(errs) / rms < BOUND / 2, max(errs) / rms


def test_offset_cuts_rescales_without_losing_the_model_its_accuracy(fp8_small):
    # against the same arithmetic without an offset (threshold 15, the most
    # fp16 allows): at most a third of the rescales, error within 2x
    n_off = n_base = 0
    e_off = e_base = 0.0
    refs = []
    for s_log2, v, ref in fp8_small:
        out, n = _model(s_log2, v, TAU, OFFSET)
        out0, n0 = _model(s_log2, v, 15.0, 0.0)
        n_off, n_base = n_off + n, n_base + n0
        e_off = max(e_off, np.abs(out - ref).max())
        e_base = max(e_base, np.abs(out0 - ref).max())
        refs.append(ref)
    assert n_base > 0 and 3 * n_off <= n_base, (n_off, n_base)
    rms = math.sqrt(np.mean(np.concatenate([r.ravel() for r in refs]) ** 2))
    assert e_off <= 2 * e_base + 1e-3 * rms, (e_off / rms, e_base / rms)
