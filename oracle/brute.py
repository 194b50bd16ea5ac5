"""Pure-Python brute force for tiny inputs.

Test infrastructure only (see ``oracle/__init__``).

It walks the same definition as ``oracle.mla`` (guide section 1.1: score =
scale * (q_abs . c + q_R . k_R), softmax over visible tokens, output the
softmax-weighted latents) one scalar at a time, with ``math.exp`` and plain
loops, and reads the cache through its own decoding path: bf16 through
``struct``, FP8 through torch's float8_e4m3fn / float8_e8m0fnu dtypes and FP4
through its own nibble and exponent arithmetic, not through the oracle's
lookup tables.  It therefore checks the vectorised
oracle's gathering, slicing, masking and reductions independently.
"""

from __future__ import annotations

import math
import struct

import numpy as np


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _fp8_row_values(row_bytes, d: int):
    import torch  # library routine for the byte formats
    raw = torch.tensor(list(int(x) for x in row_bytes[:d + d // 32]), dtype=torch.uint8)
    codes = raw[:d].view(torch.float8_e4m3fn).to(torch.float64).tolist()
    scales = raw[d:].view(torch.float8_e8m0fnu).to(torch.float64).tolist()
    return [codes[i] * scales[i // 32] for i in range(d)]


def _fp4_row_values(row_bytes, d: int):
    # e2m1 written as (2 + m) * 2^(e - 2) for e > 0 and m * 2^-1 for e = 0;
    # element 2i in the low nibble of byte i; scale byte g for elements 16g..
    vals = []
    for i in range(d):
        byte = int(row_bytes[i // 2])
        nib = (byte >> (4 * (i % 2))) & 0xF
        e, m = (nib >> 1) & 3, nib & 1
        mag = m * 0.5 if e == 0 else (2 + m) * 2.0 ** (e - 2)
        scale = 2.0 ** (int(row_bytes[d // 2 + i // 16]) - 127)
        vals.append((-mag if nib & 8 else mag) * scale)
    return vals


def _row_values(pool, page_id: int, slot: int, kv_dtype: str, d: int):
    row = pool[page_id][slot]
    if kv_dtype == "bf16":
        return [_bf16(row[i]) for i in range(d)]
    if kv_dtype == "fp4":
        return _fp4_row_values(row, d)
    return _fp8_row_values(row, d)


def mla_decode_brute(q_bits, pool, block_table, seq_lens, *, kv_dtype: str, d_c: int,
                     d_r: int, page: int, softmax_scale: float):
    B, s_q, n_h, d = np.asarray(q_bits).shape
    out = [[[[0.0] * d_c for _ in range(n_h)] for _ in range(s_q)] for _ in range(B)]
    lse = [[[0.0] * n_h for _ in range(s_q)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        rows = []
        for t in range(L):
            rows.append(_row_values(pool, int(block_table[b][t // page]), t % page, kv_dtype, d))
        for j in range(s_q):
            n_vis = max(L - s_q + 1 + j, 0)
            for h in range(n_h):
                q = [_bf16(x) for x in q_bits[b][j][h]]
                if n_vis == 0:
                    lse[b][j][h] = -math.inf
                    continue
                scores = []
                for t in range(n_vis):
                    acc = 0.0
                    for i in range(d_c):
                        acc += q[i] * rows[t][i]
                    for i in range(d_c, d_c + d_r):
                        acc += q[i] * rows[t][i]
                    scores.append(softmax_scale * acc)
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = sum(w)
                for i in range(d_c):
                    acc = 0.0
                    for t in range(n_vis):
                        acc += w[t] * rows[t][i]
                    out[b][j][h][i] = acc / z
                lse[b][j][h] = m + math.log(z)
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)


def mla_sparse_decode_brute(q_bits, pool, block_table, seq_lens, indices, *, kv_dtype: str, d_c: int,
                            d_r: int, page: int, softmax_scale: float):
    """The sparse (top-k) decode one scalar at a time: query j of sequence b
    attends to the listed tokens t with 0 <= t < L - s_q + 1 + j only."""
    B, s_q, n_h, d = np.asarray(q_bits).shape
    out = [[[[0.0] * d_c for _ in range(n_h)] for _ in range(s_q)] for _ in range(B)]
    lse = [[[0.0] * n_h for _ in range(s_q)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(s_q):
            n_vis = max(L - s_q + 1 + j, 0)
            toks = [int(t) for t in indices[b][j] if 0 <= int(t) < n_vis]
            rows = [_row_values(pool, int(block_table[b][t // page]), t % page, kv_dtype, d) for t in toks]
            for h in range(n_h):
                q = [_bf16(x) for x in q_bits[b][j][h]]
                if not rows:
                    lse[b][j][h] = -math.inf
                    continue
                scores = []
                for row in rows:
                    acc = 0.0
                    for i in range(d):
                        acc += q[i] * row[i]
                    scores.append(softmax_scale * acc)
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = sum(w)
                for i in range(d_c):
                    acc = 0.0
                    for t in range(len(rows)):
                        acc += w[t] * rows[t][i]
                    out[b][j][h][i] = acc / z
                lse[b][j][h] = m + math.log(z)
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)
