"""Absorbed MLA decode over a paged latent cache, written out in float64.

Test infrastructure only (see ``oracle/__init__``).

What is computed ("DeepSeek R1 Architecture & Deployment Guide", section 1.1)
----------------------------------------------------------------------------
Each cached token t holds one row shared by all heads, the concatenation of
the compressed latent c_t (d_c = 512 values) and the decoupled, already
rotated RoPE key k^R_t (d_R = 64 values): 576 elements.  With the key
up-projection absorbed into the query, head i of query position j scores
token t as

    s_t = scale * ( q_abs[i] . c_t  +  q_R[i] . k^R_t )

and, because the value up-projection is absorbed into the output projection
(applied downstream, outside this operation), the attention output of head i
stays in latent space:

    out[i] = sum_t softmax(s)_t * c_t          (a d_c-vector)
    lse[i] = log sum_t exp(s_t)                (natural log)

Readings where the pages leave a step open (each is listed in the design doc):

* The query row arrives as q_abs (d_c values) followed by q_R (d_R values),
  the cache's own order; q is bf16.
* Pages: the "DeepSeek-R1" record, engine kernel constraint (1), instantiates
  decode kernels per page-block size and names 64.  Logical token t of
  sequence b lives in physical page block_table[b][t // page], slot
  t % page.
* Several queries per sequence (multi-token decode): seq_lens[b] counts all
  cached tokens including the s_q new ones; query j sits at position
  L - s_q + j and sees tokens 0 .. L - s_q + j (causal).  With s_q = 1 it
  sees all L tokens.
* A query that sees no token gets out = 0 and lse = -inf.

The oracle decodes exactly the bytes the GPU reads (tail slots, spare pages
and row padding are never touched) and then runs every step in float64.
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from . import formats


def gather_rows(pool: np.ndarray, block_table_row: np.ndarray, n_tokens: int,
                page: int) -> np.ndarray:
    """Logical rows 0..n_tokens-1 of one sequence, gathered through its block table.

    ``pool`` is [num_pages, page, row_len] (raw bit patterns / bytes).
    Returns [n_tokens, row_len] of the same raw dtype.
    """
    n_pages = -(-n_tokens // page)
    ids = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    if n_pages and (ids.min() < 0 or ids.max() >= pool.shape[0]):
        raise ValueError("block table entry outside the page pool")
    rows = pool[ids].reshape(n_pages * page, pool.shape[-1])
    return rows[:n_tokens]


def decode_rows(raw_rows: np.ndarray, kv_dtype: str, d: int) -> np.ndarray:
    if kv_dtype == "bf16":
        return formats.decode_bf16_rows(raw_rows, d)
    if kv_dtype == "fp8":
        return formats.decode_fp8_rows(raw_rows, d)
    if kv_dtype == "fp4":
        return formats.decode_fp4_rows(raw_rows, d)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def attend_one_query(q_rows: np.ndarray, kv_rows: np.ndarray, d_c: int,
                     softmax_scale: float):
    """One query position, all heads, float64.

    q_rows  [n_h, d_c + d_R]   (q_abs || q_R)
    kv_rows [n, d_c + d_R]     (c || k_R), the visible tokens only
    returns out [n_h, d_c], lse [n_h]
    """
    n_h = q_rows.shape[0]
    n = kv_rows.shape[0]
    if n == 0:
        return np.zeros((n_h, d_c)), np.full(n_h, -np.inf)
    q_abs, q_rope = q_rows[:, :d_c], q_rows[:, d_c:]
    c_lat, k_rope = kv_rows[:, :d_c], kv_rows[:, d_c:]
    # score = latent part + decoupled RoPE part, both against the shared row
    scores = softmax_scale * (q_abs @ c_lat.T + q_rope @ k_rope.T)   # [n_h, n]
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    z = e.sum(axis=1)
    out = (e @ c_lat) / z[:, None]
    lse = m[:, 0] + np.log(z)
    return out, lse


def mla_decode_ref(q_bits: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                   seq_lens: np.ndarray, *, kv_dtype: str, d_c: int, d_r: int,
                   page: int, softmax_scale: float,
                   batches: Optional[Iterable[int]] = None,
                   heads: Optional[Iterable[int]] = None):
    """Reference MLA decode.

    q_bits      uint16 [B, s_q, n_h, d_c + d_r]  bf16 bit patterns
    pool        bf16: uint16 [P, page, d_c + d_r];  fp8: uint8 [P, page, stride]
    block_table int32  [B, max_blocks]
    seq_lens    int32  [B]
    batches     optional subset of sequences to evaluate (others left NaN)
    heads       optional subset of heads to evaluate (others left NaN)

    Returns out float64 [B, s_q, n_h, d_c] and lse float64 [B, s_q, n_h].
    """
    q_bits = np.asarray(q_bits)
    B, s_q, n_h, d = q_bits.shape
    if d != d_c + d_r:
        raise ValueError("query row length must be d_c + d_r")
    out = np.full((B, s_q, n_h, d_c), np.nan)
    lse = np.full((B, s_q, n_h), np.nan)
    batch_list = range(B) if batches is None else list(batches)
    head_idx = np.arange(n_h) if heads is None else np.asarray(list(heads), dtype=np.int64)
    for b in batch_list:
        L = int(seq_lens[b])
        n_max = max(L, 0)
        raw = gather_rows(pool, block_table[b], n_max, page) if n_max else pool[:0, 0]
        rows = decode_rows(raw, kv_dtype, d) if n_max else np.zeros((0, d))
        for j in range(s_q):
            n_vis = max(L - s_q + 1 + j, 0)        # causal: position L - s_q + j
            qf = formats.bf16_bits_to_f64(q_bits[b, j][head_idx])
            o, l_ = attend_one_query(qf, rows[:n_vis], d_c, softmax_scale)
            out[b, j, head_idx] = o
            lse[b, j, head_idx] = l_
    return out, lse

