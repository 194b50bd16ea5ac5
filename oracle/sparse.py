"""Sparse (top-k) MLA decode, written out in float64.

Test infrastructure only (see ``oracle/__init__``).

What is computed ("DeepSeek-V3.2" model record: the MLA skeleton and the
576-element latent cache row are unchanged; a lightweight top-k selector
with index_topk = 2048 picks, for every query token, the candidate tokens
it attends over instead of the whole context): for query position j of
sequence b the absorbed MLA decode of ``oracle.mla``, restricted to the
tokens listed in indices[b][j]:

    S     = { t in indices[b][j] : 0 <= t < n_vis }      (as listed)
    s_t   = scale * ( q_abs . c_t + q_R . k^R_t )         for t in S
    out   = sum_{t in S} softmax(s)_t * c_t ,  lse = log sum_{t in S} exp(s_t)

Readings where the record leaves a step open (each is listed in the design doc):

* indices[b][j] holds up to topk logical token positions of sequence b;
  n_vis = L_b - s_q + 1 + j is the query's causal context (the same reading
  as the dense decode).  An entry outside [0, n_vis) -- the selector's -1
  padding when the context is shorter than topk, or anything else -- does
  not take part.
* Entries count as listed.  A top-k selector returns distinct positions; a
  repeated one would be counted once per listing.  The order is irrelevant.
* A query with no valid entry gets out = 0 and lse = -inf.
* Token t is read, like in the dense decode, from physical page
  block_table[b][t // page], slot t % page.
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from . import formats, mla


def selected_tokens(indices_bj: np.ndarray, n_vis: int) -> np.ndarray:
    """The entries of one query's index list that take part, in list order."""
    idx = np.asarray(indices_bj, dtype=np.int64)
    return idx[(idx >= 0) & (idx < n_vis)]


def mla_sparse_decode_ref(q_bits: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                          seq_lens: np.ndarray, indices: np.ndarray, *, kv_dtype: str, d_c: int,
                          d_r: int, page: int, softmax_scale: float,
                          batches: Optional[Iterable[int]] = None,
                          heads: Optional[Iterable[int]] = None):
    """Reference sparse MLA decode.

    q_bits      uint16 [B, s_q, n_h, d_c + d_r]  bf16 bit patterns
    pool        bf16: uint16 [P, page, d_c + d_r];  fp8: uint8 [P, page, stride]
    block_table int32  [B, max_blocks]
    seq_lens    int32  [B]
    indices     int32  [B, s_q, topk]   logical token positions (see above)
    batches / heads: optional subsets to evaluate (others left NaN)

    Returns out float64 [B, s_q, n_h, d_c] and lse float64 [B, s_q, n_h].
    """
    q_bits = np.asarray(q_bits)
    B, s_q, n_h, d = q_bits.shape
    if d != d_c + d_r:
        raise ValueError("query row length must be d_c + d_r")
    indices = np.asarray(indices)
    if indices.shape[:2] != (B, s_q):
        raise ValueError("indices must be [B, s_q, topk]")
    out = np.full((B, s_q, n_h, d_c), np.nan)
    lse = np.full((B, s_q, n_h), np.nan)
    batch_list = range(B) if batches is None else list(batches)
    head_idx = np.arange(n_h) if heads is None else np.asarray(list(heads), dtype=np.int64)
    for b in batch_list:
        L = int(seq_lens[b])
        for j in range(s_q):
            n_vis = max(L - s_q + 1 + j, 0)
            sel = selected_tokens(indices[b, j], n_vis)
            if sel.size:
                pages = np.asarray(block_table[b], dtype=np.int64)[sel // page]
                if pages.min() < 0 or pages.max() >= pool.shape[0]:
                    raise ValueError("block table entry outside the page pool")
                raw = pool[pages, sel % page]
                rows = mla.decode_rows(raw, kv_dtype, d)
            else:
                rows = np.zeros((0, d))
            qf = formats.bf16_bits_to_f64(q_bits[b, j][head_idx])
            o, l_ = mla.attend_one_query(qf, rows, d_c, softmax_scale)
            out[b, j, head_idx] = o
            lse[b, j, head_idx] = l_
    return out, lse
