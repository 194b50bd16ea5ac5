"""Closed-form cache sizes.

Test infrastructure only (see ``oracle/__init__``).

* "DeepSeek R1 Architecture & Deployment Guide", section 1: an MHA cache
  stores K and V, n_h * d_h values each, per token and layer.
* Same guide, section 1.1: the MLA row is concat(c, k_R), d_c + d_R values
  per token and layer; compression versus MHA is 1 - row / (2 n_h d_h).
* "DeepSeek-R1" record, intro: 61 layers x 576 values x 2 bytes per token.
* Same record, engine kernel constraint (2): an FP8 row is one e4m3 byte per
  dimension plus one e8m0 byte per 32 dimensions; its fp4 variant takes 288
  bytes at 512 dimensions.
"""

from __future__ import annotations


def mla_row_elements(d_c: int = 512, d_r: int = 64) -> int:
    return d_c + d_r


def mla_bytes_per_token(layers: int = 61, d_c: int = 512, d_r: int = 64,
                        bytes_per_elem: int = 2) -> int:
    return layers * mla_row_elements(d_c, d_r) * bytes_per_elem


def mla_bytes_per_sequence(seq_len: int, layers: int = 61, d_c: int = 512,
                           d_r: int = 64, bytes_per_elem: int = 2) -> int:
    return seq_len * mla_bytes_per_token(layers, d_c, d_r, bytes_per_elem)


def mha_bytes_per_sequence(seq_len: int, layers: int = 61, n_h: int = 128,
                           d_h: int = 128, bytes_per_elem: int = 2) -> int:
    return 2 * layers * n_h * d_h * seq_len * bytes_per_elem


def compression_vs_mha(d_c: int = 512, d_r: int = 64, n_h: int = 128,
                       d_h: int = 128) -> float:
    return 1.0 - mla_row_elements(d_c, d_r) / (2 * n_h * d_h)


def fp4_row_bytes(d: int) -> int:
    """Half a byte per dimension plus one scale byte per 16 dimensions (the
    reading of the record's 288-byte fp4 row at 512 dimensions)."""
    if d % 32:
        raise ValueError("d must be a multiple of 32")
    return d // 2 + d // 16


def fp8_row_bytes(d: int) -> int:
    """One e4m3 code per dimension plus one e8m0 scale per 32 dimensions."""
    if d % 32:
        raise ValueError("d must be a multiple of 32")
    return d + d // 32
