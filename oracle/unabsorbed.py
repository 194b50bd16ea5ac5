"""MLA in its explicit, un-absorbed form -- the cross-check for absorption.

Test infrastructure only (see ``oracle/__init__``).

"DeepSeek R1 Architecture & Deployment Guide", section 1 defines the low-rank
projections: the latent c_t = W^DKV h_t, and per head i the up-projected key
k^C_{t,i} = W_i^UK c_t and value v^C_{t,i} = W_i^UV c_t (d_h = 128 rows each).
Section 1.1 adds the decoupled RoPE: the key of head i is [k^C_{t,i} ; k^R_t]
with one k^R_t shared by all heads, and the query is [q^C_i ; q^R_i].

Standard attention on those materialised keys and values,

    o_i = sum_t softmax_t(scale * [q^C_i ; q^R_i] . [W_i^UK c_t ; k^R_t]) W_i^UV c_t,

must equal the absorbed form: q_abs_i = (W_i^UK)^T q^C_i scored against the
shared row [c_t ; k^R_t], output W_i^UV applied to the latent result (the
identity printed in section 1.1, plus associativity for the value side).
"""

from __future__ import annotations

import numpy as np


def mha_materialised(q_c: np.ndarray, q_r: np.ndarray, w_uk: np.ndarray,
                     w_uv: np.ndarray, c: np.ndarray, k_r: np.ndarray,
                     softmax_scale: float) -> np.ndarray:
    """Per-head attention on explicitly up-projected keys/values.

    q_c  [n_h, d_h]      per-head compressed-part query (W^UQ c^Q)
    q_r  [n_h, d_R]      per-head RoPE query
    w_uk [n_h, d_h, d_c] key up-projection per head
    w_uv [n_h, d_h, d_c] value up-projection per head
    c    [n, d_c]        latents
    k_r  [n, d_R]        shared RoPE keys
    returns o [n_h, d_h]
    """
    n_h = q_c.shape[0]
    out = np.zeros((n_h, w_uv.shape[1]))
    for i in range(n_h):
        k_ci = c @ w_uk[i].T                    # [n, d_h]  k^C_{t,i}
        v_ci = c @ w_uv[i].T                    # [n, d_h]  v^C_{t,i}
        keys = np.concatenate([k_ci, k_r], axis=1)
        query = np.concatenate([q_c[i], q_r[i]])
        s = softmax_scale * (keys @ query)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[i] = p @ v_ci
    return out


def absorb_query(q_c: np.ndarray, q_r: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_abs_i = (W_i^UK)^T q^C_i, concatenated with q^R_i -> [n_h, d_c + d_R]."""
    q_abs = np.einsum("hdc,hd->hc", w_uk, q_c)
    return np.concatenate([q_abs, q_r], axis=1)


def apply_value_projection(latent_out: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o_i = W_i^UV latent_i -> [n_h, d_h]."""
    return np.einsum("hdc,hc->hd", w_uv, latent_out)
