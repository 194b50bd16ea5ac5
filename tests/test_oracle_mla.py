"""Pins for oracle/mla.py (CPU only).

What pins the absorbed-MLA oracle, none of which retypes its formula:
  * the absorption identity against the un-absorbed MHA on materialised
    per-head keys and values (guide section 1.1 derivation);
  * a pure-Python brute force (own decoding path) on tiny paged inputs, both
    cache dtypes, one and two queries per sequence, lengths crossing page
    edges, poisoned tails and spare pages;
  * closed forms: one visible token, q = 0 (plain mean, lse = log n),
    constant latent rows (convex combination), q_R = 0 (k_R irrelevant), a
    dominant token;
  * the log-sum-exp split/merge identity that the GPU combine relies on;
  * a mutation check: plausible mistakes planted in the oracle must each
    fail at least one of these pins.
"""

import dataclasses
import math

import numpy as np
import pytest

import oracle
from oracle import mla, unabsorbed, brute, formats
from mla_inputs import WorkloadSpec, make_workload


def _tiny_spec(kv_dtype, s_q, seed, lens=(1, 64, 65, 130), n_h=2, d_c=512):
    return WorkloadSpec(f"tiny_{kv_dtype}_{s_q}_{d_c}", len(lens), ("fixed", tuple(lens)), kv_dtype=kv_dtype,
                        s_q=s_q, n_h=n_h, spare_pages=3, seed=seed, d_c=d_c,
                        outlier_p=0.05 if kv_dtype != "bf16" else 0.0, outlier_mult=20.0)


def _run_oracle(w, **kw):
    s = w.spec
    return mla.mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=s.kv_dtype,
                              d_c=s.d_c, d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale, **kw)


# ----------------------------------------------------------------------------
# the pins, written as functions so the mutation test can re-run them
# ----------------------------------------------------------------------------

def pin_brute_force(kv_dtype, s_q, d_c=512):
    w = make_workload(_tiny_spec(kv_dtype, s_q, seed=100 + s_q + {"bf16": 0, "fp8": 7, "fp4": 13}[kv_dtype]
                                 + (0 if d_c == 512 else 50), d_c=d_c))
    s = w.spec
    out, lse = _run_oracle(w)
    bo, bl = brute.mla_decode_brute(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=s.kv_dtype,
                                    d_c=s.d_c, d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale)
    np.testing.assert_allclose(out, bo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def pin_absorption(seed=3):
    rng = np.random.default_rng(seed)
    n_h, d_h, d_c, d_r, n = 4, 16, 32, 8, 37
    w_uk = rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c)
    q_c = rng.standard_normal((n_h, d_h))
    q_r = rng.standard_normal((n_h, d_r))
    c = rng.standard_normal((n, d_c))
    k_r = rng.standard_normal((n, d_r))
    scale = 1.0 / math.sqrt(d_h + d_r)
    o_mha = unabsorbed.mha_materialised(q_c, q_r, w_uk, w_uv, c, k_r, scale)
    q_rows = unabsorbed.absorb_query(q_c, q_r, w_uk)
    latent, _ = mla.attend_one_query(q_rows, np.concatenate([c, k_r], axis=1), d_c, scale)
    o_abs = unabsorbed.apply_value_projection(latent, w_uv)
    np.testing.assert_allclose(o_abs, o_mha, rtol=1e-10, atol=1e-12)


def pin_special_cases(seed=9):
    rng = np.random.default_rng(seed)
    n_h, d_c, d_r = 3, 512, 64
    d = d_c + d_r
    scale = 1.0 / math.sqrt(192.0)
    rows = rng.standard_normal((50, d))
    q = rng.standard_normal((n_h, d))
    # one visible token: out = its latent, lse = its score
    o, l_ = mla.attend_one_query(q, rows[:1], d_c, scale)
    np.testing.assert_allclose(o, np.broadcast_to(rows[0, :d_c], o.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(l_, scale * (q @ rows[0]), rtol=1e-13)
    # q = 0: uniform weights -> plain mean, lse = log n
    o, l_ = mla.attend_one_query(np.zeros((n_h, d)), rows, d_c, scale)
    np.testing.assert_allclose(o, np.broadcast_to(np.mean(rows[:, :d_c], axis=0), o.shape), atol=1e-13)
    np.testing.assert_allclose(l_, math.log(rows.shape[0]), rtol=1e-14)
    # constant latent rows: any convex combination gives the constant back
    const = rows.copy()
    const[:, :d_c] = rows[0, :d_c]
    o, _ = mla.attend_one_query(q, const, d_c, scale)
    np.testing.assert_allclose(o, np.broadcast_to(rows[0, :d_c], o.shape), atol=1e-12)
    # q_R = 0: the RoPE keys must not matter
    q0 = q.copy()
    q0[:, d_c:] = 0
    r2 = rows.copy()
    r2[:, d_c:] = rng.standard_normal((rows.shape[0], d_r)) * 50
    o1, l1 = mla.attend_one_query(q0, rows, d_c, scale)
    o2, l2 = mla.attend_one_query(q0, r2, d_c, scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    # RoPE part alone moves the result: q_abs = 0, large q_R aligned with one token's k_R
    q_r_only = np.zeros((1, d))
    q_r_only[0, d_c:] = rows[17, d_c:] * 40
    o, _ = mla.attend_one_query(q_r_only, rows, d_c, scale)
    np.testing.assert_allclose(o[0], rows[17, :d_c], atol=1e-6)
    # dominant token through the latent part
    q_dom = np.zeros((1, d))
    q_dom[0, :d_c] = rows[23, :d_c] * 40
    o, _ = mla.attend_one_query(q_dom, rows, d_c, scale)
    np.testing.assert_allclose(o[0], rows[23, :d_c], atol=1e-6)


def pin_split_merge(seed=4):
    rng = np.random.default_rng(seed)
    n_h, d_c, d = 5, 512, 576
    rows = rng.standard_normal((300, d))
    q = rng.standard_normal((n_h, d))
    scale = 1.0 / math.sqrt(192.0)
    o_full, l_full = mla.attend_one_query(q, rows, d_c, scale)
    cuts = [0, 64, 65, 191, 300]
    parts = [mla.attend_one_query(q, rows[a:b], d_c, scale) for a, b in zip(cuts[:-1], cuts[1:])]
    lses = np.stack([p[1] for p in parts])                  # [S, n_h]
    big = lses.max(axis=0)
    lse = big + np.log(np.exp(lses - big).sum(axis=0))
    o = sum(np.exp(p[1] - lse)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(lse, l_full, rtol=1e-13)
    np.testing.assert_allclose(o, o_full, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------
# the real oracle passes every pin
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("s_q", [1, 2])
def test_oracle_matches_brute_force(kv_dtype, s_q):
    pin_brute_force(kv_dtype, s_q)


@pytest.mark.parametrize("s_q", [1, 2])
def test_oracle_matches_brute_force_on_the_528_byte_fp8_row(s_q):
    # d_c = 448 + d_r = 64: the record's 512-dim row, 528 bytes, no padding
    pin_brute_force("fp8", s_q, d_c=448)


def test_absorbed_equals_unabsorbed():
    pin_absorption()


def test_special_cases():
    pin_special_cases()


def test_split_merge_identity():
    pin_split_merge()


def test_poison_is_never_read():
    # changing every poisoned byte must not change the oracle's result
    w = make_workload(_tiny_spec("fp8", 2, seed=21, lens=(2, 64, 65, 130)))
    out1, lse1 = _run_oracle(w)
    used = set()
    for b in range(w.spec.batch):
        L = int(w.seq_lens[b])
        for t in range(L):
            used.add((int(w.block_table[b, t // 64]), t % 64))
    pool2 = w.pool.copy()
    for p in range(pool2.shape[0]):
        for s_ in range(64):
            if (p, s_) not in used:
                pool2[p, s_] = 0x11
    pool2[:, :, 594:] = 0x22                                  # row padding
    w2 = dataclasses.replace(w, pool=pool2)
    out2, lse2 = _run_oracle(w2)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)
    assert np.isfinite(out1).all() and np.isfinite(lse1).all()


def test_sampled_batches_match_full_run():
    w = make_workload(_tiny_spec("bf16", 1, seed=31, lens=(70, 3, 129), n_h=3))
    out, lse = _run_oracle(w)
    o2, l2 = _run_oracle(w, batches=[2], heads=[1, 2])
    np.testing.assert_array_equal(o2[2, :, 1:], out[2, :, 1:])
    np.testing.assert_array_equal(l2[2, :, 1:], lse[2, :, 1:])
    assert np.isnan(o2[0]).all() and np.isnan(o2[2, :, 0]).all()


def test_no_visible_token_gives_zero_and_minus_inf():
    # L < s_q: query 0 sees nothing (precondition violation, defined result)
    w = make_workload(_tiny_spec("bf16", 2, seed=41, lens=(1, 5)))
    out, lse = _run_oracle(w)
    assert np.all(out[0, 0] == 0) and np.all(lse[0, 0] == -np.inf)
    assert np.isfinite(out[0, 1]).all() and np.isfinite(lse[1]).all()


# ----------------------------------------------------------------------------
# mutation check: each planted mistake fails at least one pin
# ----------------------------------------------------------------------------

def _mutant(kind):
    real = mla.attend_one_query

    def attend(q_rows, kv_rows, d_c, softmax_scale):
        n_h = q_rows.shape[0]
        if kind == "drop_last_token" and kv_rows.shape[0] > 1:
            kv_rows = kv_rows[:-1]
        if kv_rows.shape[0] == 0:
            return np.zeros((n_h, d_c)), np.full(n_h, -np.inf)
        q_abs, q_rope = q_rows[:, :d_c], q_rows[:, d_c:]
        c_lat, k_rope = kv_rows[:, :d_c], kv_rows[:, d_c:]
        if kind == "drop_rope_term":
            scores = softmax_scale * (q_abs @ c_lat.T)
        elif kind == "no_scale":
            scores = q_abs @ c_lat.T + q_rope @ k_rope.T
        elif kind == "rope_sign":
            scores = softmax_scale * (q_abs @ c_lat.T - q_rope @ k_rope.T)
        elif kind in ("shifted_latent", "lse_without_max", "drop_last_token"):
            scores = softmax_scale * (q_abs @ c_lat.T + q_rope @ k_rope.T)
        else:
            return real(q_rows, kv_rows, d_c, softmax_scale)
        m = scores.max(axis=1, keepdims=True)
        e = np.exp(scores - m)
        z = e.sum(axis=1)
        value = kv_rows[:, 1:d_c + 1] if kind == "shifted_latent" else c_lat
        out = (e @ value) / z[:, None]
        lse = (np.log(z) if kind == "lse_without_max" else m[:, 0] + np.log(z))
        return out, lse
    return attend


@pytest.mark.parametrize("kind", ["drop_rope_term", "no_scale", "rope_sign", "shifted_latent",
                                  "drop_last_token", "lse_without_max"])
def test_planted_mistakes_fail_a_pin(kind, monkeypatch):
    monkeypatch.setattr(mla, "attend_one_query", _mutant(kind))
    failures = 0
    for pin in (lambda: pin_brute_force("bf16", 1), lambda: pin_brute_force("fp8", 2),
                pin_absorption, pin_special_cases, pin_split_merge):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"mutant {kind} passed every pin"
