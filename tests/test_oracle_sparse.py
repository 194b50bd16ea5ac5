"""Pins for oracle/sparse.py, the top-k decode ("DeepSeek-V3.2" record) (CPU only).

What pins it, none of which retypes its formula:
  * a pure-Python brute force (own cache decoding, own selection loop) on
    tiny paged inputs: both cache dtypes, one and two queries per sequence,
    index lists in random order with -1 padding, entries past the causal
    limit and past the sequence;
  * reduction to the dense decode: an index list holding every visible
    token, in any order, gives the dense oracle's result (itself pinned by
    test_oracle_mla.py);
  * closed forms: one selected token, an empty selection;
  * unselected rows are never read (NaN-poisoned rows change nothing);
  * a mutation check: plausible mistakes planted in the selection must
    each fail one of these pins.
"""

import dataclasses

import numpy as np
import pytest

from oracle import brute, mla, sparse
from mla_inputs import WorkloadSpec, make_workload


def _tiny(kv_dtype, s_q, seed, topk=40, lens=(1, 64, 65, 130)):
    return make_workload(WorkloadSpec(f"tiny_sparse_{kv_dtype}_{s_q}", len(lens), ("fixed", tuple(lens)),
                                      kv_dtype=kv_dtype, s_q=s_q, n_h=2, spare_pages=3, topk=topk, seed=seed,
                                      outlier_p=0.05 if kv_dtype == "fp8" else 0.0, outlier_mult=20.0))


def _sparse(w, indices=None, **kw):
    s = w.spec
    return sparse.mla_sparse_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens,
                                        w.indices if indices is None else indices, kv_dtype=s.kv_dtype,
                                        d_c=s.d_c, d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale, **kw)


def _dense(w):
    s = w.spec
    return mla.mla_decode_ref(w.q_bits, w.pool, w.block_table, w.seq_lens, kv_dtype=s.kv_dtype, d_c=s.d_c,
                              d_r=s.d_r, page=s.page, softmax_scale=s.softmax_scale)


def _with_bad_entries(w, seed):
    """Index lists with entries the decode must ignore: past the causal
    limit (but inside the sequence), past the sequence, and large values."""
    rng = np.random.default_rng(seed)
    idx = w.indices.copy()
    B, s_q, k = idx.shape
    for b in range(B):
        L = int(w.seq_lens[b])
        for j in range(s_q):
            n_vis = max(L - s_q + 1 + j, 0)
            pad = np.flatnonzero(idx[b, j] < 0)
            bad = [n_vis, L + 5, 1 << 30, -7]            # n_vis < L when j < s_q - 1
            for p, v in zip(pad, bad):
                idx[b, j, p] = v
            rng.shuffle(idx[b, j])
    return idx


# ----------------------------------------------------------------------------
# pins, as functions so the mutation test can re-run them
# ----------------------------------------------------------------------------

def pin_brute_force(kv_dtype, s_q):
    w = _tiny(kv_dtype, s_q, seed=300 + s_q + (5 if kv_dtype == "fp8" else 0))
    idx = _with_bad_entries(w, seed=s_q)
    s = w.spec
    out, lse = _sparse(w, idx)
    bo, bl = brute.mla_sparse_decode_brute(w.q_bits, w.pool, w.block_table, w.seq_lens, idx,
                                           kv_dtype=s.kv_dtype, d_c=s.d_c, d_r=s.d_r, page=s.page,
                                           softmax_scale=s.softmax_scale)
    np.testing.assert_allclose(out, bo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def pin_full_selection_is_dense(kv_dtype, s_q):
    # topk above every context length: each list holds all visible tokens
    w = _tiny(kv_dtype, s_q, seed=320 + s_q, topk=200)
    assert all((w.indices[b, j] >= 0).sum() == max(int(w.seq_lens[b]) - s_q + 1 + j, 0)
               for b in range(w.spec.batch) for j in range(s_q))
    so, sl = _sparse(w)
    do, dl = _dense(w)
    np.testing.assert_allclose(so, do, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sl, dl, rtol=1e-13, atol=0)


def pin_single_and_empty():
    w = _tiny("bf16", 1, seed=331, lens=(300, 5))
    idx = np.full_like(w.indices, -1)
    idx[0, 0, 7] = 123                           # one token
    out, lse = _sparse(w, idx)
    s = w.spec
    row = w.pool[w.block_table[0, 123 // 64], 123 % 64].astype(np.uint32) << 16
    vals = row.view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(out[0, 0], np.broadcast_to(vals[:s.d_c], out[0, 0].shape))
    q = (w.q_bits[0, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(lse[0, 0], s.softmax_scale * (q @ vals), rtol=1e-13)
    # sequence 1 selects nothing: out = 0, lse = -inf
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)


def pin_unselected_rows_never_read():
    w = _tiny("fp8", 2, seed=340, topk=30, lens=(200, 170))
    out, lse = _sparse(w)
    pool = w.pool.copy()
    keep = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(w.spec.batch):
        for j in range(w.spec.s_q):
            n_vis = int(w.seq_lens[b]) - w.spec.s_q + 1 + j
            for t in w.indices[b, j]:
                if 0 <= t < n_vis:
                    keep[w.block_table[b, t // 64], t % 64] = True
    pool[~keep] = 0x7F                            # NaN codes and NaN scales
    w2 = dataclasses.replace(w, pool=pool)
    out2, lse2 = _sparse(w2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


# ----------------------------------------------------------------------------
# the real oracle passes every pin
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("s_q", [1, 2])
def test_sparse_matches_brute_force(kv_dtype, s_q):
    pin_brute_force(kv_dtype, s_q)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("s_q", [1, 2])
def test_full_selection_equals_dense(kv_dtype, s_q):
    pin_full_selection_is_dense(kv_dtype, s_q)


def test_single_token_and_empty_selection():
    pin_single_and_empty()


def test_unselected_rows_never_read():
    pin_unselected_rows_never_read()


def test_generator_index_lists():
    w = make_workload("sparse_topk2048_b64_small")
    k = w.spec.topk
    for b in range(w.spec.batch):
        n_vis = int(w.seq_lens[b])
        row = w.indices[b, 0]
        valid = row[row >= 0]
        assert valid.size == min(n_vis, k) and np.unique(valid).size == valid.size
        assert valid.max() < n_vis and np.all(row[valid.size:] == -1)
    assert w.selected_tokens == sum(min(int(L), k) for L in w.seq_lens)


# ----------------------------------------------------------------------------
# mutation check: mistakes planted in the selection fail a pin
# ----------------------------------------------------------------------------

def _mutant(kind):
    real = sparse.selected_tokens

    def sel(indices_bj, n_vis):
        idx = np.asarray(indices_bj, dtype=np.int64)
        if kind == "inclusive_limit":
            return idx[(idx >= 0) & (idx <= n_vis)]
        if kind == "no_causal_limit":
            return idx[idx >= 0]
        if kind == "drop_last":
            return real(indices_bj, n_vis)[:-1]
        if kind == "first_only":
            return real(indices_bj, n_vis)[:1]
        raise AssertionError(kind)
    return sel


@pytest.mark.parametrize("kind", ["inclusive_limit", "no_causal_limit", "drop_last", "first_only"])
def test_planted_mistakes_fail_a_pin(kind, monkeypatch):
    monkeypatch.setattr(sparse, "selected_tokens", _mutant(kind))
    failed = 0
    for pin in (lambda: pin_brute_force("bf16", 2), lambda: pin_full_selection_is_dense("bf16", 2),
                pin_single_and_empty):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"mutation {kind} passed every pin"
