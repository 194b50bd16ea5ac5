"""Host-side checks of the seeded workload generator (CPU only)."""

import numpy as np
import pytest
import torch

from mla_inputs import SPECS, WorkloadSpec, make_workload, quantize_fp8_rows, fp8_row_stride
from oracle import formats


def test_fp8_stride_and_payload():
    assert fp8_row_stride(576) == 608
    assert fp8_row_stride(512) == 528


def test_quantizer_roundtrip_within_e4m3_precision():
    g = torch.Generator().manual_seed(3)
    x = torch.randn((257, 576), generator=g)
    x[5] = 0.0                                   # all-zero row -> scale byte 127
    x[7, :32] *= 1e-30                           # tiny group
    x[9, 100] = 1e4                              # outlier
    enc = quantize_fp8_rows(x, 576, 608)
    dec = formats.decode_fp8_rows(enc, 576)
    assert np.isfinite(dec).all()
    xs = x.double().numpy()
    # per group, error is at most half an e4m3 ulp at the group's scale
    amax = np.abs(xs.reshape(257, 18, 32)).max(-1)
    scale = formats.E8M0_LUT[enc[:, 576:594]]
    assert (amax <= 448 * scale + 0).all()
    err = np.abs(dec - xs).reshape(257, 18, 32).max(-1)
    assert (err <= scale * 2.0 ** 8 * 2.0 ** -4 + 1e-300).all()   # 448 = 1.75*2^8, ulp at top = 2^5
    assert (enc[5, 576:594] == 127).all() and (dec[5] == 0).all()
    assert (enc[:, 594:] == 0xFF).all()
    codes = enc[:, :576]
    assert not np.isin(codes, [0x7F, 0xFF]).any()


def test_workload_is_deterministic_and_poisoned():
    spec = SPECS["mtp2_b128_small"]
    a = make_workload(spec)
    b = make_workload(spec)
    for name in ("q_bits", "pool", "block_table", "seq_lens"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    c = make_workload(spec, seed=spec.seed + 1)
    assert not np.array_equal(a.q_bits, c.q_bits)
    # block table: each used page appears once, entries beyond a sequence are -1
    pages = (a.seq_lens + 63) // 64
    used = np.concatenate([a.block_table[i, :pages[i]] for i in range(spec.batch)])
    assert len(np.unique(used)) == used.size == pages.sum()
    assert (used >= 0).all() and (used < a.pool.shape[0]).all()
    for i in range(spec.batch):
        assert (a.block_table[i, pages[i]:] == -1).all()
        L = int(a.seq_lens[i])
        if L % 64:
            tail = a.pool[a.block_table[i, pages[i] - 1], L % 64:]
            assert (tail == 0x7FC0).all()
    spare = np.setdiff1d(np.arange(a.pool.shape[0]), used)
    assert spare.size == spec.spare_pages
    assert (a.pool[spare] == 0x7FC0).all()
    # used slots are finite bf16
    live = np.concatenate([a.pool[a.block_table[i, :pages[i]]].reshape(-1, 576)[:a.seq_lens[i]]
                           for i in range(spec.batch)])
    assert np.isfinite(formats.bf16_bits_to_f64(live)).all()


@pytest.mark.parametrize("name", ["single_1k", "paged_b32", "long_ctx_b4", "fp8_b64", "mtp2_b128"])
def test_full_specs_shapes(name):
    spec = SPECS[name]
    assert spec.n_h == 128 and spec.d_c == 512 and spec.d_r == 64 and spec.page == 64
    kind = spec.seq_lens[0]
    if kind == "fixed":
        assert len(spec.seq_lens[1]) == spec.batch
    else:
        # draw only the lengths (cheap): same generator order as make_workload
        from mla_inputs.workloads import _draw_seq_lens
        g = torch.Generator().manual_seed(spec.seed)
        lens = _draw_seq_lens(spec, g)
        lo, hi = spec.seq_lens[1], spec.seq_lens[2]
        assert lens.min() >= lo and lens.max() <= hi and lens.size == spec.batch


def test_fp8_workload_has_outliers_and_poison():
    w = make_workload(SPECS["fp8_b64_small"])
    pages = (w.seq_lens + 63) // 64
    live = np.concatenate([w.pool[w.block_table[i, :pages[i]]].reshape(-1, 608)[:w.seq_lens[i]]
                           for i in range(w.spec.batch)])
    dec = formats.decode_fp8_rows(live, 576)
    assert np.isfinite(dec).all()
    assert np.abs(dec).max() > 20          # outliers x20 survive quantisation
    assert (live[:, 594:] == 0xFF).all()
