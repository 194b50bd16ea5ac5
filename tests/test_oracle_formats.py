"""Pins for oracle/formats.py and oracle/footprint.py (CPU only).

The number formats are pinned against library routines (torch's
float8_e4m3fn / float8_e8m0fnu / bfloat16 dtypes) over every code, and
against figures the pages print (tests/golden/page_figures.json).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats, footprint

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _figures():
    with open(GOLDEN) as f:
        return {x["name"]: x for x in json.load(f)["figures"]}


def _same_or_both_nan(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_e4m3fn_lut_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same_or_both_nan(formats.E4M3FN_LUT, ref)


def test_e4m3fn_max_normal_is_448_and_nan_codes():
    fig = _figures()["e4m3_max_normal"]["value"]
    finite = formats.E4M3FN_LUT[~np.isnan(formats.E4M3FN_LUT)]
    assert finite.max() == fig == 448.0
    assert formats.e4m3fn_value(0x7E) == 448.0
    assert math.isnan(formats.e4m3fn_value(0x7F)) and math.isnan(formats.e4m3fn_value(0xFF))
    assert np.isnan(formats.E4M3FN_LUT).sum() == 2          # only S.1111.111
    assert formats.e4m3fn_value(0x01) == 2.0 ** -9          # smallest subnormal
    assert formats.e4m3fn_value(0x08) == 2.0 ** -6          # smallest normal
    assert formats.e4m3fn_value(0x80) == 0.0 and math.copysign(1, formats.e4m3fn_value(0x80)) < 0


def test_e8m0_lut_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same_or_both_nan(formats.E8M0_LUT, ref)
    assert formats.e8m0_value(127) == 1.0
    assert formats.e8m0_value(0) == 2.0 ** -127
    assert math.isnan(formats.e8m0_value(255))


def test_bf16_widening_matches_torch():
    g = torch.Generator().manual_seed(11)
    bits = torch.randint(0, 65536, (4096,), generator=g, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_bits_to_f64(bits.numpy().view(np.uint16))
    assert _same_or_both_nan(got, ref)


def test_fp8_row_scale_groups_follow_32_value_blocks():
    # one row of 576 codes, 18 distinct scales; element i must use scale i // 32
    d = 576
    g = torch.Generator().manual_seed(5)
    codes = torch.randint(0, 126, (d,), generator=g, dtype=torch.int32).to(torch.uint8)
    scales = (torch.arange(d // 32, dtype=torch.int32) * 3 + 100).to(torch.uint8)
    row = np.full(608, 0xFF, dtype=np.uint8)      # padding poisoned: must be ignored
    row[:d] = codes.numpy()
    row[d:d + d // 32] = scales.numpy()
    got = formats.decode_fp8_rows(row[None, :], d)[0]
    cv = codes.view(torch.float8_e4m3fn).to(torch.float64)
    sv = scales.view(torch.float8_e8m0fnu).to(torch.float64)
    ref = (cv * sv.repeat_interleave(32)).numpy()
    np.testing.assert_array_equal(got, ref)
    # a wrong grouping (e.g. scale i % 18) must not agree
    wrong = (cv * sv[torch.arange(d) % (d // 32)]).numpy()
    assert not np.array_equal(got, wrong)


def test_e2m1_codes():
    from mla_inputs import E2M1_MAGNITUDES, quantize_fp4_rows
    lut = formats.E2M1_LUT
    assert lut.shape == (16,) and not np.isnan(lut).any()
    # sign in bit 3, magnitudes increasing with the code, largest 6
    np.testing.assert_array_equal(lut[8:], -lut[:8])
    assert np.all(np.diff(lut[:8]) > 0) and lut.max() == 6.0 and lut[0] == 0.0
    # the generator's encoder (a magnitude table with round-to-nearest-even)
    # and the oracle's bit-field decoder are inverse on every code
    np.testing.assert_array_equal(lut[:8], E2M1_MAGNITUDES)
    vals = torch.tensor([lut[list(range(16)) * 2]], dtype=torch.float32)     # 32 values, one row
    enc = quantize_fp4_rows(vals, 32, 32)
    np.testing.assert_array_equal(formats.decode_fp4_rows(enc, 32)[0], np.asarray(vals[0], dtype=np.float64))
    # every e2m1 value is an e4m3 value (torch's decoding)
    e4 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert set(lut.tolist()) <= set(e4[~np.isnan(e4)].tolist())


def test_e2m1_ties_round_to_even_codes():
    from mla_inputs import quantize_fp4_rows
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]        # the neighbour with mantissa bit 0
    # one 32-value row, both 16-value groups with amax 6 (scale 1)
    x = torch.tensor([mids + [-v for v in mids] + [6.0, 0.0] + [6.0] + [0.0] * 15], dtype=torch.float32)
    got = formats.decode_fp4_rows(quantize_fp4_rows(x, 32, 32), 32)[0]
    np.testing.assert_array_equal(got, expect + [-v for v in expect] + [6.0, 0.0] + [6.0] + [0.0] * 15)


def test_fp4_row_nibbles_and_scale_groups():
    # element i: nibble i % 2 of byte i // 2, scale byte i // 16
    d = 576
    g = torch.Generator().manual_seed(7)
    packed = torch.randint(0, 256, (d // 2,), generator=g, dtype=torch.int32).numpy().astype(np.uint8)
    scales = (np.arange(d // 16) * 2 + 100).astype(np.uint8)
    row = np.full(336, 0xFF, dtype=np.uint8)           # padding poisoned: must be ignored
    row[:d // 2] = packed
    row[d // 2:d // 2 + d // 16] = scales
    got = formats.decode_fp4_rows(row[None, :], d)[0]
    sv = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for i in range(d):
        code = (int(packed[i // 2]) >> (4 * (i % 2))) & 0xF
        assert got[i] == formats.E2M1_LUT[code] * sv[i // 16], i
    # the other nibble order (high nibble first) must not agree
    wrong = formats.E2M1_LUT[packed >> 4]
    assert not np.array_equal(got[0::2] / np.repeat(sv, 8), wrong)


def test_fp4_row_bytes_match_page_figure():
    figs = _figures()
    assert footprint.fp4_row_bytes(512) == figs["fp4_row_bytes_512_dims"]["value"] == 288
    assert formats.fp4_row_payload_bytes(512) == 288
    assert footprint.fp4_row_bytes(576) == 324


def test_fp8_row_bytes_match_page_layout():
    figs = _figures()
    assert footprint.fp8_row_bytes(512) == figs["fp8_row_bytes_512_dims"]["value"] == 528
    assert formats.fp8_row_payload_bytes(512) == 528
    # the 576-dimension row of the same format
    assert footprint.fp8_row_bytes(576) == 594


def test_footprints_against_printed_figures():
    figs = _figures()
    assert footprint.mla_row_elements() == figs["mla_row_elements"]["value"]
    per_tok = footprint.mla_bytes_per_token(61)
    assert per_tok == figs["mla_bytes_per_token_61_layers_bf16"]["value"]
    assert round(per_tok / 1024, 1) == figs["mla_kib_per_token_61_layers_bf16"]["value"]
    seq = footprint.mla_bytes_per_sequence(131072)
    assert seq == 9_210_691_584
    assert round(seq / 1e9, 2) == figs["mla_gb_128k_context_bf16"]["value"]
    mha = footprint.mha_bytes_per_sequence(131072)
    assert mha == 523_986_010_112
    assert math.floor(mha / 1e9 * 100) / 100 == figs["mha_gb_128k_context_bf16"]["value"]
    assert round(100 * footprint.compression_vs_mha(), 2) == figs["compression_vs_mha_percent"]["value"]


def test_page_block_size_figure():
    from mla_inputs import SPECS
    figs = _figures()
    assert all(s.page == figs["page_block_size"]["value"] for s in SPECS.values())
