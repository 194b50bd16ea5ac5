"""Number formats of the latent cache, decoded exactly into float64.

Test infrastructure only (see ``oracle/__init__``).

bf16
    The upper 16 bits of an IEEE-754 binary32.  Widening to float64 is exact.

e4m3 ("fn" flavour)
    "DeepSeek R1 Architecture & Deployment Guide", section 4, gives the E4M3
    max normal as 448.0, which fixes the finite-only OCP variant: 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
    subnormals m/8 * 2^-6; the all-ones exponent is still finite except for
    mantissa 111, which is NaN.  (The "fnuz" variant would top out at 240.)

e8m0
    The "DeepSeek-R1" record, engine kernel constraint (2), names float8_e8m0
    scales, one per 32 e4m3 values.  Reading: the OCP MX scale type, a bare
    biased exponent, value 2^(e - 127); 0xFF is NaN; there is no zero.

FP8 cache row (same constraint (2))
    A token's row is D e4m3 codes over *every* dimension (the 64 RoPE
    dimensions are quantised too, there is no bf16 part), followed by D/32
    e8m0 scale bytes; scale g multiplies codes 32g .. 32g+31.  Rows may be
    padded to a larger stride; padding bytes are never read.

e2m1 (FP4)
    The same constraint names an fp4 variant of the row at 288 bytes per
    token for 512 dimensions, with per-token inlined scales, and nothing
    more.  Reading: OCP FP4 E2M1, 1 sign bit, 2 exponent bits with bias 1,
    1 mantissa bit, no inf or NaN: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.

FP4 cache row (reading of the same constraint)
    288 = 256 + 32 bytes at 512 dimensions: D/2 bytes of codes, two per
    byte (element 2i in the low nibble of byte i, 2i + 1 in the high one),
    then D/16 e8m0 scale bytes, scale g multiplying elements 16g .. 16g+15.
    At the 576 dimensions of this decode that is 288 + 36 = 324 bytes.
"""

from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# scalar definitions
# --------------------------------------------------------------------------

def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, from the bit-field definition."""
    code = int(code) & 0xFF
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        # subnormal: 0.mmm * 2^(1 - bias)
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


def e8m0_value(byte: int) -> float:
    """Value of one e8m0 scale byte: 2^(byte - 127), NaN for 0xFF."""
    byte = int(byte) & 0xFF
    if byte == 0xFF:
        return math.nan
    return 2.0 ** (byte - 127)


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code, from the bit-field definition."""
    code = int(code) & 0xF
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp_field = (code >> 1) & 0x3
    mant = code & 0x1
    if exp_field == 0:
        return sign * (mant / 2.0)               # subnormal: 0.m * 2^(1 - bias)
    return sign * (1.0 + mant / 2.0) * 2.0 ** (exp_field - 1)


# lookup tables built from the scalar definitions above.
E2M1_LUT = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3FN_LUT = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E8M0_LUT = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


# --------------------------------------------------------------------------
# array decoders
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return as_f32.astype(np.float64)


def decode_bf16_rows(rows: np.ndarray, d: int) -> np.ndarray:
    """bf16 cache rows [..., d] (uint16 bit patterns) -> float64 [..., d]."""
    rows = np.asarray(rows, dtype=np.uint16)
    if rows.shape[-1] != d:
        raise ValueError(f"bf16 row has {rows.shape[-1]} elements, expected {d}")
    return bf16_bits_to_f64(rows)


def decode_fp8_rows(rows: np.ndarray, d: int) -> np.ndarray:
    """FP8 cache rows [..., stride] (uint8) -> float64 [..., d].

    Bytes 0..d-1 are e4m3fn codes, bytes d .. d + d/32 - 1 are e8m0 scales;
    anything beyond is padding and is ignored.
    """
    rows = np.asarray(rows, dtype=np.uint8)
    if d % 32:
        raise ValueError("FP8 rows need d to be a multiple of 32 (one scale per 32 codes)")
    n_scales = d // 32
    if rows.shape[-1] < d + n_scales:
        raise ValueError("FP8 row stride smaller than its payload")
    codes = E4M3FN_LUT[rows[..., :d]]
    scales = E8M0_LUT[rows[..., d:d + n_scales]]
    # scale g covers codes 32g .. 32g+31
    return codes * np.repeat(scales, 32, axis=-1)


def decode_fp4_rows(rows: np.ndarray, d: int) -> np.ndarray:
    """FP4 cache rows [..., stride] (uint8) -> float64 [..., d].

    Bytes 0 .. d/2 - 1 hold the codes (low nibble first), bytes
    d/2 .. d/2 + d/16 - 1 the e8m0 scales; anything beyond is padding.
    """
    rows = np.asarray(rows, dtype=np.uint8)
    if d % 32:
        raise ValueError("FP4 rows need d to be a multiple of 32")
    n_code, n_scale = d // 2, d // 16
    if rows.shape[-1] < n_code + n_scale:
        raise ValueError("FP4 row stride smaller than its payload")
    packed = rows[..., :n_code]
    codes = np.empty(packed.shape[:-1] + (d,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    scales = E8M0_LUT[rows[..., n_code:n_code + n_scale]]
    # scale g covers elements 16g .. 16g+15
    return E2M1_LUT[codes] * np.repeat(scales, 16, axis=-1)


def fp4_row_payload_bytes(d: int) -> int:
    """Bytes of one FP4 row without padding: d/2 code bytes + d/16 scales."""
    return d // 2 + d // 16


def fp8_row_payload_bytes(d: int) -> int:
    """Bytes of one FP8 row without padding: d codes + d/32 scales."""
    return d + d // 32
