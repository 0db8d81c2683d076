"""Decoding of the stored number formats into float64 (oracle; test use only).

The inputs the attention path consumes are bit patterns: bf16 words and OCP
FP8 E4M3 bytes with a per-token fp32 scale. The oracle decodes those exact
bits into float64 from the formats' own definitions, so it sees the same
values as the GPU path, not the float32 values they were rounded from.

Sources: the FP8 cache entry is the "576 one-byte numbers" per token of
*Long Context* 1.2; the per-token fp32 scale follows the index-key format of
the vLLM GLM-5.3 post, footnote 3 (128 FP8 values plus a 4-byte scale).
The E4M3 definition is the OCP 8-bit floating point specification (E4M3FN:
bias 7, no infinities, S.1111.111 is NaN).

Pins: ``tests/test_oracle_formats.py`` checks all 256 E4M3 codes against
torch's ``float8_e4m3fn`` dtype and against printed format facts (max 448,
min normal 2^-6, min subnormal 2^-9); bf16 against torch's ``bfloat16``.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """bf16 word -> float64. A bf16 value is the upper 16 bits of an IEEE
    binary32 value, so widening is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes):
    """OCP E4M3FN byte -> float64, from the format definition.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    Exponent 0 encodes subnormals m/8 * 2^(1-7); exponent/mantissa all-ones
    (0x7F, 0xFF) is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * np.exp2(1.0 - 7.0)
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def fp8_cache_to_f64(codes, scale):
    """Dequantised cache entry: k_t = e4m3(code) * scale_t, one fp32 scale per
    token (broadcast over the last axis)."""
    return e4m3_to_f64(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
