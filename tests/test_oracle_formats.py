"""Pins for the oracle's format decoders (CPU only)."""

import numpy as np
import torch

from oracle import formats
import synth


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(ours[fin], lib[fin])
    # sign of zero too
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))


def test_e4m3_format_facts():
    # OCP E4M3FN: max finite 448 (S.1111.110), min normal 2^-6, min subnormal 2^-9,
    # S.1111.111 is NaN, there is no infinity.
    v = formats.e4m3_to_f64(np.array([0x7E, 0xFE, 0x08, 0x01, 0x07, 0x7F, 0xFF, 0x80, 0x38], np.uint8))
    assert v[0] == 448.0 and v[1] == -448.0
    assert v[2] == 2.0 ** -6 and v[3] == 2.0 ** -9 and v[4] == 7 * 2.0 ** -9
    assert np.isnan(v[5]) and np.isnan(v[6])
    assert v[7] == 0.0 and np.signbit(v[7])
    assert v[8] == 1.0
    assert not np.any(np.isinf(formats.e4m3_to_f64(np.arange(256, dtype=np.uint8))))


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_bits_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_generator_bf16_rounding_is_rne_like_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]  # exact ties
    ours = synth.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_generator_e4m3_scale_and_saturation():
    x = np.random.default_rng(1).standard_normal((50, 576)).astype(np.float32)
    x[3] = 0.0
    codes, scale = synth.f32_to_e4m3(x)
    assert scale[3] == 1.0
    dec = formats.fp8_cache_to_f64(codes, scale)
    amax = np.abs(x).max(-1)
    # the largest element of each row maps to +-448 * scale = +-amax (up to fp32 rounding)
    assert np.allclose(np.abs(dec).max(-1), amax, rtol=1e-6)
    # quantisation error bounded by half an E4M3 step at the value (3 mantissa bits)
    err = np.abs(dec - x)
    assert np.all(err <= np.abs(x) * 2.0 ** -4 + scale[:, None] * 2.0 ** -10 + 1e-12)


def test_slab_seeding_independent_of_threads():
    a = synth.bf16_normal(7, 1, (10, 3, 4), chunk=3)
    b = synth.bf16_normal(7, 1, (10, 3, 4), chunk=3)
    assert np.array_equal(a, b)
    g = synth.rng(7, 1, 1)
    first = g.standard_normal((3, 3, 4), dtype=np.float32)
    assert np.array_equal(a[3:6], synth.f32_to_bf16_bits(first))
