"""Pins of the FP8 E4M3 conversions the FP8 tests and the oracle's input decode
use (``synthgen.f32_to_e4m3_bits``, ``e4m3_bits_to_f64``, ``normal_e4m3``),
against torch's float8_e4m3fn dtype (the OCP E4M3 format)."""

import numpy as np
import torch

from synthgen import E4M3_MAX, e4m3_bits_to_f64, f32_to_e4m3_bits, normal_e4m3


def test_rounding_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-4, 1e-2, 1, 30, 200)])
    x = x[np.abs(x) <= E4M3_MAX]
    # exact ties between neighbours (round half to even), the subnormal range and the extremes
    ties = np.array([1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10, 5 * 2 ** -10, 448.0, -448.0, 0.0, -0.0, 2 ** -6],
                    dtype=np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e4m3_bits(x), ref)


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_bits_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert e4m3_bits_to_f64(np.array([0x7E], np.uint8))[0] == E4M3_MAX


def test_quantised_draw_is_within_half_a_step():
    bits, ds = normal_e4m3(5, 1, (2, 3, 40, 16))
    from synthgen import normal_f32

    x = normal_f32(5, 1, (2, 3, 40, 16)).astype(np.float64)
    val = e4m3_bits_to_f64(bits) * ds.astype(np.float64)[..., None, None]
    # the largest magnitude maps to 448 exactly; every value within 2^-4 relative
    # (or half the subnormal step 2^-10 of the descaled unit)
    assert np.allclose(np.abs(val).reshape(6, -1).max(axis=1), np.abs(x).reshape(6, -1).max(axis=1), rtol=1e-6)
    tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * ds.astype(np.float64)[..., None, None])
    assert np.all(np.abs(val - x) <= tol * (1 + 1e-9))
