"""Pins for the oracle's direct fp64 -> bf16 / fp32 rounding.

bf16 from fp32-exact inputs must equal torch's own float32 -> bfloat16 cast
(a library routine, ties to even); fp64 inputs just past a bf16 tie must
round away from the tie (no fp32 intermediate rounding).
"""
import numpy as np
import torch

from oracle.rounding import bf16_bits_of, round_bf16, round_f32


def _torch_bf16(x32):
    t = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-45], np.float32),
    ])
    # exact ties: bf16 value plus half an ulp
    base = (rng.standard_normal(2000).astype(np.float32).view(np.uint32)
            & np.uint32(0xFFFF0000))
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, _torch_bf16(x))


def test_bf16_direct_rounding_not_double():
    # 1 + 2**-8 is the midpoint of 1 and 1 + 2**-7; a hair above it must go up.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    # the same value through fp32 first would land on the tie and go to 1.0
    assert round_bf16(np.array([float(np.float32(x))]))[0] == 1.0
    assert round_bf16(np.array([-x]))[0] == -(1.0 + 2.0 ** -7)


def test_bf16_overflow_and_specials():
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127       # tie above the largest bf16
    got = round_bf16(np.array([big, -big, np.inf, -np.inf, np.nan]))
    assert got[0] == np.inf and got[1] == -np.inf
    assert got[2] == np.inf and got[3] == -np.inf and np.isnan(got[4])


def test_f32_rounding_matches_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000)
    np.testing.assert_array_equal(round_f32(x), x.astype(np.float32).astype(np.float64))


def test_bits_roundtrip():
    v = round_bf16(np.random.default_rng(2).standard_normal(100))
    bits = bf16_bits_of(v)
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(back, v)
