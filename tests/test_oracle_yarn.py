"""Pins for the oracle's YaRN / RoPE ("MoE-Xtend" README, ROPE + SCALING).

Each test checks the oracle against something other than its own formula:
the textbook base schedule, the NTK ratio that defines the cutpoints, the
complex-number form of a rotation, norms, relative-position invariance, and
logarithms at points where they are known exactly.
"""
import math

import numpy as np
import pytest

from oracle import yarn

CASES = [
    # d, base, factor, L, alpha, beta
    (64, 150000.0, 32.0, 4096, 1.0, 32.0),
    (96, 150000.0, 32.0, 4096, 1.0, 32.0),
    (64, 10000.0, 8.0, 2048, 1.0, 32.0),
    (128, 500000.0, 4.0, 8192, 2.0, 16.0),
]


@pytest.mark.parametrize("d,base", [(64, 10000.0), (96, 150000.0), (8, 10000.0)])
def test_s1_is_plain_rope(d, base):
    # s = 1: interpolation == extrapolation, so every pair keeps theta_i.
    got = yarn.yarn_inv_freq(d, base, 1.0, 4096, 1.0, 32.0)
    i = np.arange(d // 2)
    textbook = np.array([base ** (-(2.0 * k) / d) for k in i])
    np.testing.assert_allclose(got, textbook, rtol=2e-16 * 8, atol=0)
    assert yarn.yarn_concentration(1.0) == 1.0


@pytest.mark.parametrize("d,base,s,L,a,b", CASES)
def test_cutpoints_are_where_the_ntk_ratio_hits_alpha_beta(d, base, s, L, a, b):
    # r(i) = L*theta_i/(2 pi) for real i; the cutpoints are r = beta, r = alpha.
    i_beta, i_alpha = yarn.yarn_cutpoints(d, base, L, a, b)
    r = lambda x: L * math.pow(base, -2.0 * x / d) / (2 * math.pi)
    assert i_beta < i_alpha
    assert r(i_beta) == pytest.approx(b, rel=1e-12)
    assert r(i_alpha) == pytest.approx(a, rel=1e-12)


@pytest.mark.parametrize("d,base,s,L,a,b", CASES)
def test_three_regimes(d, base, s, L, a, b):
    inv = yarn.yarn_inv_freq(d, base, s, L, a, b)
    theta = np.array([base ** (-(2.0 * k) / d) for k in range(d // 2)])
    r = L * theta / (2 * math.pi)
    fast = r >= b          # many turns over L: unchanged
    slow = r <= a          # less than alpha turns: stretched by s
    mid = ~fast & ~slow
    np.testing.assert_allclose(inv[fast], theta[fast], rtol=1e-15)
    np.testing.assert_allclose(inv[slow], theta[slow] / s, rtol=1e-15)
    # Between the cutpoints: strictly between the two, with an interpolation
    # weight that is linear in i and reaches 1 at i_beta, 0 at i_alpha.
    w = (inv - theta / s) / (theta - theta / s)
    assert np.all((w[mid] > 0) & (w[mid] < 1))
    idx = np.nonzero(mid)[0]
    if len(idx) >= 2:
        slope, icpt = np.polyfit(idx, w[idx], 1)
        np.testing.assert_allclose(w[idx], slope * idx + icpt, atol=1e-12)
        i_beta, i_alpha = yarn.yarn_cutpoints(d, base, L, a, b)
        assert slope * i_beta + icpt == pytest.approx(1.0, abs=1e-9)
        assert slope * i_alpha + icpt == pytest.approx(0.0, abs=1e-9)
    # Monotone: the rate never increases with the pair index.
    assert np.all(np.diff(inv) < 0)


def test_region_sizes_gpt_oss_yarn():
    # d=64, base 1.5e5, L=4096, alpha=1, beta=32: pairs 0..8 have r>32,
    # 18..31 have r<1; the blend covers 9..17 (cutpoints 8.09 and 17.40).
    d, base, L = 64, 150000.0, 4096
    theta = np.array([base ** (-(2.0 * k) / d) for k in range(d // 2)])
    r = L * theta / (2 * math.pi)
    assert (r >= 32).sum() == 9 and (r <= 1).sum() == 14


def test_concentration_natural_log():
    # c = 0.1*ln(s) + 1: at s = e**k the log is exactly k.
    for k in range(0, 6):
        assert yarn.yarn_concentration(math.e ** k) == pytest.approx(1 + 0.1 * k, abs=1e-14)
    # additivity of the log part
    c = yarn.yarn_concentration
    assert (c(4.0) - 1) + (c(8.0) - 1) == pytest.approx(c(32.0) - 1, abs=1e-15)
    assert c(32.0) > c(8.0) > 1.0


def _rand(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("d", [8, 64, 96])
def test_rotation_is_complex_multiplication(d):
    inv = yarn.yarn_inv_freq(d, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn.yarn_concentration(32.0)
    x = _rand((2, 5, 3, d))
    pos = np.array([0, 1, 4097, 65536, 131135])
    y = yarn.rope_rotate(x, pos, inv, c)
    h = d // 2
    z = (x[..., :h] + 1j * x[..., h:]) * c * np.exp(1j * pos[:, None, None] * inv)
    np.testing.assert_allclose(y[..., :h], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., h:], z.imag, atol=1e-12)


def test_position_zero_scales_by_c():
    inv = yarn.yarn_inv_freq(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn.yarn_concentration(32.0)
    x = _rand((1, 1, 4, 64))
    y = yarn.rope_rotate(x, np.array([0]), inv, c)
    assert np.array_equal(y, x * c)


def test_pair_norm_scales_by_c():
    inv = yarn.yarn_inv_freq(96, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn.yarn_concentration(32.0)
    x = _rand((1, 7, 2, 96), 3)
    pos = np.arange(7) * 20011
    y = yarn.rope_rotate(x, pos, inv, c)
    nx = np.hypot(x[..., :48], x[..., 48:])
    ny = np.hypot(y[..., :48], y[..., 48:])
    np.testing.assert_allclose(ny, c * nx, rtol=1e-14)


@pytest.mark.parametrize("delta", [1, 4096, 65536, 131072])
def test_relative_position_invariance(delta):
    # <R(q, p+D), R(k, p'+D)> == <R(q, p), R(k, p')>: scores depend on p-p'.
    inv = yarn.yarn_inv_freq(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn.yarn_concentration(32.0)
    q = _rand((1, 1, 1, 64), 5)
    k = _rand((1, 1, 1, 64), 6)
    p, pk = 17, 3
    a = np.sum(yarn.rope_rotate(q, np.array([p]), inv, c) *
               yarn.rope_rotate(k, np.array([pk]), inv, c))
    b = np.sum(yarn.rope_rotate(q, np.array([p + delta]), inv, c) *
               yarn.rope_rotate(k, np.array([pk + delta]), inv, c))
    assert b == pytest.approx(a, abs=1e-9)


def test_composition_of_rotations():
    # Rotating by p1 then p2 is one rotation by p1+p2 with c applied twice.
    inv = yarn.yarn_inv_freq(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn.yarn_concentration(32.0)
    x = _rand((1, 1, 3, 64), 9)
    y = yarn.rope_rotate(yarn.rope_rotate(x, np.array([1000]), inv, c),
                         np.array([70000]), inv, c)
    z = yarn.rope_rotate(x, np.array([71000]), inv, c) * c
    np.testing.assert_allclose(y, z, atol=1e-10)


def test_global_position_offset():
    # rope_apply at offset o equals rotating at positions o + t.
    inv = yarn.yarn_inv_freq(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn.yarn_concentration(32.0)
    x = _rand((2, 6, 3, 64), 11)
    full = yarn.rope_apply(np.concatenate([np.zeros((2, 100, 3, 64)), x], 1), 0, inv, c)
    np.testing.assert_array_equal(yarn.rope_apply(x, 100, inv, c), full[:, 100:])


def test_bad_parameters_rejected():
    with pytest.raises(ValueError):
        yarn.yarn_inv_freq(63, 1e4, 1.0, 4096, 1.0, 32.0)
    with pytest.raises(ValueError):
        yarn.yarn_inv_freq(64, 1e4, 0.5, 4096, 1.0, 32.0)
    with pytest.raises(ValueError):
        yarn.yarn_inv_freq(64, 1e4, 2.0, 4096, 32.0, 1.0)
