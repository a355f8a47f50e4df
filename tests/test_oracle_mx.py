"""Pins of the oracle's MXFP4 path (E2M1 elements with one E8M0 power-of-two
scale per 32 k: the format the pages name through the kern build's
gpu_mxfp4 kernels), against the format's value sets, hand-worked blocks,
exhaustive nearest-value search and numpy's float64 product."""
import math

import numpy as np
import pytest

import oracle
import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e8m0_values():
    for b in range(255):
        assert oracle.e8m0_value(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(oracle.e8m0_value(255))


def _block(vals):
    W = np.zeros((1, 32), np.float32)
    W[0, :len(vals)] = vals
    return W


def test_worked_block():
    """amax 3 = 1.5 * 2^1: shared exponent 1 - 2 = -1 (byte 126); V / 0.5 =
    6, 2, -1.5, 0 -> codes 0x7, 0x4, 0xB, 0x0 (low nibble first)."""
    c, s = oracle.mx_quantize(_block([3.0, 1.0, -0.75, 0.0]))
    assert s[0, 0] == 126
    assert list(c[0, :2]) == [0x7 | (0x4 << 4), 0xB | (0x0 << 4)]
    assert list(oracle.mx_dequant(c, s)[0, :4]) == [3.0, 1.0, -0.75, 0.0]


def test_saturation_and_zero_block():
    """amax 7.9 (exponent 2): X = 0 and 7.9 saturates to code 7 (6); an
    all-zero block gets byte 127 and zero codes."""
    c, s = oracle.mx_quantize(_block([7.9, -7.9, 5.0]))
    assert s[0, 0] == 127 and list(c[0, :2]) == [0x7 | (0xF << 4), 0x6]   # 5: a tie of 4 and 6, to the even mantissa (4)
    z = np.zeros((2, 64), np.float32)
    c, s = oracle.mx_quantize(z)
    assert (s == 127).all() and not c.any()


@pytest.mark.parametrize("seed", range(4))
def test_round_trip_of_grid_blocks(seed):
    """Blocks of grid values times 2^X holding a +-4 or +-6 (so amax fixes the
    same X) come back exactly."""
    rng = np.random.default_rng(seed)
    n, k = 6, 128
    X = rng.integers(-20, 20, (n, k // 32))
    vals = rng.choice(GRID, (n, k)) * rng.choice([-1.0, 1.0], (n, k))
    vals[:, ::32] = rng.choice([4.0, -6.0, 6.0, -4.0], (n, k // 32))
    W = (vals * np.exp2(np.repeat(X, 32, axis=1))).astype(np.float32)
    c, s = oracle.mx_quantize(W)
    assert np.array_equal(s.astype(int) - 127, X)
    assert np.array_equal(oracle.mx_dequant(c, s), W.astype(np.float64))


def test_every_element_is_the_nearest_grid_value():
    """Exhaustive check against the grid: |V/2^X| is at most 6 away from a
    saturated code, and otherwise no grid point is nearer than the chosen one."""
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((8, 256)) * np.exp2(rng.integers(-10, 10, (8, 1)))).astype(np.float32)
    c, s = oracle.mx_quantize(W)
    D = oracle.mx_dequant(c, s)
    X = np.repeat(s.astype(int) - 127, 32, axis=1)
    t = np.abs(W.astype(np.float64)) / np.exp2(X)
    got = np.abs(D) / np.exp2(X)
    best = np.min(np.abs(t[..., None] - GRID[None, None, :]), axis=-1)
    assert np.all(np.abs(t - got) <= best + 0.0)
    assert np.all(t.max(axis=1) >= 4.0 - 1e-12)                    # the shared exponent puts amax in [4, 8)
    assert np.array_equal(np.signbit(D) | (D == 0), np.signbit(W) | (D == 0))


def test_gemv_matches_numpy_on_dequantized_weights():
    rng = np.random.default_rng(10)
    n, k, rows = 40, 224, 5
    c, s = oracle.mx_quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    xb = workloads.bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y, a, _ = oracle.mx_gemv(c, s, xb)
    D = oracle.mx_dequant(c, s)
    assert np.allclose(y, xv @ D.T, rtol=1e-12, atol=1e-15)
    assert np.allclose(a, np.abs(xv) @ np.abs(D).T, rtol=1e-12)
