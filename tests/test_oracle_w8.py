"""Pins of the oracle's W8G32_F16S path (signed 8-bit weights with one fp16
scale per 32 k: the encoding the pages name for the DFlash2 drafter's
matrices), against numpy's float16, a hand-worked group, exhaustive
nearest-code checks and numpy's float64 product."""
import numpy as np
import pytest

import oracle
import workloads


def test_f16_values_match_numpy():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(b)) for b in bits])
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin]) and np.all(np.isnan(got[np.isnan(want)]))


def test_f16_rounding_matches_numpy():
    """The quantizer's float -> fp16 step (seen through the scales it picks):
    amax / 127 rounded as numpy rounds float32 to float16, over 2000 groups
    spanning fp16's normal and subnormal ranges."""
    rng = np.random.default_rng(1)
    amax = (rng.random(2000) * np.exp2(rng.integers(-30, 16, 2000))).astype(np.float32)
    W = np.zeros((2000, 32), np.float32)
    W[:, 0] = amax
    _, s = oracle.w8_quantize(W)
    want = (amax / np.float32(127.0)).astype(np.float16).view(np.uint16)
    assert np.array_equal(s[:, 0], want)


def test_worked_group():
    """amax 2.54: scale = fp16(0.02) = 0x251F (0.0200042724609375); codes
    rint(v / scale): 2.54 -> 127, -1.0 -> -50 (49.989...), 0.01 -> 0 (0.4999...)."""
    W = np.zeros((1, 32), np.float32)
    W[0, :3] = [2.54, -1.0, 0.01]
    c, s = oracle.w8_quantize(W)
    assert s[0, 0] == np.float16(np.float32(2.54) / np.float32(127.0)).view(np.uint16)
    S = float(np.float16(np.float32(2.54) / np.float32(127.0)))
    assert list(c[0, :3]) == [int(np.rint(2.54 / S)), int(np.rint(-1.0 / S)), int(np.rint(0.01 / S))]
    assert c[0, 0] == 127


@pytest.mark.parametrize("seed", range(3))
def test_nearest_code_and_round_trip(seed):
    rng = np.random.default_rng(seed)
    n, k = 8, 256
    W = (rng.standard_normal((n, k)) * np.exp2(rng.integers(-12, 4, (n, 1)))).astype(np.float32)
    c, s = oracle.w8_quantize(W)
    S = np.repeat(s.view(np.float16).astype(np.float64), 32, axis=1)
    t = W.astype(np.float64) / S
    # the nearest integer, or the clamp at +-127 (a scale that fp16 rounds down,
    # by up to 2^-11 relative, or far more for subnormal scales, leaves |t| above 127)
    clamped = np.abs(c) == 127
    assert np.all(np.abs(t - c)[~clamped] <= 0.5 + 1e-12)
    assert np.all(np.abs(t)[clamped] >= 126.5) and np.all(np.sign(t)[clamped] == np.sign(c)[clamped])
    assert np.array_equal(oracle.w8_dequant(c, s), c.astype(np.float64) * S)
    # a second pass over the dequantized weights gives back the same codes and scales
    c2, s2 = oracle.w8_quantize((c * S).astype(np.float32))
    assert np.array_equal(s2, s) and np.array_equal(c2, c)


def test_zero_group_and_clamp():
    W = np.zeros((2, 64), np.float32)
    W[1, 32:] = 1.0
    W[1, 40] = -1.0
    c, s = oracle.w8_quantize(W)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and not c[0].any() and not c[1, :32].any()
    assert c[1, 32] == 127 and c[1, 40] == -127


def test_gemv_matches_numpy_on_dequantized_weights():
    rng = np.random.default_rng(12)
    n, k, rows = 40, 224, 5
    c, s = oracle.w8_quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    xb = workloads.bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y, a, _ = oracle.w8_gemv(c, s, xb)
    D = oracle.w8_dequant(c, s)
    assert np.allclose(y, xv @ D.T, rtol=1e-12, atol=1e-15)
    assert np.allclose(a, np.abs(xv) @ np.abs(D).T, rtol=1e-12)
