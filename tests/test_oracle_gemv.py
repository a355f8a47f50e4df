"""Pins of the oracle projection and gate/up pair: exact rational brute force on
tiny shapes, numpy fp64 matmul, one-hot and zero special cases, the hand-worked
row, row and selection independence, and scipy's logistic function for SiLU."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import workloads
from test_oracle_quantizer import load_kv


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _gamma(k):
    u = 2.0 ** -53
    return k * u / (1 - k * u)


def test_worked_row_gemv(oracle_lib):
    g = load_kv("worked_row.txt")
    W = np.array([float(v) for v in g["W"]], np.float32)[None, :]
    codes, scales, sg = oracle_lib.quantize(W)
    x = workloads.bf16_bits(np.array([[float(v) for v in g["x"]]], np.float32))
    y, a, yb = oracle_lib.gemv(codes, scales, sg, x)
    assert y[0, 0] == float(g["y"][0])
    assert a[0, 0] == float(g["absdot"][0])
    assert yb[0, 0] == int(g["y_bf16"][0], 16)


def test_gemv_exact_rational_brute_force(oracle_lib):
    rng = np.random.default_rng(21)
    for n, k, rows in [(3, 16, 1), (5, 48, 3), (8, 64, 8)]:
        c = workloads.case(n, k, rows, seed=int(rng.integers(1 << 30)))
        codes, scales, sg = oracle_lib.quantize(c["W"])
        D = oracle_lib.dequant(codes, scales, sg)
        y, a, yb = oracle_lib.gemv(codes, scales, sg, c["x"])
        xf = _bf16_to_f64(c["x"])
        for r in range(rows):
            for j in range(n):
                exact = sum(Fraction(float(D[j, t])) * Fraction(float(xf[r, t])) for t in range(k))
                absd = sum(abs(Fraction(float(D[j, t])) * Fraction(float(xf[r, t]))) for t in range(k))
                bound = _gamma(k) * float(absd)
                assert abs(Fraction(y[r, j]) - exact) <= Fraction(bound)
                assert abs(Fraction(a[r, j]) - absd) <= Fraction(bound)
                # bf16 of the exact value, by search over neighbouring bf16 values
                yf = float(exact)
                cand = np.array([workloads.bf16_bits(np.array([yf], np.float32))[0]], np.uint16)
                nb = [int(cand[0]) + d for d in (-2, -1, 0, 1, 2)]
                nb = [b for b in nb if 0 <= b < 65536]
                dist = [(abs(Fraction(float(_bf16_to_f64(np.array([b], np.uint16))[0])) - exact), b) for b in nb]
                dmin = min(d for d, _ in dist)
                assert any(b == int(yb[r, j]) and d == dmin for d, b in dist)


def test_gemv_vs_numpy_matmul(oracle_lib):
    c = workloads.case(200, 784, 5, seed=9)
    codes, scales, sg = oracle_lib.quantize(c["W"])
    D = oracle_lib.dequant(codes, scales, sg).astype(np.float64)
    xf = _bf16_to_f64(c["x"])
    ref = xf @ D.T
    refabs = np.abs(xf) @ np.abs(D).T
    y, a, _ = oracle_lib.gemv(codes, scales, sg, c["x"])
    bound = 2 * _gamma(784) * refabs
    assert np.all(np.abs(y - ref) <= bound)
    assert np.all(np.abs(a - refabs) <= bound)


def test_gemv_one_hot_zero_and_selection(oracle_lib):
    c = workloads.case(64, 256, 1, seed=10)
    codes, scales, sg = oracle_lib.quantize(c["W"])
    D = oracle_lib.dequant(codes, scales, sg)
    for col in (0, 17, 255):
        x = np.zeros((1, 256), np.float32)
        x[0, col] = 1.0
        y, _, _ = oracle_lib.gemv(codes, scales, sg, workloads.bf16_bits(x))
        assert np.array_equal(y[0], D[:, col].astype(np.float64))
    y, a, yb = oracle_lib.gemv(codes, scales, sg, np.zeros((2, 256), np.uint16))
    assert not y.any() and not a.any() and not yb.any()
    assert not np.signbit(y).any()
    zc = np.zeros_like(codes)
    y, _, _ = oracle_lib.gemv(zc, scales, sg, c["x"])
    assert not y.any()
    # a row's result does not depend on the other rows; selection = columns
    c8 = workloads.case(64, 256, 8, seed=12)
    y8, a8, b8 = oracle_lib.gemv(codes, scales, sg, c8["x"])
    y3, _, _ = oracle_lib.gemv(codes, scales, sg, c8["x"][3:4])
    assert np.array_equal(y8[3], y3[0])
    sel = np.array([63, 0, 5, 5, 40])
    ys, as_, bs = oracle_lib.gemv(codes, scales, sg, c8["x"], sel=sel)
    assert np.array_equal(ys, y8[:, sel]) and np.array_equal(bs, b8[:, sel])


def test_dual_silu_vs_scipy(oracle_lib):
    c = workloads.case(48, 320, 4, seed=13, dual=True)
    gq = oracle_lib.quantize(c["W"])
    uq = oracle_lib.quantize(c["W_up"])
    out = oracle_lib.gemv_dual_silu(gq, uq, c["x"])
    g, _, _ = oracle_lib.gemv(*gq, c["x"])
    u, _, _ = oracle_lib.gemv(*uq, c["x"])
    assert np.array_equal(out["g"], g) and np.array_equal(out["u"], u)
    ref = g * expit(g) * u
    assert np.allclose(out["o"], ref, rtol=1e-14, atol=1e-300)


def test_dual_silu_extremes(oracle_lib):
    # a weight row that yields g = 0 and one with large |g|: check the composition
    W = np.zeros((2, 16), np.float32)
    W[1, 0] = 100.0
    U = np.ones((2, 16), np.float32)
    gq = oracle_lib.quantize(W)
    uq = oracle_lib.quantize(U)
    x = workloads.bf16_bits(np.array([[1.0] * 16, [-1.0] + [0.0] * 15], np.float32))
    out = oracle_lib.gemv_dual_silu(gq, uq, x)
    assert out["o"][0, 0] == 0.0
    assert out["o"][0, 1] == pytest.approx(100.0 * 16.0, rel=1e-12)   # silu(100) = 100
    assert abs(out["o"][1, 1]) < 1e-40                                  # silu(-100) ~ 0


# ---- the plain fp32 definition (dequantize, sequential fp32 dot) ------------------

def _gamma32(k):
    u = 2.0 ** -24
    return k * u / (1 - k * u)


def test_f32seq_within_recursive_summation_bound(oracle_lib):
    """fp32 sequential sum of k exact products: within gamma_k * sum|D*x| of
    the exact rational value; its bf16 copy is the RNE of its fp32 result."""
    rng = np.random.default_rng(22)
    for n, k, rows in [(3, 16, 1), (5, 48, 3), (8, 64, 8)]:
        c = workloads.case(n, k, rows, seed=int(rng.integers(1 << 30)))
        codes, scales, sg = oracle_lib.quantize(c["W"])
        D = oracle_lib.dequant(codes, scales, sg)
        y32, y16 = oracle_lib.gemv_f32seq(codes, scales, sg, c["x"])
        xf = _bf16_to_f64(c["x"])
        for r in range(rows):
            for j in range(n):
                terms = [Fraction(float(D[j, t])) * Fraction(float(xf[r, t])) for t in range(k)]
                exact, absd = sum(terms), sum(abs(t) for t in terms)
                assert abs(Fraction(float(y32[r, j])) - exact) <= Fraction(_gamma32(k)) * absd
        assert np.array_equal(y16, workloads.bf16_bits(y32))


def test_f32seq_sums_in_ascending_k(oracle_lib):
    """Products [2^24, 1, 1] (D = 16, 2, 2 with x = 2^20, 0.5, 0.5): summed in
    ascending k in fp32 they give 2^24 (each +1 is a tie that rounds to even),
    while the exact sum, and the fp64 projection, give 2^24 + 2.  Reversed
    (k order 1, 1, 2^24) the fp32 sum is exact."""
    codes = np.zeros((1, 8), np.uint8)
    codes[0, 0] = 0x16          # k0: code 0x6 (4.0), k1: code 0x1 (0.5)
    codes[0, 1] = 0x01          # k2: code 0x1 (0.5)
    scales = np.array([[0x48]], np.uint8)   # E4M3 4.0: D = 16, 2, 2
    x = workloads.bf16_bits(np.array([[2.0 ** 20, 0.5, 0.5] + [0.0] * 13], np.float32))
    y32, _ = oracle_lib.gemv_f32seq(codes, scales, np.float32(1.0), x)
    y64, _, _ = oracle_lib.gemv(codes, scales, np.float32(1.0), x)
    assert y32[0, 0] == np.float32(2.0 ** 24)
    assert y64[0, 0] == 2.0 ** 24 + 2
    rcodes = np.zeros((1, 8), np.uint8)
    rcodes[0, 0] = 0x11
    rcodes[0, 1] = 0x06
    xr = workloads.bf16_bits(np.array([[0.5, 0.5, 2.0 ** 20] + [0.0] * 13], np.float32))
    y32r, _ = oracle_lib.gemv_f32seq(rcodes, scales, np.float32(1.0), xr)
    assert y32r[0, 0] == np.float32(2.0 ** 24 + 2)


def test_f32seq_equals_fp64_where_every_partial_sum_is_exact(oracle_lib):
    """codes x scales in {0.5, 1, 2} x x in {0, +-0.5, +-1}: every partial sum
    is a multiple of 2^-3 below 2^17, so fp32 and fp64 agree exactly; one-hot
    activations return a column of D."""
    rng = np.random.default_rng(23)
    n, k, rows = 33, 1040, 5
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), size=(n, k // 16))
    x = workloads.bf16_bits(rng.choice(np.array([-1.0, -0.5, 0.0, 0.5, 1.0], np.float32), size=(rows, k)))
    y32, y16 = oracle_lib.gemv_f32seq(codes, scales, np.float32(1.0), x)
    y64, _, y64b = oracle_lib.gemv(codes, scales, np.float32(1.0), x)
    assert np.array_equal(y32.astype(np.float64), y64)
    assert np.array_equal(y16, y64b)
    D = oracle_lib.dequant(codes, scales, np.float32(1.0))
    onehot = np.zeros((1, k), np.float32)
    onehot[0, 777] = 1.0
    y1, _ = oracle_lib.gemv_f32seq(codes, scales, np.float32(1.0), workloads.bf16_bits(onehot))
    assert np.array_equal(y1[0], D[:, 777])


def test_projection_row_limit_is_enforced_in_c(oracle_lib):
    """The C entry points refuse rows outside 1..64 (their per-thread row
    buffers hold 64) and write nothing; the Python wrappers raise."""
    lib = oracle_lib._load()
    assert lib.nvo_gemv(None, None, 1.0, 1, 16, None, 65, None, 0, None, None, None) == -1
    assert lib.nvo_gemv(None, None, 1.0, 1, 16, None, 0, None, 0, None, None, None) == -1
    assert lib.nvo_gemv_f32seq(None, None, 1.0, 1, 16, None, 65, None, 0, None, None) == -1
    assert lib.nvo_gemv_dual_silu(None, None, 1.0, None, None, 1.0, 1, 16, None, 65, None, 0,
                                  None, None, None, None, None, None) == -1
    codes = np.zeros((1, 8), np.uint8)
    scales = np.zeros((1, 1), np.uint8)
    with pytest.raises(ValueError):
        oracle_lib.gemv(codes, scales, 1.0, np.zeros((65, 16), np.uint16))
