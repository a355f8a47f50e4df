"""Pins of the oracle quantizer and dequantizer: a hand-worked row, invariants
(nearest-grid codes, sign and power-of-two symmetry, the amax group), exact
round trips on grid tensors, and the special cases of the readings."""
import math
import os

import numpy as np
import pytest
import torch

from test_oracle_codecs import E2M1_TABLE, _torch_e4m3_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def _code_values(codes: np.ndarray) -> np.ndarray:
    """Unpack low-nibble-first codes into signed E2M1 values (float64)."""
    lo = codes & 15
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    mag = np.array(E2M1_TABLE)[c & 7]
    return np.where(c & 8, -mag, mag), c


def test_worked_row_quantize(oracle_lib):
    g = load_kv("worked_row.txt")
    W = np.array([float(v) for v in g["W"]], np.float32)[None, :]
    codes, scales, sg = oracle_lib.quantize(W)
    assert sg == np.float32(float(g["s_g"][0]))
    assert [int(b, 16) for b in g["scales"]] == scales[0].tolist()
    assert [int(b, 16) for b in g["codes"]] == codes[0].tolist()
    D = oracle_lib.dequant(codes, scales, sg)
    ref = np.array([float(v) for v in g["D"]], np.float32)
    assert np.array_equal(D[0], ref)
    assert np.array_equal(np.signbit(D[0]), np.signbit(ref))


def test_dequant_vs_library_decodes(oracle_lib):
    """D = fp32(e2m1 * e4m3) * s_g with the E4M3 factor decoded by torch."""
    rng = np.random.default_rng(11)
    n, k = 37, 96
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (n, k // 16), dtype=np.uint8)  # finite, non-negative
    sg = np.float32(0.0123)
    vals, _ = _code_values(codes)
    sc = np.repeat(_torch_e4m3_values()[scales].astype(np.float64), 16, axis=1)
    ref = (vals * sc).astype(np.float32) * sg
    D = oracle_lib.dequant(codes, scales, sg)
    assert np.array_equal(D, ref)
    assert np.array_equal(np.signbit(D), np.signbit(ref))


def _quant_invariants(oracle_lib, W):
    codes, scales, sg = oracle_lib.quantize(W)
    n, k = W.shape
    vals, c = _code_values(codes)
    S = np.repeat(_torch_e4m3_values()[scales].astype(np.float32), 16, axis=1) * sg  # fp32 product
    # (ii) each code is a nearest grid point to W/S (ties: even mantissa) ...
    q = np.where(S != 0, W / np.where(S != 0, S, 1), 0).astype(np.float32)
    a = np.abs(q.astype(np.float64))
    grid = np.array(E2M1_TABLE)
    d = np.abs(a[..., None] - grid)                       # distance to every grid point
    dmin = d.min(axis=-1)
    chosen = d[np.arange(n)[:, None], np.arange(k)[None, :], c & 7]
    assert np.all((chosen == dmin) | (S == 0))
    tie = (np.sum(d == dmin[..., None], axis=-1) > 1)
    assert np.all(~tie | ((c & 1) == 0) | (S == 0))
    # ... and carries the sign of W (zero groups excepted)
    assert np.all(((c & 8) != 0) == np.signbit(W) | (S == 0))
    # scales are finite and non-negative; the amax group gets 448, its amax code is +-6
    assert np.all(scales <= 0x7E)
    amax = np.abs(W).max()
    r, col = np.unravel_index(np.argmax(np.abs(W)), W.shape)
    if amax > 0:
        assert scales[r, col // 16] == 0x7E
        assert (c[r, col] & 7) == 7
    return codes, scales, sg


def test_quantizer_invariants_random(oracle_lib):
    rng = np.random.default_rng(3)
    for n, k, outl in [(16, 64, 0.0), (40, 256, 0.01), (7, 48, 0.2)]:
        W = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
        if outl:
            gi = rng.choice(n * k // 16, size=max(1, int(outl * n * k // 16)), replace=False)
            W.reshape(-1, 16)[gi] *= np.float32(50)
        _quant_invariants(oracle_lib, W)


def test_quantizer_sign_symmetry(oracle_lib):
    rng = np.random.default_rng(4)
    W = rng.standard_normal((24, 128), dtype=np.float32) * np.float32(0.02)
    c1, s1, g1 = oracle_lib.quantize(W)
    c2, s2, g2 = oracle_lib.quantize(-W)
    assert g1 == g2 and np.array_equal(s1, s2)
    assert np.array_equal(c1 ^ 0x88, c2)


def test_quantizer_power_of_two_scaling(oracle_lib):
    rng = np.random.default_rng(5)
    W = rng.standard_normal((24, 128), dtype=np.float32) * np.float32(0.02)
    c1, s1, g1 = oracle_lib.quantize(W)
    for j in (-3, 1, 5):
        c2, s2, g2 = oracle_lib.quantize(W * np.float32(2.0 ** j))
        assert g2 == g1 * np.float32(2.0 ** j)
        assert np.array_equal(s1, s2) and np.array_equal(c1, c2)


def _grid_tensor(rng, n, k, sg):
    """Random codes with a +-6 in every group and random non-zero E4M3 scales
    (one group at 448), dequantized exactly with a power-of-two s_g."""
    c = rng.integers(0, 16, (n, k), dtype=np.uint8)
    pos = rng.integers(0, 16, (n, k // 16))
    for g in range(k // 16):
        c[np.arange(n), 16 * g + pos[:, g]] = 7 | (rng.integers(0, 2, n) * 8).astype(np.uint8)
    scales = rng.integers(1, 0x7F, (n, k // 16), dtype=np.uint8)
    scales[rng.integers(0, n), rng.integers(0, k // 16)] = 0x7E
    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    mag = np.array(E2M1_TABLE)[c & 7]
    v = np.where(c & 8, -mag, mag)
    W = (v * np.repeat(_torch_e4m3_values()[scales].astype(np.float64), 16, axis=1) * float(sg))
    W32 = W.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), W)  # exact
    return W32, codes, scales


def test_quantizer_round_trip_on_grid_tensors(oracle_lib):
    rng = np.random.default_rng(6)
    for sg in (2.0 ** -12, 2.0 ** -3, 1.0):
        W, codes, scales = _grid_tensor(rng, 33, 160, sg)
        c2, s2, g2 = oracle_lib.quantize(W)
        assert g2 == np.float32(sg)
        assert np.array_equal(s2, scales)
        assert np.array_equal(c2, codes)
        # and dequantization reproduces the tensor bit for bit
        D = oracle_lib.dequant(c2, s2, g2)
        assert np.array_equal(D, W) and np.array_equal(np.signbit(D), np.signbit(W))


def test_quantizer_zero_tensor_and_zero_groups(oracle_lib):
    W = np.zeros((3, 32), np.float32)
    c, s, g = oracle_lib.quantize(W)
    assert g == 0 and not s.any() and not c.any()
    W = np.zeros((2, 48), np.float32)
    W[0, 0] = 1.0
    W[1, 16:32] = -0.0
    W[1, 32:48] = -1e-9       # rounds to a zero E4M3 scale
    c, s, g = oracle_lib.quantize(W)
    assert s[1, 1] == 0 and s[1, 2] == 0
    assert not c[1].any()      # every code 0x0 in zero-scale groups


def test_quantizer_rejects_non_finite(oracle_lib):
    for bad in (np.nan, np.inf, -np.inf):
        W = np.ones((2, 16), np.float32)
        W[1, 3] = bad
        with pytest.raises(ValueError):
            oracle_lib.quantize(W)
    with pytest.raises(ValueError):
        oracle_lib.quantize(np.ones((2, 24), np.float32))


def test_quantizer_subnormal_scales(oracle_lib):
    # a group whose max is tiny relative to amax gets a subnormal E4M3 scale
    W = np.zeros((1, 48), np.float32)
    W[0, 0] = 2688.0                      # s_g = 1
    W[0, 16] = 6.0 * 2.0 ** -9 * 3        # t = 3 * 2^-9 -> subnormal code 3
    W[0, 32] = 6.0 * 2.0 ** -9 * 0.4      # t = 0.4 * 2^-9 -> rounds to zero scale
    c, s, g = oracle_lib.quantize(W)
    assert g == 1.0
    assert s[0].tolist() == [0x7E, 0x03, 0x00]
    assert (c[0, 8] & 15) == 7            # 18*2^-9 / (3*2^-9) = 6
    assert not c[0, 16:].any()
