"""Pins of the oracle's scalar codecs against things other than itself:
the E2M1 value set, brute-force nearest-grid search, torch's float8_e4m3fn and
bfloat16 conversions (library routines), and hand-derived fixtures."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# The E2M1 (FP4) value set by code 0..7, as the OCP microscaling format tables it.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden_pairs(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            out.append((a, b))
    return out


# ---- E2M1 -----------------------------------------------------------------

def test_e2m1_decode_exhaustive(oracle_lib):
    for c in range(16):
        v = oracle_lib.e2m1_value(c)
        mag = E2M1_TABLE[c & 7]
        assert abs(v) == mag
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0), c


def _e2m1_brute(v: float) -> int:
    """Nearest grid point by exhaustive search; ties -> even mantissa bit."""
    a = abs(v)
    best = None
    for c in range(8):
        d = abs(Fraction(a) - Fraction(E2M1_TABLE[c]))
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    return sign | best[1]


def test_e2m1_encode_golden(oracle_lib):
    for a, b in _golden_pairs("e2m1_rounding.txt"):
        v = float(np.float32(float(a)))
        assert oracle_lib.e2m1_encode(v) == int(b, 16), a


def test_e2m1_encode_all_bf16_inputs(oracle_lib):
    # every finite bf16 bit pattern, as fp32
    bits = np.arange(65536, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # restrict brute force to the interesting range; beyond it saturation is
    # checked on a sample
    inrange = vals[np.abs(vals) <= 16.0]
    for v in inrange:
        assert oracle_lib.e2m1_encode(float(v)) == _e2m1_brute(float(v)), v
    big = vals[np.abs(vals) > 16.0][::97]
    for v in big:
        assert oracle_lib.e2m1_encode(float(v)) == (8 if v < 0 else 0) | 7


def test_e2m1_encode_midpoints_and_neighbours(oracle_lib):
    mids = [(E2M1_TABLE[i] + E2M1_TABLE[i + 1]) / 2 for i in range(7)]
    vals = []
    for m in mids + E2M1_TABLE:
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(100))]
    for v in vals:
        for s in (1.0, -1.0):
            x = float(v) * s
            assert oracle_lib.e2m1_encode(x) == _e2m1_brute(x), x


def test_e2m1_encode_random(oracle_lib):
    rng = np.random.default_rng(123)
    vals = (rng.standard_normal(20000) * 3).astype(np.float32)
    for v in vals:
        assert oracle_lib.e2m1_encode(float(v)) == _e2m1_brute(float(v))


# ---- E4M3 -----------------------------------------------------------------

def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_exhaustive_vs_torch(oracle_lib):
    ref = _torch_e4m3_values()
    for b in range(256):
        v = oracle_lib.e4m3_value(b)
        if np.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), b
    assert oracle_lib.e4m3_value(0x7E) == 448.0


def test_e4m3_golden(oracle_lib):
    for a, b in _golden_pairs("e4m3_values.txt"):
        v = oracle_lib.e4m3_value(int(a, 16))
        if b == "nan":
            assert math.isnan(v)
        else:
            assert v == float(b) and math.copysign(1, v) == math.copysign(1, float(b)), a


def _torch_e4m3_encode(vals: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().astype(np.int64)


def _e4m3_brute(v: float) -> int:
    grid = _torch_e4m3_values()
    best = None
    a = Fraction(abs(v))
    for b in range(0x7F):  # finite non-negative codes 0x00..0x7E
        d = abs(a - Fraction(float(grid[b])))
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return (0x80 if math.copysign(1.0, v) < 0 else 0) | best[1]


def test_e4m3_encode_vs_torch_and_brute_force(oracle_lib):
    grid = _torch_e4m3_values()[:0x7F].astype(np.float64)
    vals = []
    for i in range(len(grid) - 1):
        m = np.float32((grid[i] + grid[i + 1]) / 2)
        vals += [np.float32(grid[i]), m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    rng = np.random.default_rng(7)
    vals += list((2.0 ** rng.uniform(-12, np.log2(448), 3000)).astype(np.float32))
    vals = np.array(vals, np.float32)
    vals = vals[vals <= 448]
    ref = _torch_e4m3_encode(vals)
    for v, r in zip(vals, ref):
        got = oracle_lib.e4m3_encode(float(v))
        assert got == r, (v, got, r)
        assert oracle_lib.e4m3_encode(-float(v)) == (r | 0x80)
    for v in vals[::50]:
        assert oracle_lib.e4m3_encode(float(v)) == _e4m3_brute(float(v))


def test_e4m3_encode_saturates_never_nan(oracle_lib):
    for v in [448.0, 448.00003, 463.9, 464.0, 465.0, 1e6, 3.0e38, float("inf")]:
        assert oracle_lib.e4m3_encode(v) == 0x7E, v
    # torch (non-saturating) agrees up to the rounding boundary
    assert _torch_e4m3_encode(np.array([463.9], np.float32))[0] == 0x7E
    # smallest subnormal and the tie below it
    assert oracle_lib.e4m3_encode(2.0 ** -9) == 0x01
    assert oracle_lib.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle_lib.e4m3_encode(1.5 * 2.0 ** -10) == 0x01


# ---- bf16 -----------------------------------------------------------------

def test_bf16_from_double_vs_torch_on_fp32_values(oracle_lib):
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # bf16 subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(vals, ref):
        assert oracle_lib.bf16_from_double(float(v)) == int(r), v


def test_bf16_from_double_no_double_rounding(oracle_lib):
    # 1 + 2^-8 is the exact midpoint between bf16 1.0 and 1.0078125; nudged up
    # by 2^-40 it must round up, although its nearest fp32 is the midpoint itself
    # (where ties-to-even would round down to 1.0).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)
    assert oracle_lib.bf16_from_double(v) == 0x3F81
    assert oracle_lib.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle_lib.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle_lib.bf16_from_double(-0.0) == 0x8000
    assert oracle_lib.bf16_from_double(float("inf")) == 0x7F80
    assert oracle_lib.bf16_from_double(3.5e38) == 0x7F80


def test_bf16_value_exhaustive(oracle_lib):
    bits = np.arange(0, 65536, 37, dtype=np.uint32)
    ref = (bits << 16).view(np.float32)
    for b, r in zip(bits, ref):
        v = oracle_lib.bf16_value(int(b))
        if np.isnan(r):
            assert math.isnan(v)
        else:
            assert v == float(r)
