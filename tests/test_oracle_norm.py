"""Pins of the oracle's residual add + RMSNorm (the step producing a
projection's activations: the Qwen3.8-27B-NVFP4 blueprint page's kernel table,
norm::residual_add_rms_norm; kern's gemma_rms_norm adds the Gemma offset),
against hand-derived values, closed forms and numpy."""
import numpy as np

import oracle
import workloads


def _bf16(a):
    return workloads.bf16_bits(np.asarray(a, np.float32))


def _val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_worked_row():
    """v = (3, 4, 0, 0): mean(v^2) = 25/4, rms 2.5, so x = (1.2, 1.6, 0, 0) with
    w = 1, which round to bf16 0x3F9A (1.203125) and 0x3FCD (1.6015625); with
    the Gemma offset and w = 0 the same."""
    r = _bf16([[1.0, 4.0, 0.0, -2.0]])
    h = _bf16([[2.0, 0.0, 0.0, 2.0]])
    ro, x, inv = oracle.residual_rmsnorm(r, h, _bf16([1.0, 1.0, 1.0, 1.0]), 0.0)
    assert list(ro[0]) == list(_bf16([3.0, 4.0, 0.0, 0.0]))
    assert inv[0] == 0.4
    assert list(x[0]) == [0x3F9A, 0x3FCD, 0, 0]
    _, xg, _ = oracle.residual_rmsnorm(r, h, _bf16([0.0] * 4), 0.0, gemma_offset=True)
    assert list(xg[0]) == [0x3F9A, 0x3FCD, 0, 0]


def test_residual_is_the_rounded_sum():
    """r_out = RNE(r + h): numpy's float32 sum of the two bf16 values (exact or
    rounded far below a bf16 half-ulp) rounded to bf16."""
    rng = np.random.default_rng(3)
    r = _bf16(rng.standard_normal((5, 300)))
    h = _bf16(rng.standard_normal((5, 300)) * np.exp2(rng.integers(-20, 20, (5, 300))))
    ro, _, _ = oracle.residual_rmsnorm(r, h, _bf16(np.ones(300)), 1e-6)
    want = _bf16((_val(r) + _val(h)).astype(np.float32))
    assert np.array_equal(ro, want)


def test_constant_row_gives_sign_times_weight():
    """A row of one value c with eps = 0 has rms |c|: x = sign(c) * w exactly."""
    rng = np.random.default_rng(4)
    k = 64
    w = _bf16(rng.standard_normal(k))
    for c in (-3.5, 0.0078125, 96.0):
        _, x, _ = oracle.residual_rmsnorm(_bf16(np.full((1, k), c)), np.zeros((1, k), np.uint16), w, 0.0)
        assert np.array_equal(x[0], _bf16(np.sign(c) * _val(w)))


def test_power_of_two_scaling_invariance_and_eps():
    """With eps = 0, scaling a row by 2^s leaves x unchanged; eps adds to the
    mean square (inv_rms matches the closed form from numpy)."""
    rng = np.random.default_rng(6)
    k = 257
    v = _bf16(rng.standard_normal((1, k)))
    w = _bf16(rng.standard_normal(k))
    z = np.zeros((1, k), np.uint16)
    _, x0, _ = oracle.residual_rmsnorm(v, z, w, 0.0)
    for s in (-8, 5):
        _, xs, _ = oracle.residual_rmsnorm(_bf16(_val(v) * 2.0 ** s), z, w, 0.0)
        assert np.array_equal(x0, xs)
    _, _, inv = oracle.residual_rmsnorm(v, z, w, 0.25)
    assert np.isclose(inv[0], 1.0 / np.sqrt(np.mean(_val(v) ** 2) + 0.25), rtol=1e-15)
