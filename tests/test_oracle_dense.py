"""Pins of the oracle's dense bf16 projection (the lm head kept in bf16: the
Qwen3.8-27B-NVFP4 blueprint page, "Precision" table and its kernel table,
gemv::dense_gemv_bf16), each against something other than the oracle's own
loop: exact closed forms, numpy's integer matrix product, and hand-derived
bf16 rounding ties."""
import numpy as np
import pytest

import oracle
import workloads


def _bf16(a):
    return workloads.bf16_bits(np.asarray(a, np.float32))


def _val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_one_hot_rows_pick_scaled_columns():
    """W[j] = 2^s_j at column perm[j], zero elsewhere: y[r][j] = 2^s_j x[r][perm[j]]
    exactly.  A transposed W or a wrong index fails this."""
    rng = np.random.default_rng(1)
    n, k, rows = 37, 48, 5
    perm = rng.permutation(k)[:n] if n <= k else rng.integers(0, k, n)
    s = rng.integers(-6, 7, n)
    W = np.zeros((n, k), np.float32)
    W[np.arange(n), perm] = np.exp2(s)
    xb = _bf16(rng.standard_normal((rows, k)))
    y, a, yb = oracle.dense_gemv(_bf16(W), xb)
    want = _val(xb)[:, perm] * np.exp2(s)[None, :]
    assert np.array_equal(y, want)
    assert np.array_equal(a, np.abs(want))
    assert np.array_equal(yb, _bf16(want.astype(np.float32)))   # exact values round to themselves


@pytest.mark.parametrize("n,k,rows", [(1, 16, 1), (33, 200, 3), (64, 1024, 8), (7, 4112, 16)])
def test_small_integers_match_numpy_integer_product(n, k, rows):
    """Values q * 2^-2 with |q| <= 15: every product and partial sum is exact in
    fp64, so y equals numpy's int64 matrix product (scaled) exactly, and
    sum|W x| equals the product of the absolute values."""
    rng = np.random.default_rng(n * k + rows)
    wq = rng.integers(-15, 16, (n, k))
    xq = rng.integers(-15, 16, (rows, k))
    y, a, _ = oracle.dense_gemv(_bf16(wq * 0.25), _bf16(xq * 0.25))
    assert np.array_equal(y, (xq @ wq.T).astype(np.float64) / 16.0)
    assert np.array_equal(a, (np.abs(xq) @ np.abs(wq).T).astype(np.float64) / 16.0)


def test_bf16_copy_rounds_ties_to_even():
    """y = 1 + 2^-8 lies halfway between bf16 1.0 (0x3F80) and 1 + 2^-7 (0x3F81):
    it rounds to 0x3F80; y = 1 + 3 * 2^-8, halfway between 0x3F81 and 0x3F82,
    rounds to 0x3F82; y = -(1 + 2^-8) to 0xBF80."""
    W = _bf16([[1.0, 2.0 ** -8], [1.0, 3 * 2.0 ** -8], [-1.0, -(2.0 ** -8)]])
    y, _, yb = oracle.dense_gemv(W, _bf16([[1.0, 1.0]]))
    assert list(y[0]) == [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]
    assert list(yb[0]) == [0x3F80, 0x3F82, 0xBF80]


def test_selected_features_equal_the_full_result():
    rng = np.random.default_rng(5)
    W = _bf16(rng.standard_normal((50, 96)) * 0.02)
    x = _bf16(rng.standard_normal((4, 96)))
    full = oracle.dense_gemv(W, x)
    sel = np.array([49, 0, 17, 17, 3])
    part = oracle.dense_gemv(W, x, sel=sel)
    for f, p in zip(full, part):
        assert np.array_equal(f[:, sel], p)
