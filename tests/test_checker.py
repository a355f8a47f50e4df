"""The tolerance checks can fail: mistakes planted in a copy of the oracle's
own result (on the CPU) must be caught by R14 (fp32 bound), R15 (bf16 within
one ulp outside the cancellation band) and R16 (pair), and results inside the
band are exempt and counted."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import check


def _case(seed=5):
    c = workloads.case(96, 1040, 3, seed=seed)
    q = oracle.quantize(c["W"])
    ref, absd, ref16 = oracle.gemv(*q, c["x"])
    return q, c["x"], ref, absd, ref16


def test_oracle_own_result_passes():
    _, _, ref, absd, ref16 = _case()
    y32 = ref.astype(np.float32)
    st = check.check_gemv(y32, workloads.bf16_bits(y32), ref, absd, ref16, label="self")
    assert st["bf16_max_ulp"] <= 1


def test_r15_catches_a_few_ulp_error_that_r14_allows():
    """Scale every output by (1 + 2^-6): about four bf16 ulps, while the fp32
    error stays under 1e-3 * sum|D*x| wherever |y| < 0.064 sum|D*x|."""
    _, _, ref, absd, ref16 = _case(6)
    y32 = (ref * (1 + 2.0 ** -6)).astype(np.float32)
    inside = np.abs(ref) * 2.0 ** -6 < 1e-3 * absd          # R14 still holds here
    outside_band = np.abs(ref) >= 2.0 ** -12 * absd
    assert np.any(inside & outside_band)
    keep = inside
    # outputs R14 itself would reject are replaced by the oracle's value
    y32 = np.where(keep, y32, ref.astype(np.float32))
    with pytest.raises(AssertionError, match="more than 1 ulp"):
        check.check_gemv(y32, workloads.bf16_bits(y32), ref, absd, ref16, label="planted")


def test_r15_exempts_the_cancellation_band():
    """An output below 2^-12 sum|D*x| may be several bf16 ulps off: exempt and
    counted, R14 alone applies."""
    ref = np.array([[1.0, -3.0, 2.0 ** -20]])
    absd = np.array([[2.0 ** 14, 2.0 ** 15, 1.0]])
    y32 = (ref * (1 + 2.0 ** -5)).astype(np.float32)
    ref16 = workloads.bf16_bits(ref.astype(np.float32))
    st = check.check_gemv(y32, workloads.bf16_bits(y32), ref, absd, ref16, label="band")
    assert st["bf16_exempt"] == 3


def test_r14_catches_a_group_lost_to_a_large_activation():
    """x = 2^16 on a zero code and 2^-8 on 15 codes +-1: a path that scales a
    group's activations by its largest and keeps 21 binades below it returns 0
    here; R14 rejects that (error = the whole result)."""
    codes = np.zeros((8, 8), np.uint8)
    nib = np.array([0x0] + [0x2, 0xA] * 7 + [0x2], np.uint8)
    codes[:, :] = nib[0::2] | (nib[1::2] << 4)
    scales = np.full((8, 1), 0x38, np.uint8)
    xv = np.array([[2.0 ** 16] + [2.0 ** -8] * 15], np.float32)
    ref, absd, ref16 = oracle.gemv(codes, scales, np.float32(1.0), workloads.bf16_bits(xv))
    assert np.all(ref == 2.0 ** -8) and np.all(absd == 15 * 2.0 ** -8)
    with pytest.raises(AssertionError, match="exceed"):
        check.check_gemv(np.zeros_like(ref, np.float32), None, ref, absd, ref16, label="lost group")


def test_r16_catches_planted_pair_errors():
    c = workloads.case(64, 512, 2, seed=8, dual=True)
    gq, uq = oracle.quantize(c["W"]), oracle.quantize(c["W_up"])
    d = oracle.gemv_dual_silu(gq, uq, c["x"])
    o = d["o"].astype(np.float32)
    check.check_dual(o, workloads.bf16_bits(o), d, label="pair self")
    bad = (d["o"] * (1 + 2.0 ** -5)).astype(np.float32)
    with pytest.raises(AssertionError):
        check.check_dual(bad, workloads.bf16_bits(bad), d, label="pair planted")
