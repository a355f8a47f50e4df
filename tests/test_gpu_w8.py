"""GPU parity of the W8G32_F16S projection (signed 8-bit weights with one fp16
scale per 32 k, symmetric: the encoding the pages name for the DFlash2
drafter's matrices) against the CPU oracle.

* fp32 within 1e-3 * sum|w*x| of the fp64 oracle, bf16 = RNE of the device
  fp32 and within one ulp of the oracle's bf16 (oracle.check), ragged n, row
  counts 1-40 (chunks past 16);
* exact equality where every product and partial sum is exact in fp32;
* run-to-run bitwise determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_weight_only_nvfp4_amd as nv
    nv.lib()
    return nv


def _run(nv, c, s, xb):
    cd = torch.from_numpy(np.ascontiguousarray(c)).cuda()
    sd = torch.from_numpy(np.ascontiguousarray(s).view(np.float16)).cuda()
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(torch.bfloat16)
    y32 = nv.nvfp4_w8g32_gemv(cd, sd, x, out_dtype=torch.float32)
    y16 = nv.nvfp4_w8g32_gemv(cd, sd, x)
    y32b = nv.nvfp4_w8g32_gemv(cd, sd, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = y32.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), y32b.cpu().numpy().view(np.uint32)), "not deterministic"
    return a, y16.cpu().view(torch.int16).numpy().view(np.uint16)


# from 8192 features on the kernel runs 16 features per workgroup, below 32
@pytest.mark.parametrize("n,k", [(1, 128), (65, 4096), (200, 768), (1000, 5120), (64, 17408), (130, 128),
                                 (8200, 1024)])
def test_w8_random(nv, n, k):
    rng = np.random.default_rng(n * 17 + k)
    c, s = oracle.w8_quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    for rows in (1, 2, 8, 16, 17, 40):
        xb = workloads.bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
        y32, y16 = _run(nv, c, s, xb)
        ref, absd, ref16 = oracle.w8_gemv(c, s, xb)
        check.check_gemv(y32, y16, ref, absd, ref16, label="w8g32 %dx%d rows=%d" % (n, k, rows))


@pytest.mark.parametrize("n,k", [(64, 256), (97, 4096), (300, 2048), (8211, 256)])
def test_w8_exact_arithmetic(nv, n, k):
    """Scales 2^-3..2^-1 (exact fp16), codes +-127, x = q / 4 with |q| <= 3:
    each product is a multiple of 2^-5 of magnitude < 48, so every partial sum
    over k <= 4096 stays below 2^18 and is exact in fp32."""
    rng = np.random.default_rng(n + 5 * k)
    c = rng.integers(-127, 128, (n, k)).astype(np.int8)
    s = np.exp2(rng.integers(-3, 0, (n, k // 32))).astype(np.float16).view(np.uint16)
    for rows in (1, 5, 16):
        xb = workloads.bf16_bits((rng.integers(-3, 4, (rows, k)) * 0.25).astype(np.float32))
        y32, y16 = _run(nv, c, s, xb)
        ref, _, ref16 = oracle.w8_gemv(c, s, xb)
        assert np.array_equal(y32.astype(np.float64), ref), (n, k, rows)
        assert np.array_equal(y16, ref16), (n, k, rows)
