"""GPU parity of the MXFP4 projection (E2M1 with one E8M0 scale per 32 k, the
format the pages name through the kern build's gpu_mxfp4 kernels) against
the CPU oracle, in the format's own row-major layout.

* fp32 within 1e-3 * sum|w*x| of the fp64 oracle, bf16 = RNE of the device
  fp32 and within one ulp of the oracle's bf16 (oracle.check), ragged n and
  k, row counts 1-40 (chunks past 16);
* exact equality on inputs whose every partial sum is exact in fp32;
* one-hot activation rows read single dequantized weights back, bit for bit,
  over scale bytes from 0 (2^-127) to 252 (2^125: 6 * 2^125 is the largest
  weight bf16 holds), which pins the conversion's use of the scale;
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


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def _x(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(nv, c, s, xb):
    cd, sd, x = _u8(c), _u8(s), _x(xb)
    y32 = nv.nvfp4_mxfp4_gemv(cd, sd, x, out_dtype=torch.float32)
    y16 = nv.nvfp4_mxfp4_gemv(cd, sd, x)
    y32b = nv.nvfp4_mxfp4_gemv(cd, sd, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = y32.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), y32b.cpu().numpy().view(np.uint32)), "not deterministic"
    return a, y16.cpu().view(torch.int16).numpy().view(np.uint16)


# groups of 32 features with one wave over all of k below 32768 (the first six), of 64 with two
# waves over halves of k from there on (the last two)
@pytest.mark.parametrize("n,k", [(1, 32), (65, 4128), (200, 800), (1000, 5120), (64, 17408), (130, 96),
                                 (32800, 256), (40000, 288)])
def test_mx_random(nv, n, k):
    rng = np.random.default_rng(n * 13 + k)
    c, s = oracle.mx_quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    for rows in (1, 2, 8, 16, 17, 40):
        xb = workloads.bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
        y32, y16 = _run(nv, c, s, xb)
        ref, absd, ref16 = oracle.mx_gemv(c, s, xb)
        check.check_gemv(y32, y16, ref, absd, ref16, label="mxfp4 %dx%d rows=%d" % (n, k, rows))


@pytest.mark.parametrize("n,k", [(64, 256), (97, 4128), (300, 2048)])
def test_mx_exact_arithmetic(nv, n, k):
    """Scale bytes 125..129 (2^-2..2^2), x = q / 4 with |q| <= 7: products are
    multiples of 2^-5 below 2^5 and sums stay below 2^18: exact in fp32."""
    rng = np.random.default_rng(n + 3 * k)
    c = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    s = rng.integers(125, 130, (n, k // 32)).astype(np.uint8)
    for rows in (1, 5, 16):
        xb = workloads.bf16_bits((rng.integers(-7, 8, (rows, k)) * 0.25).astype(np.float32))
        y32, y16 = _run(nv, c, s, xb)
        ref, _, ref16 = oracle.mx_gemv(c, s, xb)
        assert np.array_equal(y32.astype(np.float64), ref), (n, k, rows)
        assert np.array_equal(y16, ref16), (n, k, rows)


def test_mx_single_weights_over_the_scale_range(nv):
    """Row r of x is one-hot at column j_r: y[r][f] = weight[f][j_r] exactly,
    for every code and scale bytes 0, 1, 2, 100, 127, 200, 252."""
    n, k = 16 * 7, 64
    rng = np.random.default_rng(21)
    c = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    c[:, 0] = np.arange(n, dtype=np.uint8)          # every code pair in column 0..1 somewhere
    sb = np.array([0, 1, 2, 100, 127, 200, 252], np.uint8)
    s = np.repeat(sb, 16)[:, None].repeat(k // 32, axis=1)
    D = oracle.mx_dequant(c, s)
    cols = np.array([0, 1, 2, 31, 32, 33, 63, 40])
    xv = np.zeros((len(cols), k), np.float32)
    xv[np.arange(len(cols)), cols] = 1.0
    y32, _ = _run(nv, c, s, workloads.bf16_bits(xv))
    want = D[:, cols].T
    ok = y32.astype(np.float64) == want
    bad = np.argwhere(~ok)
    assert ok.all(), "first mismatches (row, feature, got, want, scale byte): %s" % [
        (int(r), int(f), float(y32[r, f]), float(want[r, f]), int(s[f, 0])) for r, f in bad[:6]]


@pytest.mark.parametrize("offset", [0, 1, 4])
def test_mx_scale_pointer_alignment(nv, offset):
    """k a multiple of 256 takes 8-byte scale loads when the scale pointer is
    8-byte aligned and byte loads otherwise: the same matrix with its scales at
    a byte offset inside a larger buffer must give the same, correct result."""
    n, k = 300, 1024
    rng = np.random.default_rng(4242)
    c, s = oracle.mx_quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    big = torch.zeros(s.size + 16, dtype=torch.uint8, device="cuda")
    big[offset:offset + s.size] = _u8(s.reshape(-1))
    sd = big[offset:offset + s.size].view(n, k // 32)
    cd = _u8(c)
    for rows in (1, 8):
        xb = workloads.bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
        x = _x(xb)
        y32 = nv.nvfp4_mxfp4_gemv(cd, sd, x, out_dtype=torch.float32)
        y16 = nv.nvfp4_mxfp4_gemv(cd, sd, x)
        torch.cuda.synchronize()
        ref, absd, ref16 = oracle.mx_gemv(c, s, xb)
        check.check_gemv(y32.cpu().numpy(), y16.cpu().view(torch.int16).numpy().view(np.uint16), ref, absd, ref16,
                         label="mxfp4 scales at +%d rows=%d" % (offset, rows))
