"""GPU parity of the dense bf16 projection (the lm head, whose weights stay
bf16: the Qwen3.8-27B-NVFP4 blueprint page, "Precision" table and its kernel
table, gemv::dense_gemv_bf16) against the CPU oracle, through the C ABI.

* fp32 within 1e-3 * sum|w*x| of the fp64 oracle and bf16 = RNE of the device
  fp32, within one ulp of the oracle's bf16 (oracle.check), over ragged n and k
  and every row tier (chunks past 16 rows);
* exact equality on inputs whose every partial sum is exact in fp32;
* run-to-run bitwise determinism;
* a full-size lm head [151936 x 5120] at 1 and 8 rows on sampled outputs.
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


def _bf16(a):
    return workloads.bf16_bits(np.asarray(a, np.float32))


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(nv, Wb, xb):
    W, x = _dev(Wb), _dev(xb)
    y32 = nv.nvfp4_dense_gemv_bf16(W, x, out_dtype=torch.float32)
    y16 = nv.nvfp4_dense_gemv_bf16(W, x)
    y32b = nv.nvfp4_dense_gemv_bf16(W, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = y32.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), y32b.cpu().numpy().view(np.uint32)), "not deterministic"
    return a, y16.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n,k", [(1, 16), (33, 4112), (200, 784), (1000, 5120), (64, 17408), (4133, 528)])
def test_dense_random(nv, n, k):
    rng = np.random.default_rng(n * 31 + k)
    Wb = _bf16(rng.standard_normal((n, k)) * 0.02)
    for rows in (1, 2, 5, 8, 16, 17, 40):
        xb = _bf16(rng.standard_normal((rows, k)))
        y32, y16 = _run(nv, Wb, xb)
        ref, absd, ref16 = oracle.dense_gemv(Wb, xb)
        check.check_gemv(y32, y16, ref, absd, ref16, label="dense %dx%d rows=%d" % (n, k, rows))


@pytest.mark.parametrize("n,k", [(64, 256), (97, 4112), (300, 2048)])
def test_dense_exact_arithmetic(nv, n, k):
    """Values q * 2^-2 with |q| <= 7: products are multiples of 2^-4 and every
    partial sum stays below 2^20, so any fp32 summation order is exact and the
    device result must equal the oracle's bit for bit."""
    rng = np.random.default_rng(n + k)
    Wb = _bf16(rng.integers(-7, 8, (n, k)) * 0.25)
    for rows in (1, 3, 16, 20):
        xb = _bf16(rng.integers(-7, 8, (rows, k)) * 0.25)
        y32, y16 = _run(nv, Wb, xb)
        ref, _, ref16 = oracle.dense_gemv(Wb, xb)
        assert np.array_equal(y32.astype(np.float64), ref), (n, k, rows)
        assert np.array_equal(y16, ref16), (n, k, rows)


def test_dense_zero_and_single_hot(nv):
    """All-zero x gives +0 everywhere; one-hot weight rows pick columns of x."""
    n, k, rows = 70, 336, 3
    rng = np.random.default_rng(9)
    Wb = _bf16(rng.standard_normal((n, k)))
    y32, y16 = _run(nv, Wb, np.zeros((rows, k), np.uint16))
    assert not y32.any() and not np.signbit(y32).any() and not y16.any()
    cols = rng.integers(0, k, n)
    W = np.zeros((n, k), np.float32)
    W[np.arange(n), cols] = 1.0
    xb = _bf16(rng.standard_normal((rows, k)))
    y32, _ = _run(nv, _bf16(W), xb)
    xv = (xb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(y32, xv[:, cols])


@pytest.mark.slow
def test_dense_full_size_lm_head_sampled(nv):
    """[151936 x 5120] bf16 (an lm head of a vocabulary-sized n; the pages give
    no vocabulary size) at 1 and 8 rows: 256 sampled outputs per row against
    the oracle, computed from those weight rows alone."""
    n, k = 151936, 5120
    g = torch.Generator(device="cuda").manual_seed(1234)
    W = (torch.randn((n, k), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    rng = np.random.default_rng(77)
    sel = np.sort(rng.choice(n, 256, replace=False))
    Wsel = W[torch.from_numpy(sel).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
    for rows in (1, 8):
        print("full-size lm head, rows=%d" % rows, flush=True)
        x = (torch.randn((rows, k), generator=g, device="cuda")).to(torch.bfloat16)
        y32 = nv.nvfp4_dense_gemv_bf16(W, x, out_dtype=torch.float32)
        y16 = nv.nvfp4_dense_gemv_bf16(W, x)
        torch.cuda.synchronize()
        xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
        ref, absd, ref16 = oracle.dense_gemv(Wsel, xb)
        check.check_gemv(y32.cpu().numpy()[:, sel], y16.cpu().view(torch.int16).numpy().view(np.uint16)[:, sel],
                         ref, absd, ref16, label="lm head rows=%d" % rows)
    del W
