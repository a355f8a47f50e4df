"""GPU parity of the residual add + RMSNorm (the step producing a projection's
activations: the blueprint page's norm::residual_add_rms_norm, kern's
gemma_rms_norm for the offset variant) against the CPU oracle.

* residual_out bit-exact (bf16 RNE of a sum that fp32 holds exactly or far
  below a bf16 half-ulp);
* x within one bf16 ulp of the oracle's RNE of the fp64 value (fp32 sum of
  squares, square root and products on the device), every element;
* in place (residual_out = residual) equals out of place; closed forms exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

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


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _ordered(b):
    b = b.astype(np.int64)
    return np.where(b >= 0x8000, -(b & 0x7FFF), b)


@pytest.mark.parametrize("rows,k", [(1, 5120), (8, 5120), (3, 16), (5, 784), (2, 65536), (300, 2048), (16, 17408)])
@pytest.mark.parametrize("gemma", [False, True])
def test_norm_random(nv, rows, k, gemma):
    rng = np.random.default_rng(rows * 7 + k + gemma)
    r = _bf16(rng.standard_normal((rows, k)) * 4.0)
    h = _bf16(rng.standard_normal((rows, k)))
    w = _bf16(rng.standard_normal(k) * 0.1 + (0.0 if gemma else 1.0))
    eps = 1e-6
    ro, x = nv.nvfp4_residual_rmsnorm(_dev(r), _dev(h), _dev(w), eps=eps, gemma_offset=gemma)
    ro2, x2 = nv.nvfp4_residual_rmsnorm(_dev(r), _dev(h), _dev(w), eps=eps, gemma_offset=gemma)
    torch.cuda.synchronize()
    ro_ref, x_ref, _ = oracle.residual_rmsnorm(r, h, w, eps, gemma_offset=gemma)
    assert np.array_equal(_bits(ro), ro_ref)
    assert np.array_equal(_bits(x), _bits(x2)), "not deterministic"
    d = np.abs(_ordered(_bits(x)) - _ordered(x_ref))
    assert d.max() <= 1, (rows, k, gemma, int(d.max()))
    print("norm rows=%d k=%d gemma=%d: %.4f%% of x one ulp from the oracle" % (rows, k, gemma, 100 * np.mean(d)))


def test_norm_in_place_equals_out_of_place(nv):
    rng = np.random.default_rng(11)
    rows, k = 4, 5120
    r = _bf16(rng.standard_normal((rows, k)))
    h = _bf16(rng.standard_normal((rows, k)))
    w = _bf16(rng.standard_normal(k))
    ro, x = nv.nvfp4_residual_rmsnorm(_dev(r), _dev(h), _dev(w))
    rd = _dev(r)
    ro2, x2 = nv.nvfp4_residual_rmsnorm(rd, _dev(h), _dev(w), residual_out=rd)
    torch.cuda.synchronize()
    assert ro2.data_ptr() == rd.data_ptr()
    assert np.array_equal(_bits(ro), _bits(rd)) and np.array_equal(_bits(x), _bits(x2))


def test_norm_closed_forms(nv):
    """Rows of the value 2 (split over residual and delta) with eps = 0: the
    mean square is 4, 1/sqrt(4) = 0.5 exactly, x = w bit for bit.  All-zero
    rows with eps > 0 give x = 0."""
    rows, k = 3, 1024
    rng = np.random.default_rng(12)
    w = _bf16(rng.standard_normal(k))
    one = _bf16(np.ones((rows, k)))
    ro, x = nv.nvfp4_residual_rmsnorm(_dev(one), _dev(one), _dev(w), eps=0.0)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ro), _bf16(np.full((rows, k), 2.0)))
    assert np.array_equal(_bits(x), np.broadcast_to(w, (rows, k)))
    z = np.zeros((rows, k), np.uint16)
    _, x = nv.nvfp4_residual_rmsnorm(_dev(z), _dev(z), _dev(w), eps=1e-5)
    torch.cuda.synchronize()
    assert not (_bits(x) & 0x7FFF).any()
