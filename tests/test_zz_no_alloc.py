"""nvfp4_gemv_noalloc (the entry point for callers that cannot allocate, with
its workspace in the library's static per-device scratch array) against
nvfp4_gemv with a caller workspace, bit for bit, through the C ABI: two calls
in a row, the second with a smaller input, then the first shape again (the
scratch keeps the previous call's contents; its counters must be back at
zero)."""
import ctypes

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


def _case(nv, n, k, rows, seed):
    c = workloads.case(n, k, rows, seed=seed, outlier_frac=0.01)
    codes, scales, sg = oracle.quantize(c["W"])
    w = nv.nvfp4_pack(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), float(sg))
    x = torch.from_numpy(c["x"].view(np.int16)).cuda().view(torch.bfloat16)
    return w, x


def _noalloc(nv, w, x, out):
    st = nv.lib().nvfp4_gemv_noalloc(ctypes.byref(w.desc), x.data_ptr(), x.shape[0], out.data_ptr(),
                                     nv.NVFP4_OUT_F32 if out.dtype == torch.float32 else nv.NVFP4_OUT_BF16,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0, nv.lib().nvfp4_last_error()
    return out


def test_noalloc_matches_gemv_two_calls_then_smaller(nv):
    # down-like shape with split-K pieces (uses the scratch's partials and
    # counters), then a smaller one, then the first again
    cases = [(5120, 17408, 8, 31), (1000, 4112, 3, 32), (5120, 17408, 8, 31)]
    for n, k, rows, seed in cases:
        assert nv.nvfp4_workspace_bytes(n, k, rows) > 0
        w, x = _case(nv, n, k, rows, seed)
        for dt in (torch.float32, torch.bfloat16):
            ref = nv.nvfp4_gemv(w, x, out_dtype=dt)
            out = torch.full((rows, n), -7.0, dtype=dt, device="cuda")
            _noalloc(nv, w, x, out)
            torch.cuda.synchronize()
            assert torch.equal(ref.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               out.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), (n, k, rows, dt)


def test_noalloc_through_the_binding(nv):
    w, x = _case(nv, 300, 4352, 5, 33)
    a = nv.nvfp4_gemv(w, x, out_dtype=torch.float32)
    b = nv.nvfp4_gemv_noalloc(w, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
