"""HIP graph capture of the library's calls (the pages drive a whole decode
step as one captured graph: kern README, "Layout", decode programs): a
projection, a gate/up pair and a whole sequence (one cooperative launch per
row count, with fused norm calls) are captured once with torch.cuda.graph and
replayed several times, with eager work between the replays that changes
their inputs; every replay equals the eager calls on the same inputs, bit for
bit.  The library enqueues kernels only (no memset, copy or allocation), so a
capture holds nothing but kernel nodes."""
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


def _x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _pack(nv, rng, n, k):
    q = oracle.quantize(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
    return nv.nvfp4_pack(torch.from_numpy(q[0]).cuda(), torch.from_numpy(q[1]).cuda(), float(q[2]))


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("rows", [1, 8])
def test_graph_replays_of_single_calls(nv, rows):
    rng = np.random.default_rng(300 + rows)
    w = _pack(nv, rng, 5120, 17408)    # split-K: the counters and partial sums of the workspace
    g, u = _pack(nv, rng, 2048, 5120), _pack(nv, rng, 2048, 5120)
    xd = _x_dev(workloads.draw_x(rng, rows, 17408))
    xg = _x_dev(workloads.draw_x(rng, rows, 5120))
    need = max(nv.nvfp4_workspace_bytes(5120, 17408, rows), nv.nvfp4_workspace_bytes(2048, 5120, rows, True))
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((rows, 5120), dtype=torch.float32, device="cuda")
    o = torch.empty((rows, 2048), dtype=torch.bfloat16, device="cuda")
    # eager once (no first-call set-up inside the capture)
    nv.nvfp4_gemv(w, xd, out_dtype=torch.float32, out=y, workspace=ws)
    nv.nvfp4_gemv_dual_silu(g, u, xg, out=o, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.nvfp4_gemv(w, xd, out_dtype=torch.float32, out=y, workspace=ws)
        nv.nvfp4_gemv_dual_silu(g, u, xg, out=o, workspace=ws)
    for rep in range(4):
        print("graph replay %d, rows=%d" % (rep, rows), flush=True)
        xd.copy_(_x_dev(workloads.draw_x(rng, rows, 17408)))
        xg.copy_(_x_dev(workloads.draw_x(rng, rows, 5120)))
        y.zero_()
        o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ye = nv.nvfp4_gemv(w, xd, out_dtype=torch.float32, workspace=ws)
        oe = nv.nvfp4_gemv_dual_silu(g, u, xg, workspace=ws)
        torch.cuda.synchronize()
        assert _same(y, ye) and _same(o, oe), rep
    assert nv.counters_clear(ws), "counters not returned to zero"


@pytest.mark.parametrize("rows", [1, 8])
def test_graph_replays_of_a_sequence(nv, rows):
    """Two small decoder layers with norms (12 calls, one cooperative launch)."""
    rng = np.random.default_rng(400 + rows)
    H, NQ, NI = 512, 768, 1024
    mats = [{"qkv": _pack(nv, rng, NQ, H), "o": _pack(nv, rng, H, NQ), "gate": _pack(nv, rng, NI, H),
             "up": _pack(nv, rng, NI, H), "down": _pack(nv, rng, H, NI)} for _ in range(2)]
    lns = [_x_dev(workloads.bf16_bits((rng.standard_normal(H) * 0.1).astype(np.float32))) for _ in range(4)]
    R = _x_dev(workloads.draw_x(rng, rows, H))
    down = torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda")
    xn = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    qkv = torch.empty((rows, NQ), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((rows, NI), dtype=torch.bfloat16, device="cuda")
    calls = []
    for li, m in enumerate(mats):
        calls += [nv.Norm(R, down, lns[2 * li], xn, gemma_offset=True), (m["qkv"], None, xn, qkv),
                  (m["o"], None, qkv, o), nv.Norm(R, o, lns[2 * li + 1], xn, gemma_offset=True),
                  (m["gate"], m["up"], xn, h), (m["down"], None, h, down)]
    seq = nv.Sequence(calls)
    ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    outs = (R, down, xn, qkv, o, h)
    r0 = R.clone()
    seq.launch(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        seq.launch(ws)
    for rep in range(4):
        print("sequence graph replay %d, rows=%d" % (rep, rows), flush=True)
        start = _x_dev(workloads.draw_x(rng, rows, H))
        R.copy_(start)
        down.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        R.copy_(start)
        down.zero_()
        seq.launch(ws)
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert _same(a, b), rep
        assert not torch.equal(R, start)
    assert nv.wait_flag(ws) == 0
    assert nv.counters_clear(ws), "counters not returned to zero"
    del r0
