"""GPU parity of residual add + RMSNorm calls inside a projection sequence (the
blueprint page's decode step: norm::residual_add_rms_norm before the attention
projections and before the MLP, fused here into the sequence's launch).

* a decoder layer run as one sequence -- norm, qkv, o, norm, gate/up pair,
  down, several layers deep, the residual stream updated in place -- equals
  the same calls made one by one (nvfp4_residual_rmsnorm, nvfp4_gemv,
  nvfp4_gemv_dual_silu), bit for bit, for one launch per row count, for a
  launch per call (event handles), and for row counts past one kernel call;
* the first layer's norm against the oracle: residual_out bit-exact, x within
  one bf16 ulp of the fp64 value's RNE; the projection fed by it within the
  projection's bound of the oracle on the device's x.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import check

pytestmark = pytest.mark.gpu

H, NQKV, NO, NI = 512, 768, 384, 1024   # hidden, qkv out, attention width, MLP width


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_weight_only_nvfp4_amd as nv
    nv.lib()
    return nv


def _x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _ordered(b):
    b = b.astype(np.int64)
    return np.where(b >= 0x8000, -(b & 0x7FFF), b)


def _layers(nv, rng, nlayers):
    out = []
    for li in range(nlayers):
        lm = {}
        for name, (n, k) in (("qkv", (NQKV, H)), ("o", (H, NO)), ("gate", (NI, H)), ("up", (NI, H)),
                             ("down", (H, NI))):
            q = oracle.quantize(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.03))
            lm[name] = (nv.nvfp4_pack(torch.from_numpy(q[0]).cuda(), torch.from_numpy(q[1]).cuda(), float(q[2])), q)
        lm["ln1"] = workloads.bf16_bits((rng.standard_normal(H) * 0.1 + 1.0).astype(np.float32))
        lm["ln2"] = workloads.bf16_bits((rng.standard_normal(H) * 0.1).astype(np.float32))   # Gemma offset
        out.append(lm)
    return out


class _State:
    """The buffers of a decode step: the residual stream R, the previous
    layer's down output (the first norm's delta), the attention output (o's
    input, synthetic), and the per-layer outputs."""

    def __init__(self, rows, rng):
        self.R0 = workloads.bf16_bits((rng.standard_normal((rows, H)) * 4.0).astype(np.float32))
        self.D0 = workloads.draw_x(rng, rows, H)
        self.A = _x_dev(workloads.draw_x(rng, rows, NO))
        self.R = _x_dev(self.R0)
        self.down = _x_dev(self.D0)
        self.xn = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
        self.qkv = torch.empty((rows, NQKV), dtype=torch.bfloat16, device="cuda")
        self.o = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
        self.h = torch.empty((rows, NI), dtype=torch.bfloat16, device="cuda")

    def outputs(self):
        return [t.clone() for t in (self.R, self.down, self.xn, self.qkv, self.o, self.h)]


def _sequence_calls(nv, layers, st, eps):
    calls = []
    for lm in layers:
        w1, w2 = _x_dev(lm["ln1"]), _x_dev(lm["ln2"])
        lm["_w"] = (w1, w2)
        calls += [nv.Norm(st.R, st.down, w1, st.xn, eps=eps),
                  (lm["qkv"][0], None, st.xn, st.qkv),
                  (lm["o"][0], None, st.A, st.o),
                  nv.Norm(st.R, st.o, w2, st.xn, eps=eps, gemma_offset=True),
                  (lm["gate"][0], lm["up"][0], st.xn, st.h),
                  (lm["down"][0], None, st.h, st.down)]
    return calls


def _one_by_one(nv, layers, st, eps, ws):
    for lm in layers:
        w1, w2 = lm["_w"]
        nv.nvfp4_residual_rmsnorm(st.R, st.down, w1, eps=eps, residual_out=st.R, x=st.xn)
        nv.nvfp4_gemv(lm["qkv"][0], st.xn, out=st.qkv, workspace=ws)
        nv.nvfp4_gemv(lm["o"][0], st.A, out=st.o, workspace=ws)
        nv.nvfp4_residual_rmsnorm(st.R, st.o, w2, eps=eps, gemma_offset=True, residual_out=st.R, x=st.xn)
        nv.nvfp4_gemv_dual_silu(lm["gate"][0], lm["up"][0], st.xn, out=st.h, workspace=ws)
        nv.nvfp4_gemv(lm["down"][0], st.h, out=st.down, workspace=ws)


@pytest.mark.parametrize("rows", [1, 2, 5, 8, 16, 24])
def test_decoder_layers_with_norms_match_separate_calls(nv, rows):
    rng = np.random.default_rng(40 + rows)
    layers = _layers(nv, rng, 3)
    eps = 1e-6
    st = _State(rows, rng)
    print("sequence with norms: rows=%d, %d calls" % (rows, 6 * len(layers)), flush=True)
    seq = nv.Sequence(_sequence_calls(nv, layers, st, eps))
    assert seq.n == 18
    ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    seq.launch(ws)
    torch.cuda.synchronize()
    fused = st.outputs()
    assert nv.wait_flag(ws) == 0
    assert nv.counters_clear(ws), "counters not returned to zero"
    # a launch per call (event handles) from the same start
    st.R.copy_(_x_dev(st.R0))
    st.down.copy_(_x_dev(st.D0))
    seq.launch(ws, events=[None] * (2 * seq.n))
    torch.cuda.synchronize()
    per_call = st.outputs()
    # one by one
    st.R.copy_(_x_dev(st.R0))
    st.down.copy_(_x_dev(st.D0))
    _one_by_one(nv, layers, st, eps, ws)
    torch.cuda.synchronize()
    alone = st.outputs()
    names = ("residual", "down", "x", "qkv", "o", "gate/up")
    for name, a, b, c in zip(names, fused, per_call, alone):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16)), (rows, name, "fused")
        assert torch.equal(b.view(torch.int16), c.view(torch.int16)), (rows, name, "per call")
    assert nv.counters_clear(ws), "counters not returned to zero"


@pytest.mark.parametrize("rows", [1, 8])
def test_norm_in_sequence_against_oracle(nv, rows):
    """One layer: the first norm's outputs against the oracle; qkv, fed by
    the norm's x inside the launch, against the oracle on that x."""
    rng = np.random.default_rng(90 + rows)
    layers = _layers(nv, rng, 1)
    eps = 1e-5
    st = _State(rows, rng)
    seq = nv.Sequence(_sequence_calls(nv, layers, st, eps)[:2])
    ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    seq.launch(ws)
    torch.cuda.synchronize()
    ro_ref, x_ref, _ = oracle.residual_rmsnorm(st.R0, st.D0, layers[0]["ln1"], eps)
    assert np.array_equal(_bits(st.R), ro_ref)
    d = np.abs(_ordered(_bits(st.xn)) - _ordered(x_ref))
    assert d.max() <= 1, int(d.max())
    ref, absd, ref16 = oracle.gemv(*layers[0]["qkv"][1], _bits(st.xn))
    check.check_gemv(st.qkv.float().cpu().numpy(), _bits(st.qkv), ref, absd, ref16,
                     label="norm+qkv sequence r%d" % rows)


def test_norm_only_sequence_and_out_of_place(nv):
    """A sequence of norm calls alone (no projection in the launch), with
    residual_out apart from the residual, equals nvfp4_residual_rmsnorm."""
    rng = np.random.default_rng(7)
    rows, k = 3, 2064
    r = workloads.bf16_bits((rng.standard_normal((rows, k)) * 2.0).astype(np.float32))
    h1 = workloads.draw_x(rng, rows, k)
    h2 = workloads.draw_x(rng, rows, k)
    w = workloads.bf16_bits(rng.standard_normal(k).astype(np.float32))
    R, D1, D2, W = _x_dev(r), _x_dev(h1), _x_dev(h2), _x_dev(w)
    R1 = torch.empty_like(R)
    R2 = torch.empty_like(R)
    X1 = torch.empty_like(R)
    X2 = torch.empty_like(R)
    seq = nv.Sequence([nv.Norm(R, D1, W, X1, residual_out=R1), nv.Norm(R1, D2, W, X2, residual_out=R2)])
    ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    seq.launch(ws)
    torch.cuda.synchronize()
    a1, b1 = nv.nvfp4_residual_rmsnorm(R, D1, W)
    a2, b2 = nv.nvfp4_residual_rmsnorm(a1, D2, W)
    torch.cuda.synchronize()
    for u, v in ((R1, a1), (X1, b1), (R2, a2), (X2, b2)):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
    assert np.array_equal(_bits(R), r), "the residual was written"
