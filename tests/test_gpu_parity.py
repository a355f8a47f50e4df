"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* pack/unpack: byte-exact; the packed buffer equals the layout written out
  independently here in numpy.
* dequant: bit-exact (including the sign of zero) over every finite E4M3 scale
  byte and every E2M1 code.
* projection / gate-up pair: fp32 within 1e-3 * sum|w*x| of the fp64 oracle,
  bf16 = RNE of the device fp32 and within one ulp of the oracle's bf16
  (oracle.check); exact equality on "exact-arithmetic" inputs where every
  partial sum is representable in fp32, so any dropped, duplicated or misplaced
  term shows; run-to-run bitwise determinism.
* device quantizer: codes, scales and s_g bit-identical to the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import check

ALL_ROWS = range(1, 17)   # every row count one kernel call takes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_weight_only_nvfp4_amd as nv
    nv.lib()
    return nv


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _pack(nv, q):
    return nv.nvfp4_pack(_dev(q[0]), _dev(q[1]), float(q[2]))


def _run_gemv(nv, w, xb):
    x = _x_dev(xb)
    y32 = nv.nvfp4_gemv(w, x, out_dtype=torch.float32)
    y16 = nv.nvfp4_gemv(w, x, out_dtype=torch.bfloat16)
    y32b = nv.nvfp4_gemv(w, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = y32.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), y32b.cpu().numpy().view(np.uint32)), "not deterministic"
    return a, _bits(y16)


def _run_dual(nv, gw, uw, xb):
    x = _x_dev(xb)
    o32 = nv.nvfp4_gemv_dual_silu(gw, uw, x, out_dtype=torch.float32)
    o16 = nv.nvfp4_gemv_dual_silu(gw, uw, x, out_dtype=torch.bfloat16)
    o32b = nv.nvfp4_gemv_dual_silu(gw, uw, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = o32.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), o32b.cpu().numpy().view(np.uint32)), "not deterministic"
    return a, _bits(o16)


# ---- layout -----------------------------------------------------------------

def _layout_numpy(codes, scales, sg, n, k):
    """The packed layout (version 3), written out from its definition: per
    super-tile, 8 code chunks then one scale chunk of 64 16-byte entries each
    (entry l of a chunk: lane l = 16 q + j).  Code chunk c, entry l, dword d:
    canonical code bytes of feature 16 (c // 2) + j for k = 32 (4 (c % 2) + d)
    + 8 q .. + 7; scale entry l, byte 8 b + t: scale of feature
    16 (2 (q // 2) + b) + j, group 2 t + (q % 2)."""
    S, T = -(-n // 64), -(-k // 256)
    out = np.zeros(256 + S * T * 9216, np.uint8)
    out[0:4] = np.frombuffer(np.float32(sg).tobytes(), np.uint8)
    out[4:8] = np.frombuffer(np.uint32(0x34465056).tobytes(), np.uint8)
    out[8:12] = np.frombuffer(np.uint32(3).tobytes(), np.uint8)
    out[16:24] = np.frombuffer(np.int64(n).tobytes(), np.uint8)
    out[24:32] = np.frombuffer(np.int64(k).tobytes(), np.uint8)
    cpad = np.zeros((S * 64, T * 128), np.uint8)
    cpad[:n, : k // 2] = codes
    spad = np.zeros((S * 64, T * 16), np.uint8)
    spad[:n, : k // 16] = scales
    for s in range(S):
        for u in range(T):
            base = 256 + (s * T + u) * 9216
            for c in range(8):
                for q in range(4):
                    for j in range(16):
                        e = base + 1024 * c + 16 * (16 * q + j)
                        f = 64 * s + 16 * (c // 2) + j
                        for d in range(4):
                            kk = 256 * u + 32 * (4 * (c % 2) + d) + 8 * q
                            out[e + 4 * d: e + 4 * d + 4] = cpad[f, kk // 2: kk // 2 + 4]
            for q in range(4):
                for j in range(16):
                    e = base + 8192 + 16 * (16 * q + j)
                    for b in range(2):
                        for t in range(8):
                            f = 64 * s + 16 * (2 * (q // 2) + b) + j
                            out[e + 8 * b + t] = spad[f, 16 * u + 2 * t + q % 2]
    return out


@pytest.mark.parametrize("n,k", [(1, 16), (64, 256), (65, 272), (200, 784), (130, 1040)])
def test_pack_layout_and_roundtrip(nv, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (n, k // 16), dtype=np.uint8)
    w = nv.nvfp4_pack(_dev(codes), _dev(scales), 0.375)
    torch.cuda.synchronize()
    assert np.array_equal(w.data.cpu().numpy(), _layout_numpy(codes, scales, 0.375, n, k))
    c2, s2, g2 = nv.nvfp4_unpack(w)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy(), scales)
    assert g2.item() == 0.375
    assert w.global_scale() == 0.375


# ---- dequant ------------------------------------------------------------------

@pytest.mark.parametrize("sg", [1.0, 0.0123, 2.0 ** -20])
def test_dequant_exhaustive_codes_and_scales(nv, sg):
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)   # 254 bytes
    n, k = finite.size, 32
    scales = np.stack([finite, finite], axis=1)
    up = np.arange(16, dtype=np.uint8)
    down = up[::-1]
    row = np.concatenate([up[0::2] | (up[1::2] << 4), down[0::2] | (down[1::2] << 4)]).astype(np.uint8)
    codes = np.tile(row, (n, 1))
    w = nv.nvfp4_pack(_dev(codes), _dev(scales), sg)
    D = nv.nvfp4_dequant(w)
    torch.cuda.synchronize()
    got = D.cpu().numpy()
    ref = oracle.dequant(codes, scales, np.float32(sg))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_random_ragged(nv):
    c = workloads.case(200, 784, 1, seed=31)
    q = oracle.quantize(c["W"])
    D = nv.nvfp4_dequant(_pack(nv, q))
    torch.cuda.synchronize()
    ref = oracle.dequant(*q)
    assert np.array_equal(D.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ---- exact-arithmetic projections ---------------------------------------------

def _exact_case(rng, n, k, rows):
    """codes random; scales in {0.5, 1, 2}; s_g = 1; x in {0, +-0.5, +-1}: every
    product is a multiple of 2^-3 and |partial sums| < 2^17, so every fp32
    partial sum in any order is exact."""
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), size=(n, k // 16))
    xv = rng.choice(np.array([-1.0, -0.5, 0.0, 0.5, 1.0], np.float32), size=(rows, k))
    return codes, scales, np.float32(1.0), workloads.bf16_bits(xv)


@pytest.mark.parametrize("n,k", [(1, 16), (64, 256), (200, 784), (130, 4112), (300, 4352)])
def test_gemv_exact_arithmetic_all_rows(nv, n, k):
    assert k * 6 * 2 < 2 ** 17
    rng = np.random.default_rng(n + k)
    for rows in ALL_ROWS:
        codes, scales, sg, xb = _exact_case(rng, n, k, rows)
        w = nv.nvfp4_pack(_dev(codes), _dev(scales), float(sg))
        y32, y16 = _run_gemv(nv, w, xb)
        ref, _, ref16 = oracle.gemv(codes, scales, sg, xb)
        assert np.array_equal(y32.astype(np.float64), ref), (n, k, rows)
        assert np.array_equal(y16, ref16), (n, k, rows)


@pytest.mark.parametrize("n,k", [(64, 256), (200, 784), (130, 2064)])
def test_dual_exact_arithmetic(nv, n, k):
    """gate rows give g = 192 exactly (silu(192) = 192 in fp32 and fp64), so
    o = 192 * u must match the oracle exactly."""
    rng = np.random.default_rng(7 * n + k)
    for rows in (1, 3, 8, 13, 16):
        ucodes, uscales, sg, xb = _exact_case(rng, n, k, rows)
        xv = ((xb.astype(np.uint32) << 16).view(np.float32)).copy()
        xv[:, :16] = 1.0
        xb = workloads.bf16_bits(xv)
        gcodes = np.zeros((n, k // 2), np.uint8)
        gcodes[:, :8] = 0x77                          # sixteen +6 codes in group 0
        gscales = np.zeros((n, k // 16), np.uint8)
        gscales[:, 0] = 0x40                          # scale 2: 16 * 6 * 2 * 1 = 192
        gw = nv.nvfp4_pack(_dev(gcodes), _dev(gscales), 1.0)
        uw = nv.nvfp4_pack(_dev(ucodes), _dev(uscales), 1.0)
        o32, o16 = _run_dual(nv, gw, uw, xb)
        d = oracle.gemv_dual_silu((gcodes, gscales, 1.0), (ucodes, uscales, 1.0), xb)
        assert np.all(d["g"] == 192.0)
        assert np.array_equal(o32.astype(np.float64), d["o"]), rows
        assert np.array_equal(o16, d["o_bf16"])


# ---- random projections, every row count --------------------------------------

SHAPES = [(256, 512), (200, 784), (64, 2048), (130, 4112), (72, 17408)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_gemv_random_all_rows(nv, n, k):
    for rows in ALL_ROWS:
        c = workloads.case(n, k, rows, seed=100 * rows + n, outlier_frac=0.01)
        q = oracle.quantize(c["W"])
        w = _pack(nv, q)
        y32, y16 = _run_gemv(nv, w, c["x"])
        ref, absd, ref16 = oracle.gemv(*q, c["x"])
        check.check_gemv(y32, y16, ref, absd, ref16, label="gemv %dx%d rows=%d" % (n, k, rows))


@pytest.mark.parametrize("n,k", [(256, 512), (200, 784), (130, 4112)])
def test_dual_random_all_rows(nv, n, k):
    for rows in ALL_ROWS:
        c = workloads.case(n, k, rows, seed=200 * rows + n, dual=True)
        gq, uq = oracle.quantize(c["W"]), oracle.quantize(c["W_up"])
        o32, o16 = _run_dual(nv, _pack(nv, gq), _pack(nv, uq), c["x"])
        d = oracle.gemv_dual_silu(gq, uq, c["x"])
        check.check_dual(o32, o16, d, label="dual %dx%d rows=%d" % (n, k, rows))


@pytest.mark.parametrize("n,k", [(130, 4112), (300, 4352), (72, 17408)])
def test_rows_invariant_1_to_16(nv, n, k):
    """A row's result does not depend on how many rows share the call: every
    row count 1..16 gives every row bit-identical fp32 and bf16 outputs (one
    arithmetic for every row count; the plan, the product positions of a row
    and every summation order are independent of the row count).  Single
    projection and gate/up pair; shapes with and without split-K pieces."""
    c = workloads.case(n, k, 16, seed=n + 7 * k, dual=True)
    gq, uq = oracle.quantize(c["W"]), oracle.quantize(c["W_up"])
    gw, uw = _pack(nv, gq), _pack(nv, uq)
    y_ref, y16_ref = _run_gemv(nv, gw, c["x"])
    o_ref, o16_ref = _run_dual(nv, gw, uw, c["x"])
    for rows in range(1, 16):
        y, y16 = _run_gemv(nv, gw, c["x"][:rows])
        o, o16 = _run_dual(nv, gw, uw, c["x"][:rows])
        assert np.array_equal(y.view(np.uint32), y_ref[:rows].view(np.uint32)), (n, k, rows)
        assert np.array_equal(y16, y16_ref[:rows]), (n, k, rows)
        assert np.array_equal(o.view(np.uint32), o_ref[:rows].view(np.uint32)), (n, k, rows)
        assert np.array_equal(o16, o16_ref[:rows]), (n, k, rows)


# ---- more than 16 rows: row chunks ----------------------------------------------

MANY_ROWS = (17, 24, 32, 33, 64, 128)


def _oracle_rows(fn, *args, x):
    """The oracle takes up to 64 rows per call; every output row depends on its
    own activation row only, so larger row counts go through it in blocks."""
    parts = [fn(*args, x[r:r + 64]) for r in range(0, x.shape[0], 64)]
    if isinstance(parts[0], dict):
        return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))


@pytest.mark.parametrize("n,k", [(130, 4112), (300, 784), (72, 17408)])
def test_gemv_random_many_rows(nv, n, k):
    """Calls of 17..128 rows (the pages' draft and multi-sequence row tiers)
    run as balanced chunks of at most 16 rows; every output against the
    oracle, with and without split-K pieces."""
    for rows in MANY_ROWS:
        c = workloads.case(n, k, rows, seed=400 * rows + n, outlier_frac=0.01)
        q = oracle.quantize(c["W"])
        y32, y16 = _run_gemv(nv, _pack(nv, q), c["x"])
        ref, absd, ref16 = _oracle_rows(oracle.gemv, *q, x=c["x"])
        check.check_gemv(y32, y16, ref, absd, ref16, label="gemv %dx%d rows=%d" % (n, k, rows))


def test_dual_random_many_rows(nv):
    for rows in (17, 32, 128):
        c = workloads.case(130, 4112, rows, seed=500 + rows, dual=True)
        gq, uq = oracle.quantize(c["W"]), oracle.quantize(c["W_up"])
        o32, o16 = _run_dual(nv, _pack(nv, gq), _pack(nv, uq), c["x"])
        d = _oracle_rows(oracle.gemv_dual_silu, gq, uq, x=c["x"])
        check.check_dual(o32, o16, d, label="dual 130x4112 rows=%d" % rows)


@pytest.mark.parametrize("n,k", [(130, 4112), (72, 17408)])
def test_rows_invariant_1_to_128(nv, n, k):
    """Every row count 1..128 (one row chunk up to 16 rows, balanced chunks
    beyond) gives every row the same bits as the 128-row call, single
    projection and gate/up pair."""
    c = workloads.case(n, k, 128, seed=n + 11 * k, dual=True)
    gq, uq = oracle.quantize(c["W"]), oracle.quantize(c["W_up"])
    gw, uw = _pack(nv, gq), _pack(nv, uq)
    y_ref, y16_ref = _run_gemv(nv, gw, c["x"])
    o_ref, o16_ref = _run_dual(nv, gw, uw, c["x"])
    for rows in range(1, 128):
        y, y16 = _run_gemv(nv, gw, c["x"][:rows])
        o, o16 = _run_dual(nv, gw, uw, c["x"][:rows])
        assert np.array_equal(y.view(np.uint32), y_ref[:rows].view(np.uint32)), (n, k, rows)
        assert np.array_equal(y16, y16_ref[:rows]), (n, k, rows)
        assert np.array_equal(o.view(np.uint32), o_ref[:rows].view(np.uint32)), (n, k, rows)
        assert np.array_equal(o16, o16_ref[:rows]), (n, k, rows)


def test_sequence_with_many_row_calls(nv):
    """A call list whose calls have 40 rows (three row chunks each), the
    second reading the first's output as its activations, equals the calls
    made one by one, bit for bit, with and without per-call events; the
    workspace's counters are back at zero afterwards."""
    dev = torch.device("cuda")
    c1 = workloads.case(320, 784, 40, seed=61)
    c2 = workloads.case(130, 320, 1, seed=62)
    w1 = _pack(nv, oracle.quantize(c1["W"]))
    w2 = _pack(nv, oracle.quantize(c2["W"]))
    x1 = _x_dev(c1["x"])
    y1 = torch.empty((40, 320), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((40, 130), dtype=torch.float32, device=dev)
    seq = nv.Sequence([(w1, None, x1, y1), (w2, None, y1, y2)])
    ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device=dev)
    for events in (None, [None] * 4):
        y1.zero_()
        y2.zero_()
        seq.launch(ws, events=events)
        torch.cuda.synchronize()
        assert nv.counters_clear(ws), "counters not returned to zero"
        a1 = nv.nvfp4_gemv(w1, x1)
        a2 = nv.nvfp4_gemv(w2, a1, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(a1.view(torch.int16), y1.view(torch.int16))
        assert torch.equal(a2.view(torch.int32), y2.view(torch.int32))


def _wide_x(rng, rows, k, binades):
    """bf16 activations sign * 2^u, u uniform over [-binades, binades]: groups
    and super-tiles whose values span up to 2 * binades binades."""
    u = rng.uniform(-binades, binades, size=(rows, k))
    xv = (np.where(rng.random((rows, k)) < 0.5, -1.0, 1.0) * np.exp2(u)).astype(np.float32)
    return workloads.bf16_bits(xv)


@pytest.mark.parametrize("n,k", [(200, 784), (130, 4112)])
@pytest.mark.parametrize("binades", [16, 60])
def test_gemv_wide_range_activations_all_rows(nv, n, k, binades):
    """Activations sign * 2^u, u uniform in [-binades, binades], inside every
    group: the activations enter the products as stored, so R14/R15 hold at
    any spread (60 binades: products from about 2^-70 to 2^63, all inside the
    fp32 range)."""
    rng = np.random.default_rng(31 * n + k + binades)
    for rows in ALL_ROWS:
        c = workloads.case(n, k, rows, seed=300 * rows + n, outlier_frac=0.01)
        q = oracle.quantize(c["W"])
        xb = _wide_x(rng, rows, k, binades)
        y32, y16 = _run_gemv(nv, _pack(nv, q), xb)
        ref, absd, ref16 = oracle.gemv(*q, xb)
        check.check_gemv(y32, y16, ref, absd, ref16, label="wide(%d) gemv %dx%d rows=%d" % (binades, n, k, rows))


def _big_on_zero_code_case(k, rows, g0):
    """One group g0 of every row: x = 2^16 on a weight whose code is 0, and
    2^-8 on 15 weights of code +-1 (scale 1, s_g 1); every other k has x = 0.
    The exact result is 15 * 2^-8 * (+-1 sums), which a path that scales each
    group's activations by its largest loses entirely."""
    n = 64
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    rng = np.random.default_rng(k + rows + g0)
    signs = rng.integers(0, 2, (n, 15))
    nib = np.concatenate([np.zeros((n, 1), np.uint8), np.where(signs == 1, 0xA, 0x2).astype(np.uint8)], axis=1)
    codes[:, 8 * g0: 8 * g0 + 8] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    scales[:, g0] = 0x38                                # E4M3 1.0
    xv = np.zeros((rows, k), np.float32)
    xv[:, 16 * g0] = 2.0 ** 16
    xv[:, 16 * g0 + 1: 16 * g0 + 16] = 2.0 ** -8
    return codes, scales, np.float32(1.0), workloads.bf16_bits(xv)


@pytest.mark.parametrize("k,g0", [(16, 0), (5120, 0), (5120, 137), (5120, 319)])
def test_gemv_large_activation_on_zero_code(nv, k, g0):
    """The wide-range case that an activation split per group loses: checked
    exactly (every partial sum is a multiple of 2^-8 below 2^17) at every row
    count, as a lone group and inside k = 5120."""
    for rows in ALL_ROWS:
        codes, scales, sg, xb = _big_on_zero_code_case(k, rows, g0)
        w = nv.nvfp4_pack(_dev(codes), _dev(scales), float(sg))
        y32, y16 = _run_gemv(nv, w, xb)
        ref, absd, ref16 = oracle.gemv(codes, scales, sg, xb)
        assert np.any(ref != 0)
        assert np.array_equal(y32.astype(np.float64), ref), (k, g0, rows)
        assert np.array_equal(y16, ref16), (k, g0, rows)


def test_gemv_zero_inputs(nv):
    c = workloads.case(130, 784, 3, seed=5)
    q = oracle.quantize(c["W"])
    w = _pack(nv, q)
    y32, y16 = _run_gemv(nv, w, np.zeros_like(c["x"]))
    assert not y32.any() and not np.signbit(y32).any() and not y16.any()
    zq = oracle.quantize(np.zeros((130, 784), np.float32))
    y32, _ = _run_gemv(nv, _pack(nv, zq), c["x"])
    assert not y32.any()


def test_workspace_reuse_and_mixed_calls(nv):
    """Counters are left at zero: interleaved calls of different shapes, few and
    many strips, that share one workspace stay correct."""
    cases = [workloads.case(300, 4352, r, seed=40 + r) for r in (1, 8, 3, 16, 11)]
    cases.append(workloads.case(4480, 2048, 2, seed=44))
    qs = [oracle.quantize(c["W"]) for c in cases]
    need = max(nv.nvfp4_workspace_bytes(c["n"], c["k"], c["rows"]) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        for c, q in zip(cases, qs):
            w = _pack(nv, q)
            y = nv.nvfp4_gemv(w, _x_dev(c["x"]), out_dtype=torch.float32, workspace=ws)
            torch.cuda.synchronize()
            ref, absd, ref16 = oracle.gemv(*q, c["x"])
            check.check_gemv(y.cpu().numpy(), None, ref, absd, ref16)
    torch.cuda.synchronize()
    assert not ws[: 4 * 70].any().item()     # the strip counters are back at zero


# ---- device quantizer ------------------------------------------------------------

def _quantize_dev(nv, W):
    wt = _dev(W)
    ws = torch.zeros(nv.nvfp4_quantize_workspace_bytes(*W.shape), dtype=torch.uint8, device="cuda")
    pw = nv.nvfp4_quantize(wt, workspace=ws)
    c, s, g = nv.nvfp4_unpack(pw)
    torch.cuda.synchronize()
    return pw, c.cpu().numpy(), s.cpu().numpy(), np.float32(g.item()), int(ws[:4].view(torch.int32).item())


def _assert_same_quant(nv, W):
    pw, c, s, g, status = _quantize_dev(nv, W)
    assert status == 0
    rc, rs, rg = oracle.quantize(W)
    assert g == rg
    assert np.array_equal(s, rs), int(np.sum(s != rs))
    assert np.array_equal(c, rc), int(np.sum(c != rc))
    return pw


@pytest.mark.parametrize("n,k,outl", [(256, 512, 0.0), (200, 784, 0.01), (65, 4112, 0.2), (1, 16, 0.0)])
def test_quantize_device_bit_exact_random(nv, n, k, outl):
    c = workloads.case(n, k, 1, seed=n + k, outlier_frac=outl)
    _assert_same_quant(nv, c["W"])
    _assert_same_quant(nv, -c["W"] * np.float32(3.7))


def test_quantize_device_special_cases(nv):
    from test_oracle_quantizer import load_kv
    g = load_kv("worked_row.txt")
    _assert_same_quant(nv, np.array([[float(v) for v in g["W"]]], np.float32))
    _assert_same_quant(nv, np.zeros((3, 32), np.float32))
    W = np.zeros((2, 48), np.float32)
    W[0, 0] = 2688.0
    W[0, 16] = 6.0 * 2.0 ** -9 * 3
    W[0, 32] = 6.0 * 2.0 ** -9 * 0.4
    W[1, 16:32] = -1e-9
    _assert_same_quant(nv, W)
    # exact E2M1 ties everywhere: W/S lands on every midpoint
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    row = np.concatenate([mids, -mids])
    W = np.tile(row * np.float32(1.75), (64, 4)).astype(np.float32)
    W[:, 7::16] = np.float32(10.5)         # 6 * S with S = 1.75 -> scale 448 per group
    _assert_same_quant(nv, W)


def test_quantize_device_flags_non_finite(nv):
    W = np.ones((64, 256), np.float32)
    W[5, 7] = np.inf
    _, _, _, _, status = _quantize_dev(nv, W)
    assert status != 0


# ---- the four single-call workloads at full size ---------------------------------

def _full_gemv(nv, c):
    pw = _assert_same_quant(nv, c["W"])
    q = oracle.quantize(c["W"])
    y32, y16 = _run_gemv(nv, pw, c["x"])
    ref, absd, ref16 = oracle.gemv(*q, c["x"])
    return check.check_gemv(y32, y16, ref, absd, ref16, label="full %dx%d rows=%d" % (c["n"], c["k"], c["rows"]))


def test_full_tiny(nv):
    st = _full_gemv(nv, workloads.tiny())
    assert st["max_err_over_absdot"] < 1e-5


def test_full_qkv_rows1(nv):
    st = _full_gemv(nv, workloads.qkv_rows1())
    assert st["max_err_over_absdot"] < 1e-5


def test_full_down_rows8_outliers(nv):
    st = _full_gemv(nv, workloads.down_rows8())
    assert st["max_err_over_absdot"] < 1e-5


def test_full_gate_up_rows1(nv):
    c = workloads.gate_up_rows1()
    gw = _assert_same_quant(nv, c["W"])
    uw = _assert_same_quant(nv, c["W_up"])
    gq, uq = oracle.quantize(c["W"]), oracle.quantize(c["W_up"])
    o32, o16 = _run_dual(nv, gw, uw, c["x"])
    d = oracle.gemv_dual_silu(gq, uq, c["x"])
    st = check.check_dual(o32, o16, d, label="full gate/up")
    assert st["max_err_over_bound"] < 0.05


# ---- strips left over past whole strips per workgroup ------------------------------

@pytest.mark.parametrize("n,k,dual", [(16448, 5120, False), (16448, 512, True), (19200, 1024, False),
                                      (32896, 256, True)])
def test_leftover_strips(nv, n, k, dual):
    """More strips of 64 features than workgroups: each workgroup owns whole
    strips and the strips left over are cut into a few pieces on the last
    workgroups -- also where the leftover holds fewer super-tiles than there
    are workgroups (257 strips of 2 or 20 super-tiles, 514 strips of one).
    Every leftover feature and 128 others are checked against the oracle at
    rows 1 and 8, and the calls inside one sequence equal the calls made one
    by one, bit for bit."""
    rng = np.random.default_rng(n + k)
    W = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    q = oracle.quantize(W)
    w = _pack(nv, q)
    if dual:
        qu = oracle.quantize(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
        wu = _pack(nv, qu)
    owned = (n // 64 // 256) * 256 * 64
    sel = np.unique(np.concatenate([np.arange(owned, n), rng.choice(owned, 128, replace=False)]))
    for rows in (1, 8):
        print("leftover strips %dx%d dual=%d rows=%d" % (n, k, dual, rows), flush=True)
        xb = workloads.draw_x(rng, rows, k)
        if dual:
            o32, o16 = _run_dual(nv, w, wu, xb)
            d = oracle.gemv_dual_silu(q, qu, xb, sel=sel)
            check.check_dual(o32[:, sel], o16[:, sel], d, label="leftover dual %dx%d r%d" % (n, k, rows))
        else:
            o32, o16 = _run_gemv(nv, w, xb)
            ref, absd, ref16 = oracle.gemv(*q, xb, sel=sel)
            check.check_gemv(o32[:, sel], o16[:, sel], ref, absd, ref16, label="leftover %dx%d r%d" % (n, k, rows))
        x = _x_dev(xb)
        ys = [torch.empty((rows, n), dtype=torch.float32, device="cuda") for _ in range(3)]
        seq = nv.Sequence([(w, wu if dual else None, x, y) for y in ys])
        ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device="cuda")
        seq.launch(ws)
        torch.cuda.synchronize()
        assert nv.counters_clear(ws), "counters not returned to zero"
        for y in ys:
            assert np.array_equal(y.cpu().numpy().view(np.uint32), o32.view(np.uint32)), rows


# ---- the decode-step sweep: one layer, sampled outputs -------------------------------

def test_sweep_layer_sampled(nv):
    dev = torch.device("cuda")
    rng = np.random.default_rng(77)
    layer = 0
    mats = {}
    for pi, (name, n, k) in enumerate(workloads.LAYER_PROJECTIONS):
        Wd = workloads.draw_weights_device(n, k, workloads.sweep_seed(layer, pi), dev)
        ws = torch.empty(nv.nvfp4_quantize_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
        pw = nv.nvfp4_quantize(Wd, workspace=ws)
        W = Wd.cpu().numpy()
        q = oracle.quantize(W)
        c, s, g = nv.nvfp4_unpack(pw)
        torch.cuda.synchronize()
        assert np.float32(g.item()) == q[2]
        assert np.array_equal(c.cpu().numpy(), q[0]) and np.array_equal(s.cpu().numpy(), q[1])
        mats[name] = (pw, q)
        del Wd
    for rows in workloads.SWEEP_ROWS:
        for name, n, k in workloads.LAYER_PROJECTIONS:
            if name == "up":
                continue
            xd = workloads.draw_x_device(rows, k, 999 + rows, dev)
            xb = _bits(xd)
            sel = np.sort(rng.choice(n, 256, replace=False))
            if name == "gate":
                o = nv.nvfp4_gemv_dual_silu(mats["gate"][0], mats["up"][0], xd, out_dtype=torch.float32)
                o16 = nv.nvfp4_gemv_dual_silu(mats["gate"][0], mats["up"][0], xd)
                torch.cuda.synchronize()
                d = oracle.gemv_dual_silu(mats["gate"][1], mats["up"][1], xb, sel=sel)
                check.check_dual(o.cpu().numpy()[:, sel], _bits(o16)[:, sel], d, label="sweep gate/up r%d" % rows)
            else:
                y = nv.nvfp4_gemv(mats[name][0], xd, out_dtype=torch.float32)
                y16 = nv.nvfp4_gemv(mats[name][0], xd)
                torch.cuda.synchronize()
                ref, absd, ref16 = oracle.gemv(*mats[name][1], xb, sel=sel)
                check.check_gemv(y.cpu().numpy()[:, sel], _bits(y16)[:, sel], ref, absd, ref16,
                                 label="sweep %s r%d" % (name, rows))


# ---- sequence executor -------------------------------------------------------------

def test_sequence_matches_individual_calls(nv):
    """A small decode step (qkv, o, gate/up pair, down fed by the pair) for 11
    layers -- 44 calls, so two launches of the shared-launch executor -- through
    nvfp4_gemv_sequence equals the same calls made one by one, bit for bit;
    with event handles every call gets a launch of its own, and the events are
    recorded around the requested calls.  Afterwards the workspace's counters
    are back to zero."""
    shapes = {"qkv": (384, 512), "o": (128, 768), "gate": (512, 512), "up": (512, 512), "down": (128, 512)}
    rng = np.random.default_rng(3)
    layers = []
    for li in range(11):
        lm = {}
        for name, (n, k) in shapes.items():
            W = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
            lm[name] = _pack(nv, oracle.quantize(W))
        layers.append(lm)
    for rows in (1, 3, 8):
        print("sequence of 44 small calls, rows=%d" % rows, flush=True)
        x512 = _x_dev(workloads.draw_x(rng, rows, 512))
        x768 = _x_dev(workloads.draw_x(rng, rows, 768))
        outs = [torch.empty((rows, n), dtype=torch.bfloat16 if i % 2 else torch.float32, device="cuda")
                for i, n in enumerate((384, 128, 512, 128))]
        pair16 = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")   # feeds down
        calls = []
        for lm in layers:
            calls += [(lm["qkv"], None, x512, outs[0]), (lm["o"], None, x768, outs[1]),
                      (lm["gate"], lm["up"], x512, pair16), (lm["down"], None, pair16, outs[3])]
        seq = nv.Sequence(calls)
        assert seq.n == 44
        ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device="cuda")
        seq.launch(ws)
        torch.cuda.synchronize()
        fused = [o.clone() for o in (outs[0], outs[1], pair16, outs[3])]
        assert nv.counters_clear(ws), "counters not returned to zero"
        for o in (outs[0], outs[1], pair16, outs[3]):
            o.zero_()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in ev:
            e.record()
        handles = [None] * (2 * seq.n)
        handles[2 * 2], handles[2 * 2 + 1] = ev[0].cuda_event, ev[1].cuda_event
        seq.launch(ws, events=handles)
        torch.cuda.synchronize()
        timed = [o.clone() for o in (outs[0], outs[1], pair16, outs[3])]
        assert ev[0].elapsed_time(ev[1]) >= 0.0
        # one by one
        for lm in layers:
            nv.nvfp4_gemv(lm["qkv"], x512, out=outs[0], out_dtype=outs[0].dtype, workspace=ws)
            nv.nvfp4_gemv(lm["o"], x768, out=outs[1], out_dtype=outs[1].dtype, workspace=ws)
            nv.nvfp4_gemv_dual_silu(lm["gate"], lm["up"], x512, out=pair16, workspace=ws)
            nv.nvfp4_gemv(lm["down"], pair16, out=outs[3], out_dtype=outs[3].dtype, workspace=ws)
        torch.cuda.synchronize()
        for a, t, b in zip(fused, timed, (outs[0], outs[1], pair16, outs[3])):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rows
            assert torch.equal(t.view(torch.uint8), b.view(torch.uint8)), rows
        assert nv.counters_clear(ws), "counters not returned to zero"


def test_sequence_many_short_segments(nv):
    """Calls whose workgroups close several one-super-tile segments each (600
    strips of 64 features, k = 256: two owned strips per workgroup plus a
    leftover strip for some), so that at 1-4 rows, where segment ends take no
    workgroup barrier, the waves without a tile in a segment run ahead to the
    slot buffers of later segments and calls: 10 such calls -- single
    projections and a gate/up pair, independent and chained -- in one
    sequence equal the same calls made one by one, bit for bit, with the
    workspace's counters and wait flag back at zero."""
    rng = np.random.default_rng(21)
    n, k = 64 * 600, 256
    mats = [_pack(nv, oracle.quantize(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)))
            for _ in range(9)]
    chain = _pack(nv, oracle.quantize(rng.standard_normal((256, n), dtype=np.float32) * np.float32(0.02)))
    for rows in (1, 2, 4, 6):
        print("sequence of short segments, rows=%d" % rows, flush=True)
        x = _x_dev(workloads.draw_x(rng, rows, k))
        ys = [torch.empty((rows, n), dtype=torch.bfloat16 if i % 2 else torch.float32, device="cuda")
              for i in range(6)]
        h = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
        z = torch.empty((rows, 256), dtype=torch.float32, device="cuda")
        calls = [(mats[i], None, x, ys[i]) for i in range(6)]
        calls += [(mats[6], mats[7], x, h), (chain, None, h, z), (mats[8], None, x, ys[0]), (mats[0], None, x, ys[1])]
        seq = nv.Sequence(calls)
        assert seq.waits >= 2
        ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
        seq.launch(ws)
        torch.cuda.synchronize()
        fused = [t.clone() for t in ys + [h, z]]
        assert nv.wait_flag(ws) == 0
        assert nv.counters_clear(ws), "counters not returned to zero"
        for i in range(6):
            nv.nvfp4_gemv(mats[i], x, out=ys[i], out_dtype=ys[i].dtype, workspace=ws)
        nv.nvfp4_gemv_dual_silu(mats[6], mats[7], x, out=h, workspace=ws)
        nv.nvfp4_gemv(chain, h, out=z, out_dtype=torch.float32, workspace=ws)
        nv.nvfp4_gemv(mats[8], x, out=ys[0], out_dtype=ys[0].dtype, workspace=ws)
        nv.nvfp4_gemv(mats[0], x, out=ys[1], out_dtype=ys[1].dtype, workspace=ws)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(fused, ys + [h, z])):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rows, i)
        assert nv.counters_clear(ws), "counters not returned to zero"


def test_sequence_independent_calls_and_hazards(nv):
    """Calls that depend on no earlier call run without a wait, up to four at
    once in workspace regions of their own: 12 independent split-K calls (every
    region in use) equal the calls made one by one; so do a call that
    overwrites an earlier call's input (it must wait for the reader), two
    calls writing one buffer (the later one's result stays), and a chain."""
    rng = np.random.default_rng(17)
    shapes = [(200, 4096), (320, 2304), (130, 5120)]   # skinny: split-K pieces
    for rows in (1, 5, 16):
        ws_list = [_pack(nv, oracle.quantize(rng.standard_normal(shapes[i % 3], dtype=np.float32)
                                             * np.float32(0.02))) for i in range(12)]
        xs = [_x_dev(workloads.draw_x(rng, rows, shapes[i % 3][1])) for i in range(12)]
        ys = [torch.empty((rows, shapes[i % 3][0]), dtype=torch.float32, device="cuda") for i in range(12)]
        seq = nv.Sequence([(ws_list[i], None, xs[i], ys[i]) for i in range(12)])
        assert seq.waits == 2   # a wait after every run of four
        ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device="cuda")
        seq.launch(ws)
        torch.cuda.synchronize()
        assert nv.counters_clear(ws)
        for i in range(12):
            alone = nv.nvfp4_gemv(ws_list[i], xs[i], out_dtype=torch.float32, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(alone.view(torch.int32), ys[i].view(torch.int32)), (rows, i)
        # hazards: A reads xa; C overwrites xa (write after read); B and D write one buffer
        # (write after write); E reads B's... D's output (read after write)
        wA, wB, wC, wD, wE = (_pack(nv, oracle.quantize(rng.standard_normal((n, k), dtype=np.float32)
                                                         * np.float32(0.02)))
                              for n, k in ((256, 512), (384, 768), (512, 1024), (384, 512), (256, 384)))
        xa0 = workloads.draw_x(rng, rows, 512)
        xa = _x_dev(xa0)
        xb, xc = _x_dev(workloads.draw_x(rng, rows, 768)), _x_dev(workloads.draw_x(rng, rows, 1024))
        ya = torch.empty((rows, 256), dtype=torch.bfloat16, device="cuda")
        yb = torch.empty((rows, 384), dtype=torch.bfloat16, device="cuda")
        ye = torch.empty((rows, 256), dtype=torch.bfloat16, device="cuda")
        calls = [(wA, None, xa, ya), (wB, None, xb, yb), (wC, None, xc, xa), (wD, None, xa, yb),
                 (wE, None, yb, ye)]
        seq = nv.Sequence(calls)
        assert seq.waits == 3   # C (overwrites A's input), D (reads C's output), E (reads D's)
        ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device="cuda")
        seq.launch(ws)
        torch.cuda.synchronize()
        got = [t.clone() for t in (ya, yb, ye, xa)]
        xa.copy_(_x_dev(xa0))
        for w, _, x, y in calls:
            nv.nvfp4_gemv(w, x, out=y, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(got, (ya, yb, ye, xa)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), rows
        assert nv.counters_clear(ws)


def test_sequence_mixed_rows(nv):
    """Calls with different row counts in one sequence (one launch per run of
    equal row counts) equal the calls made one by one."""
    rng = np.random.default_rng(5)
    w = [_pack(nv, oracle.quantize(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)))
         for n, k in ((200, 784), (130, 2064), (640, 1024))]
    xs = {(r, k): _x_dev(workloads.draw_x(rng, r, k)) for r in (1, 2, 5) for k in (784, 2064, 1024)}
    plan = [(0, 1), (1, 1), (2, 2), (0, 2), (1, 5), (2, 5), (0, 1)]
    ks = (784, 2064, 1024)
    ns = (200, 130, 640)
    outs = [torch.empty((r, ns[i]), dtype=torch.float32, device="cuda") for i, r in plan]
    seq = nv.Sequence([(w[i], None, xs[(r, ks[i])], outs[j]) for j, (i, r) in enumerate(plan)])
    ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device="cuda")
    seq.launch(ws)
    torch.cuda.synchronize()
    for j, (i, r) in enumerate(plan):
        alone = nv.nvfp4_gemv(w[i], xs[(r, ks[i])], out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(alone.view(torch.int32), outs[j].view(torch.int32)), (j, i, r)
    assert nv.counters_clear(ws)


_RANDOM_LIST_DIMS = (256, 512, 1024, 1536)
_random_pool = {}


def _random_list_pool(nv):
    """Two packed weights per (n, k) over _RANDOM_LIST_DIMS, built once."""
    if not _random_pool:
        rng = np.random.default_rng(999)
        for n in _RANDOM_LIST_DIMS:
            for k in _RANDOM_LIST_DIMS:
                _random_pool[(n, k)] = [
                    _pack(nv, oracle.quantize(rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.05)))
                    for _ in range(2)]
    return _random_pool


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_sequence_random_call_lists(nv, seed):
    """Seeded random call lists -- single projections and gate/up pairs of
    several shapes over a pool of activation buffers, so that calls read
    earlier calls' outputs, overwrite what earlier calls read or write, or
    depend on nothing (any mix of waits, runs of up to four and workspace
    regions) -- at one row count per list: the sequence leaves every buffer
    as the same calls made one by one do, bit for bit, with the workspace's
    counters and wait flag back at zero."""
    dims = _RANDOM_LIST_DIMS
    rows = (1, 2, 4, 8)[seed]
    pool = _random_list_pool(nv)
    rng = np.random.default_rng(1000 + seed)
    start = {d: [workloads.draw_x(rng, rows, d) for _ in range(3)] for d in dims}
    plan = []
    for _ in range(28):
        k, n = int(rng.choice(dims)), int(rng.choice(dims))
        i = int(rng.integers(3))
        j = int(rng.integers(3))
        if k == n and i == j:
            j = (j + 1) % 3
        pair = bool(rng.random() < 0.25)
        plan.append((n, k, i, j, pair, int(rng.integers(2))))

    def fresh():
        return {d: [_x_dev(b) for b in start[d]] for d in dims}

    def calls_of(bufs):
        out = []
        for n, k, i, j, pair, wi in plan:
            w = pool[(n, k)][wi]
            up = pool[(n, k)][1 - wi] if pair else None
            out.append((w, up, bufs[k][i], bufs[n][j]))
        return out

    print("random call list seed=%d rows=%d" % (seed, rows), flush=True)
    bufs = fresh()
    seq = nv.Sequence(calls_of(bufs))
    ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    seq.launch(ws)
    torch.cuda.synchronize()
    assert nv.wait_flag(ws) == 0
    assert nv.counters_clear(ws), "counters not returned to zero"
    ref = fresh()
    for w, up, x, y in calls_of(ref):
        if up is None:
            nv.nvfp4_gemv(w, x, out=y, workspace=ws)
        else:
            nv.nvfp4_gemv_dual_silu(w, up, x, out=y, workspace=ws)
    torch.cuda.synchronize()
    for d in dims:
        for i in range(3):
            assert torch.equal(bufs[d][i].view(torch.int16), ref[d][i].view(torch.int16)), (seed, d, i, seq.waits)
    assert nv.counters_clear(ws), "counters not returned to zero"


_LEFTOVER_LIST_SHAPES = ((16448, 512), (16448, 1536), (512, 16448), (1536, 16448), (512, 512), (1536, 512),
                         (512, 1536))
_leftover_pool = {}


@pytest.mark.parametrize("seed", [0, 1])
def test_sequence_random_call_lists_leftover_strips(nv, seed):
    """Random call lists as above over shapes with strips left over past one
    per workgroup (257 strips of 2 and 6 super-tiles: 2 and 4 pieces on the
    last workgroups), skinny shapes with k = 16448, and small ones, singles
    and pairs, reading and overwriting each other's buffers: the sequence
    equals the same calls made one by one, bit for bit, at 1 and 8 rows."""
    rows = (1, 8)[seed]
    if not _leftover_pool:
        r0 = np.random.default_rng(4242)
        for n, k in _LEFTOVER_LIST_SHAPES:
            _leftover_pool[(n, k)] = [
                _pack(nv, oracle.quantize(r0.standard_normal((n, k), dtype=np.float32) * np.float32(0.05)))
                for _ in range(2)]
    dims = (512, 1536, 16448)
    rng = np.random.default_rng(2000 + seed)
    start = {d: [workloads.draw_x(rng, rows, d) for _ in range(3)] for d in dims}
    plan = []
    for _ in range(24):
        n, k = _LEFTOVER_LIST_SHAPES[int(rng.integers(len(_LEFTOVER_LIST_SHAPES)))]
        i, j = int(rng.integers(3)), int(rng.integers(3))
        if k == n and i == j:
            j = (j + 1) % 3
        plan.append((n, k, i, j, bool(rng.random() < 0.3), int(rng.integers(2))))

    def fresh():
        return {d: [_x_dev(b) for b in start[d]] for d in dims}

    def calls_of(bufs):
        return [(_leftover_pool[(n, k)][wi], _leftover_pool[(n, k)][1 - wi] if pair else None, bufs[k][i], bufs[n][j])
                for n, k, i, j, pair, wi in plan]

    print("random leftover-strip call list seed=%d rows=%d" % (seed, rows), flush=True)
    bufs = fresh()
    seq = nv.Sequence(calls_of(bufs))
    ws = torch.zeros(max(seq.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    seq.launch(ws)
    torch.cuda.synchronize()
    assert nv.wait_flag(ws) == 0
    assert nv.counters_clear(ws), "counters not returned to zero"
    ref = fresh()
    for w, up, x, y in calls_of(ref):
        if up is None:
            nv.nvfp4_gemv(w, x, out=y, workspace=ws)
        else:
            nv.nvfp4_gemv_dual_silu(w, up, x, out=y, workspace=ws)
    torch.cuda.synchronize()
    for d in dims:
        for i in range(3):
            assert torch.equal(bufs[d][i].view(torch.int16), ref[d][i].view(torch.int16)), (seed, d, i, seq.waits)
    assert nv.counters_clear(ws), "counters not returned to zero"


def test_sequence_full_size_decode_step(nv):
    """Two full-size decode-step layers through one sequence (a shared launch
    per row count, the weight pipeline running across calls): the last layer's
    qkv, o and gate/up outputs match the oracle on sampled features; its down
    projection, fed by the pair's output inside the same launch, equals a
    launch of its own on that output bit for bit; the counters are back to zero."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(78)
    layers = []
    for layer in range(2):
        lm = {}
        for pi, (name, n, k) in enumerate(workloads.LAYER_PROJECTIONS):
            Wd = workloads.draw_weights_device(n, k, workloads.sweep_seed(layer, pi), dev)
            qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
            pw = nv.nvfp4_quantize(Wd, workspace=qws)
            lm[name] = (pw, oracle.quantize(Wd.cpu().numpy()) if layer == 1 else None)
            del Wd
        layers.append(lm)
    last = layers[1]
    for rows in (1, 8):
        print("full-size sequence, rows=%d" % rows, flush=True)
        xa = workloads.draw_x_device(rows, 5120, 500 + rows, dev)
        xo = workloads.draw_x_device(rows, 6144, 600 + rows, dev)
        y_qkv = torch.empty((rows, 12288), dtype=torch.float32, device=dev)
        y_o = torch.empty((rows, 5120), dtype=torch.float32, device=dev)
        o32 = torch.empty((rows, 17408), dtype=torch.float32, device=dev)
        o_gu = torch.empty((rows, 17408), dtype=torch.bfloat16, device=dev)
        y_down = torch.empty((rows, 5120), dtype=torch.float32, device=dev)
        calls = []
        for lm in layers:
            calls += [(lm["qkv"][0], None, xa, y_qkv), (lm["o"][0], None, xo, y_o),
                      (lm["gate"][0], lm["up"][0], xa, o32), (lm["gate"][0], lm["up"][0], xa, o_gu),
                      (lm["down"][0], None, o_gu, y_down)]
        seq = nv.Sequence(calls)
        ws = torch.zeros(seq.workspace_bytes, dtype=torch.uint8, device=dev)
        seq.launch(ws)
        torch.cuda.synchronize()
        assert nv.counters_clear(ws), "counters not returned to zero"
        alone = nv.nvfp4_gemv(last["down"][0], o_gu, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(alone.view(torch.int32), y_down.view(torch.int32))
        xab, xob = _bits(xa), _bits(xo)
        for name, y, xb in (("qkv", y_qkv, xab), ("o", y_o, xob)):
            sel = np.sort(rng.choice(y.shape[1], 256, replace=False))
            ref, absd, ref16 = oracle.gemv(*last[name][1], xb, sel=sel)
            check.check_gemv(y.cpu().numpy()[:, sel], None, ref, absd, ref16,
                             label="sequence %s r%d" % (name, rows))
        sel = np.sort(rng.choice(17408, 256, replace=False))
        d = oracle.gemv_dual_silu(last["gate"][1], last["up"][1], xab, sel=sel)
        check.check_dual(o32.cpu().numpy()[:, sel], _bits(o_gu)[:, sel], d, label="sequence gate/up r%d" % rows)
