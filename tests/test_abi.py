"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/nvfp4.h declares, sizes its buffers as documented, and rejects bad
arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def nv():
    import bit_weight_only_nvfp4_amd as nv
    if not os.path.exists(nv.LIB_PATH):
        from bit_weight_only_nvfp4_amd import build
        build.build()
    nv.lib()
    return nv


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(nv):
    names = _declared_functions()
    assert len(names) >= 20, names
    L = ctypes.CDLL(nv.LIB_PATH)
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(nv.EXPORTS)


def test_version_and_strerror(nv):
    assert nv.nvfp4_abi_version() == nv.NVFP4_ABI_VERSION == 2
    for code in nv.STATUS:
        assert nv.nvfp4_strerror(code) != "unknown status"
    assert nv.nvfp4_strerror(-99) == "unknown status"


def test_packed_bytes(nv):
    # header + strips(64 features) * super-tiles(256 k) * 9216 bytes
    assert nv.nvfp4_packed_bytes(256, 512) == 256 + 4 * 2 * 9216
    assert nv.nvfp4_packed_bytes(12288, 5120) == 256 + 192 * 20 * 9216
    assert nv.nvfp4_packed_bytes(65, 272) == 256 + 2 * 2 * 9216
    assert nv.nvfp4_packed_bytes(1, 16) == 256 + 9216
    for n, k in [(0, 512), (-1, 512), (256, 0), (256, 24), (256, 8)]:
        assert nv.nvfp4_packed_bytes(n, k) == 0


def test_workspace_bytes(nv):
    # whole strips per workgroup (short k, or enough strips to fill the GPU): no split-K
    assert nv.nvfp4_workspace_bytes(256, 512, 1) == 0
    assert nv.nvfp4_workspace_bytes(256, 1024, 8) == 0
    assert nv.nvfp4_workspace_bytes(12288, 5120, 1) == 0
    # skinny shapes and the strips left over past 256 workgroups are cut into pieces
    w1 = nv.nvfp4_workspace_bytes(5120, 17408, 1)
    assert w1 > 0 and w1 == nv.nvfp4_workspace_bytes(5120, 17408, 1)
    assert nv.nvfp4_workspace_bytes(5120, 17408, 8) > w1
    assert nv.nvfp4_workspace_bytes(17408, 5120, 1, dual=True) > nv.nvfp4_workspace_bytes(17408, 5120, 1) > 0
    # Strips left over past one per workgroup: at most 4 pieces each, never more
    # than the leftover's super-tiles; partial sums of R strips x pieces x
    # matrices x rows x 64 fp32 after the 161 KiB of counters.
    state, strip = 161 << 10, 64 * 4
    assert nv.nvfp4_workspace_bytes(17408, 5120, 1, dual=True) == state + 16 * 4 * 2 * 1 * strip
    assert nv.nvfp4_workspace_bytes(17408, 5120, 8, dual=True) == state + 16 * 4 * 2 * 8 * strip
    assert nv.nvfp4_workspace_bytes(16448, 5120, 1) == state + 1 * 4 * strip     # 257 strips of 20 super-tiles
    assert nv.nvfp4_workspace_bytes(16448, 512, 1) == state + 1 * 2 * strip      # 2 super-tiles: 2 pieces
    assert nv.nvfp4_workspace_bytes(16448, 256, 1) == 0                          # one super-tile: one owner
    assert nv.nvfp4_workspace_bytes(19200, 1024, 1) == state + 44 * 4 * strip    # 44 strips of 4 super-tiles
    assert nv.nvfp4_workspace_bytes(32896, 256, 1, dual=True) == 0               # two leftover super-tiles
    # more than 16 rows run as row chunks, whose launch needs the counters and waits
    assert nv.nvfp4_workspace_bytes(256, 512, 16) == 0
    assert nv.nvfp4_workspace_bytes(256, 512, 17) == SEQ_WS
    assert nv.nvfp4_workspace_bytes(256, 512, 128) == SEQ_WS
    # row chunks run as calls of a sequence: 4 regions of the largest partial sums
    p16 = nv.nvfp4_workspace_bytes(5120, 17408, 16) - SEQ_WS
    assert nv.nvfp4_workspace_bytes(5120, 17408, 128) == SEQ_WS + 4 * (-(-p16 // 256) * 256)
    for bad in [(256, 512, 0), (256, 512, 129), (0, 512, 1), (256, 24, 1)]:
        assert nv.nvfp4_workspace_bytes(*bad) == 0
    assert nv.nvfp4_quantize_workspace_bytes(256, 512) > 0
    assert nv.nvfp4_quantize_workspace_bytes(256, 20) == 0


# a sequence workspace with no partial sums: the counters and waits
SEQ_WS = 161 * 1024
FAKE = 0x10000      # 64 KiB-aligned addresses that are never dereferenced:
XF = 0x1000000      # weights at FAKE, activations at XF, outputs at YF,
YF = 0x2000000      # workspaces at WF (16 MiB apart: no two overlap)
WF = 0x3000000


def _weight(nv, n=256, k=512, magic=None, layout=None, data=FAKE):
    w = nv.nvfp4_weight()
    w.magic = nv.NVFP4_LAYOUT_MAGIC if magic is None else magic
    w.layout = nv.NVFP4_LAYOUT_VERSION if layout is None else layout
    w.n, w.k, w.data = n, k, data
    return w


def _gemv(nv, w, x=XF, rows=1, y=YF, dtype=0, ws=None, wsb=0):
    return nv.lib().nvfp4_gemv(ctypes.byref(w) if w is not None else None, x, rows, y, dtype, ws, wsb, None)


def test_gemv_argument_errors(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    assert _gemv(nv, None) == E["NVFP4_E_NULL"]
    assert "w is NULL" in nv.nvfp4_last_error()
    assert _gemv(nv, _weight(nv, magic=0x1234)) == E["NVFP4_E_LAYOUT"]
    assert _gemv(nv, _weight(nv, layout=7)) == E["NVFP4_E_LAYOUT"]
    assert _gemv(nv, _weight(nv, k=24)) == E["NVFP4_E_SHAPE"]
    assert _gemv(nv, _weight(nv, n=0)) == E["NVFP4_E_SHAPE"]
    assert _gemv(nv, _weight(nv, data=None)) == E["NVFP4_E_NULL"]
    assert _gemv(nv, _weight(nv, data=FAKE + 8)) == E["NVFP4_E_ALIGN"]
    assert _gemv(nv, _weight(nv), x=None) == E["NVFP4_E_NULL"]
    assert _gemv(nv, _weight(nv), y=None) == E["NVFP4_E_NULL"]
    assert _gemv(nv, _weight(nv), rows=0) == E["NVFP4_E_ROWS"]
    assert _gemv(nv, _weight(nv), rows=129) == E["NVFP4_E_ROWS"]
    assert _gemv(nv, _weight(nv), dtype=2) == E["NVFP4_E_DTYPE"]
    assert _gemv(nv, _weight(nv), x=XF + 2) == E["NVFP4_E_ALIGN"]
    assert _gemv(nv, _weight(nv), y=YF + 1) == E["NVFP4_E_ALIGN"]
    assert _gemv(nv, _weight(nv), y=YF + 2, dtype=1) == E["NVFP4_E_ALIGN"]
    big = _weight(nv, n=5120, k=17408)
    need = nv.nvfp4_workspace_bytes(5120, 17408, 1)
    assert _gemv(nv, big) == E["NVFP4_E_WORKSPACE"]
    assert _gemv(nv, big, ws=WF, wsb=need - 1) == E["NVFP4_E_WORKSPACE"]
    assert _gemv(nv, big, ws=WF + 4, wsb=need) == E["NVFP4_E_ALIGN"]


def test_overlap_errors(nv):
    """An output may not overlap its activations, the weight or the workspace;
    in a sequence, no output may overlap any call's weight."""
    E = {v: k for k, v in nv.STATUS.items()}
    L = nv.lib()
    w = _weight(nv)                                   # 256 x 512: bytes [FAKE, FAKE + 73984)
    assert _gemv(nv, w, y=XF) == E["NVFP4_E_OVERLAP"]
    assert _gemv(nv, w, x=YF + 256) == E["NVFP4_E_OVERLAP"]          # y = [YF, YF + 512)
    assert _gemv(nv, w, y=FAKE + 73984 - 2) == E["NVFP4_E_OVERLAP"]
    big = _weight(nv, n=5120, k=17408)
    need = nv.nvfp4_workspace_bytes(5120, 17408, 1)
    assert _gemv(nv, big, y=WF + need - 2, ws=WF, wsb=need) == E["NVFP4_E_OVERLAP"]
    assert "workspace" in nv.nvfp4_last_error()
    arr = (nv.nvfp4_call * 3)()
    ws = [_weight(nv, 256, 512, data=FAKE + i * 0x100000) for i in range(3)]
    for i, c in enumerate(arr):
        c.w = ctypes.pointer(ws[i])
        c.x, c.y, c.rows, c.out_dtype = XF, YF + i * 0x10000, 1, 0
    arr[0].y = FAKE + 2 * 0x100000 + 4096                # into call 2's weight
    sneed = L.nvfp4_sequence_workspace_bytes(arr, 3)
    assert L.nvfp4_gemv_sequence(arr, 3, WF, sneed, None, None) == E["NVFP4_E_OVERLAP"]
    assert "call 0" in nv.nvfp4_last_error() and "call 2" in nv.nvfp4_last_error()


def test_dual_and_pack_argument_errors(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    L = nv.lib()
    g, u = _weight(nv, 256, 512), _weight(nv, 256, 1024)
    assert L.nvfp4_gemv_dual_silu(ctypes.byref(g), ctypes.byref(u), FAKE, 1, FAKE, 0, None, 0, None) == \
        E["NVFP4_E_SHAPE"]
    assert L.nvfp4_gemv_dual_silu(ctypes.byref(g), None, FAKE, 1, FAKE, 0, None, 0, None) == E["NVFP4_E_NULL"]
    out = nv.nvfp4_weight()
    need = nv.nvfp4_packed_bytes(256, 512)
    assert L.nvfp4_pack(None, FAKE, 1.0, 256, 512, FAKE, need, ctypes.byref(out), None) == E["NVFP4_E_NULL"]
    assert L.nvfp4_pack(FAKE, FAKE, 1.0, 256, 520, FAKE, need, ctypes.byref(out), None) == E["NVFP4_E_SHAPE"]
    assert L.nvfp4_pack(FAKE, FAKE, 1.0, 256, 512, FAKE + 4, need, ctypes.byref(out), None) == E["NVFP4_E_ALIGN"]
    assert L.nvfp4_pack(FAKE, FAKE, 1.0, 256, 512, FAKE, need - 1, ctypes.byref(out), None) == \
        E["NVFP4_E_LAYOUT"]
    qneed = nv.nvfp4_quantize_workspace_bytes(256, 512)
    assert L.nvfp4_quantize(FAKE, 256, 512, FAKE, need, FAKE, qneed - 1, ctypes.byref(out), None) == \
        E["NVFP4_E_WORKSPACE"]
    assert L.nvfp4_quantize(FAKE + 4, 256, 512, FAKE, need, FAKE, qneed, ctypes.byref(out), None) == \
        E["NVFP4_E_ALIGN"]
    w = _weight(nv)
    assert L.nvfp4_dequant(ctypes.byref(w), FAKE + 4, None) == E["NVFP4_E_ALIGN"]
    assert L.nvfp4_unpack(ctypes.byref(w), None, FAKE, None, None) == E["NVFP4_E_NULL"]


def test_sequence_argument_errors(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    L = nv.lib()
    arr = (nv.nvfp4_call * 3)()
    good = _weight(nv, 256, 512)
    bad = _weight(nv, 256, 512, magic=1)
    for c in arr:
        c.w = ctypes.pointer(good)
        c.x, c.y, c.rows, c.out_dtype = XF, YF, 1, 0
    assert L.nvfp4_gemv_sequence(arr, 0, None, 0, None, None) == 0       # nothing to do
    arr[2].w = ctypes.pointer(bad)
    assert L.nvfp4_gemv_sequence(arr, 3, None, 0, None, None) == E["NVFP4_E_LAYOUT"]
    assert "call 2" in nv.nvfp4_last_error()
    arr[2].w = ctypes.pointer(good)
    arr[1].rows = 129
    assert L.nvfp4_gemv_sequence(arr, 3, None, 0, None, None) == E["NVFP4_E_ROWS"]
    assert "call 1" in nv.nvfp4_last_error()
    arr[1].rows = 8
    up = _weight(nv, 256, 1024)
    arr[0].up = ctypes.pointer(up)
    assert L.nvfp4_gemv_sequence(arr, 3, None, 0, None, None) == E["NVFP4_E_SHAPE"]
    arr[0].up = None
    big = _weight(nv, 5120, 17408)
    arr[1].w = ctypes.pointer(big)
    need = L.nvfp4_sequence_workspace_bytes(arr, 3)
    # 4 regions of the largest partial sums (rows 8 of the 5120 x 17408 call) plus the counters
    p8 = nv.nvfp4_workspace_bytes(5120, 17408, 8) - SEQ_WS
    assert need == SEQ_WS + 4 * (-(-p8 // 256) * 256)
    assert L.nvfp4_gemv_sequence(arr, 3, WF, need - 16, None, None) == E["NVFP4_E_WORKSPACE"]
    # several calls always need the counters, split-K or not
    arr[1].w = ctypes.pointer(good)
    assert L.nvfp4_sequence_workspace_bytes(arr, 3) == SEQ_WS
    assert L.nvfp4_sequence_workspace_bytes(arr, 1) == 0
    assert L.nvfp4_sequence_launches(arr, 0) == 0 and L.nvfp4_sequence_launches(None, 3) == 0
    assert 1 <= L.nvfp4_sequence_launches(arr, 3) <= 3
    # a call of 40 rows runs as three row chunks (14, 13, 13): one call alone
    # needs the counters, and up to three launches
    arr[0].rows = 40
    assert L.nvfp4_sequence_workspace_bytes(arr, 1) == SEQ_WS
    assert 2 <= L.nvfp4_sequence_launches(arr, 1) <= 3
    arr[0].rows = 1
    assert L.nvfp4_gemv_sequence(None, 3, None, 0, None, None) == E["NVFP4_E_NULL"]


def _norm_sequence(nv, rows=1, k=512):
    """[residual add + RMSNorm, projection reading its x, projection writing
    the next norm's delta, residual add + RMSNorm]: the four calls of half a
    decode layer, at fake addresses."""
    keep = []
    w = _weight(nv, 256, k)                                   # [FAKE, FAKE + 73984)
    wo = _weight(nv, k, 256, data=FAKE + 0x100000)
    keep += [w, wo]
    norms = []
    for i in range(2):
        nm = nv.nvfp4_norm()
        nm.residual = nm.residual_out = XF + 0x400000         # updated in place by both
        nm.delta = YF + 0x300000                              # the second: written by call 2
        nm.weight = FAKE + 0x800000 + i * 0x10000
        nm.k, nm.eps, nm.gemma_offset = k, 1e-6, i
        norms.append(nm)
    arr = (nv.nvfp4_call * 4)()
    for c, nm in ((arr[0], norms[0]), (arr[3], norms[1])):
        c.norm = ctypes.pointer(nm)
        c.y, c.rows, c.out_dtype = YF + 0x500000, rows, 0
    arr[1].w, arr[1].x, arr[1].y = ctypes.pointer(w), YF + 0x500000, YF + 0x600000
    arr[2].w, arr[2].x, arr[2].y = ctypes.pointer(wo), YF + 0x600000, YF + 0x300000
    for c in (arr[1], arr[2]):
        c.rows, c.out_dtype = rows, 0
    return arr, norms, keep


def test_sequence_norm_call_errors(nv):
    """Residual add + RMSNorm calls inside a sequence: the checks of
    nvfp4_residual_rmsnorm, plus the sequence's own (a norm's delta may be an
    earlier call's output; its outputs may not overlap any weight)."""
    E = {v: k for k, v in nv.STATUS.items()}
    L = nv.lib()
    arr, norms, keep = _norm_sequence(nv)
    need = L.nvfp4_sequence_workspace_bytes(arr, 4)
    assert need == SEQ_WS and L.nvfp4_sequence_workspace_bytes(arr, 1) == 0
    assert 1 <= L.nvfp4_sequence_launches(arr, 4) <= 4

    def run():
        return L.nvfp4_gemv_sequence(arr, 4, WF, need, None, None)

    def expect(status, text):
        assert run() == E[status], nv.nvfp4_last_error()
        assert text in nv.nvfp4_last_error(), nv.nvfp4_last_error()

    if torch.cuda.device_count() == 0:
        assert run() == E["NVFP4_E_DEVICE"]      # every check passed
    arr[0].w = arr[1].w
    expect("NVFP4_E_NULL", "call 0")
    arr[0].w = None
    norms[1].residual = None
    expect("NVFP4_E_NULL", "call 3")
    norms[1].residual = XF + 0x400000
    norms[0].k = 24
    expect("NVFP4_E_SHAPE", "call 0")
    norms[0].k = 65536 + 16
    expect("NVFP4_E_SHAPE", "call 0")
    norms[0].k = 512
    arr[3].rows = 129
    expect("NVFP4_E_ROWS", "call 3")
    arr[3].rows = 1
    arr[3].out_dtype = 1
    expect("NVFP4_E_DTYPE", "call 3")
    arr[3].out_dtype = 0
    norms[1].eps = float("nan")
    expect("NVFP4_E_SHAPE", "call 3")
    norms[1].eps = 1e-6
    norms[0].delta = YF + 0x300000 + 8
    expect("NVFP4_E_ALIGN", "call 0")
    norms[0].delta = YF + 0x300000
    norms[0].residual_out = XF + 0x400000 + 512              # partly over its residual
    expect("NVFP4_E_OVERLAP", "call 0")
    norms[0].residual_out = YF + 0x300000                    # over its delta
    expect("NVFP4_E_OVERLAP", "call 0")
    norms[0].residual_out = FAKE + 0x100000 + 4096           # over call 2's weight
    expect("NVFP4_E_OVERLAP", "call 2")
    norms[0].residual_out = YF + 0x600000                    # over call 1's y
    expect("NVFP4_E_OVERLAP", "call 1")
    norms[0].residual_out = FAKE + 0x800000 + 0x10000        # over the other norm's weight
    expect("NVFP4_E_OVERLAP", "call 3")
    norms[0].residual_out = XF + 0x400000
    arr[3].y = FAKE + 0x800000                               # its y over the first norm's weight
    expect("NVFP4_E_OVERLAP", "weight of call 0")
    arr[3].y = XF + 0x400000                                 # its y over its residual
    expect("NVFP4_E_OVERLAP", "call 3")
    arr[3].y = YF + 0x500000
    arr[2].y = FAKE + 0x800000 + 0x10000                     # a projection's y over a norm weight
    expect("NVFP4_E_OVERLAP", "weight of call 3")
    arr[2].y = YF + 0x300000
    arr[2].y = WF + 64                                       # over the workspace
    expect("NVFP4_E_OVERLAP", "workspace")
    arr[2].y = YF + 0x300000
    if torch.cuda.device_count() == 0:
        assert run() == E["NVFP4_E_DEVICE"]
    del keep


def test_sequence_norm_launch_grouping(nv):
    """A norm call runs in the launch of the projections of its row count
    (rows past 16: the kernel of their row chunks)."""
    L = nv.lib()
    for rows in (1, 5, 8, 24, 40):
        arr, norms, keep = _norm_sequence(nv, rows=rows)
        alone = L.nvfp4_sequence_launches(arr, 1)
        assert alone == 1
        chunks = -(-rows // 16)
        # per call: one launch per row chunk of a projection, one for a norm
        assert L.nvfp4_sequence_launches(arr, 4) <= 2 * chunks + 2
        del keep


def test_sequence_plan_errors(nv):
    """nvfp4_sequence_plan validates once what nvfp4_gemv_sequence validates
    each time; nvfp4_sequence_plan_launch checks the header, the workspace
    and the device only."""
    E = {v: k for k, v in nv.STATUS.items()}
    L = nv.lib()
    arr, norms, keep = _norm_sequence(nv)
    nb = L.nvfp4_sequence_plan_bytes(arr, 4)
    assert nb > 0 and nb % 8 == 0
    buf = (ctypes.c_uint64 * (nb // 8 + 4))()
    base = ctypes.addressof(buf)
    plan = base + (-base % 16)
    assert L.nvfp4_sequence_plan(arr, 4, plan, nb - 8) == E["NVFP4_E_WORKSPACE"]
    assert L.nvfp4_sequence_plan(arr, 4, plan + 8, nb) == E["NVFP4_E_ALIGN"]
    assert L.nvfp4_sequence_plan(arr, 4, None, nb) == E["NVFP4_E_NULL"]
    assert L.nvfp4_sequence_plan(arr, 0, plan, nb) == E["NVFP4_E_SHAPE"]
    assert L.nvfp4_sequence_plan(arr, 4, plan, nb) == 0
    need = L.nvfp4_sequence_workspace_bytes(arr, 4)
    assert L.nvfp4_sequence_plan_launch(plan, WF, need - 16, None) == E["NVFP4_E_WORKSPACE"]
    assert L.nvfp4_sequence_plan_launch(plan, WF + 4, need, None) == E["NVFP4_E_ALIGN"]
    assert L.nvfp4_sequence_plan_launch(plan, YF + 0x600000 - 64, need, None) == E["NVFP4_E_OVERLAP"]
    assert L.nvfp4_sequence_plan_launch(plan, XF + 0x400000, need, None) == E["NVFP4_E_OVERLAP"]  # residual_out
    if torch.cuda.device_count() == 0:
        assert L.nvfp4_sequence_plan_launch(plan, WF, need, None) == E["NVFP4_E_DEVICE"]
    assert L.nvfp4_sequence_plan_launch(plan + 16, WF, need, None) == E["NVFP4_E_LAYOUT"]
    assert L.nvfp4_sequence_plan_launch(None, WF, need, None) == E["NVFP4_E_NULL"]
    # invalid calls: no size, and the plan call names the call
    arr[2].rows = 0
    assert L.nvfp4_sequence_plan_bytes(arr, 4) == 0
    assert "call 2" in nv.nvfp4_last_error()
    assert L.nvfp4_sequence_plan(arr, 4, plan, nb) == E["NVFP4_E_ROWS"]
    arr[2].rows = 1
    arr[2].y = FAKE + 0x800000                               # over a norm weight: found at plan time
    assert L.nvfp4_sequence_plan(arr, 4, plan, nb) == E["NVFP4_E_OVERLAP"]
    arr[2].y = YF + 0x300000
    # the Python Sequence validates at construction
    del keep


def test_sequence_object_validates_once(nv):
    w = _weight(nv, 256, 512)
    x = torch.empty((1, 512), dtype=torch.bfloat16)
    y = torch.empty((1, 300), dtype=torch.bfloat16)
    pw = nv.PackedWeight(torch.empty(0, dtype=torch.uint8), w)
    with pytest.raises(ValueError):
        nv.Sequence([(pw, None, x, y)])                     # y is not [1, 256]
    x0 = torch.empty((0, 512), dtype=torch.bfloat16)
    y0 = torch.empty((0, 256), dtype=torch.bfloat16)
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.Sequence([(pw, None, x0, y0), (pw, None, x0, y0)])
    assert "call 0" in str(e.value)   # empty tensors: a NULL x


def test_sequence_waits(nv):
    """Where a launch of several calls waits between them (the host's reading
    of the calls' address ranges): a call waits when it reads what a call
    since the last wait writes, or writes what one reads or writes, and after
    every 4 calls run without one."""
    L = nv.lib()
    MB = 0x100000
    keep = []

    def w(n, k, i):
        wt = _weight(nv, n, k, data=0x100000000 + i * 0x10000000)
        keep.append(wt)
        return ctypes.pointer(wt)

    def proj(wp, x, y, up=None, rows=1):
        c = nv.nvfp4_call()
        c.w, c.up, c.x, c.y, c.rows, c.out_dtype = wp, up, x, y, rows, 0
        return c

    def norm(resid, delta, weight, xout, k=512, rows=1):
        nm = nv.nvfp4_norm(resid, delta, weight, resid, k, 1e-6, 1)
        keep.append(nm)
        c = nv.nvfp4_call()
        c.norm, c.y, c.rows, c.out_dtype = ctypes.pointer(nm), xout, rows, 0
        return c

    def waits(calls):
        arr = (nv.nvfp4_call * len(calls))(*calls)
        return L.nvfp4_sequence_waits(arr, len(calls))

    X1, X2, Yq, Yo, H, Yd = (XF + i * 16 * MB for i in range(6))
    # the benchmark's step: qkv and o read fixed x, the pair too, down reads the pair's output
    step = []
    for l in range(3):
        step += [proj(w(768, 512, 5 * l), X1, Yq), proj(w(512, 384, 5 * l + 1), X2, Yo),
                 proj(w(1024, 512, 5 * l + 2), X1, H, up=w(1024, 512, 5 * l + 3)),
                 proj(w(512, 1024, 5 * l + 4), H, Yd)]
    # layer 0: down waits (reads H); later layers: the pair waits too (overwrites what down read)
    assert waits(step) == 1 + 2 + 2
    # the pair's output alternating between two buffers: down alone waits, and the
    # runs between waits are down, qkv, o, pair (four calls)
    H2 = XF + 10 * 16 * MB
    step2 = []
    for l in range(4):
        h = (H, H2)[l % 2]
        step2 += [proj(w(768, 512, 40 + 5 * l), X1, Yq), proj(w(512, 384, 41 + 5 * l), X2, Yo),
                  proj(w(1024, 512, 42 + 5 * l), X1, h, up=w(1024, 512, 43 + 5 * l)),
                  proj(w(512, 1024, 44 + 5 * l), h, Yd)]
    assert waits(step2) == 4
    # independent calls: a wait after every run of 4
    ind = [proj(w(256, 512, 100 + i), XF + i * MB, 0x40000000 + i * MB) for i in range(9)]
    assert waits(ind) == 2
    # a chain: each reads the previous output
    chain = [proj(w(512, 512, 200 + i), XF + i * 16 * MB, XF + (i + 1) * 16 * MB) for i in range(5)]
    assert waits(chain) == 4
    # two writers of one buffer
    assert waits([proj(w(256, 512, 300), X1, Yq), proj(w(256, 512, 301), X2, Yq)]) == 1
    # a decoder layer with norms: norm, qkv, o, norm, pair, down -- qkv waits for the
    # norm's x, the second norm for o's output, the pair for its x, down for the
    # pair's output, the next layer's first norm for down's output: o alone runs
    # beside qkv
    R, XN, A = XF + 7 * 16 * MB, XF + 8 * 16 * MB, XF + 9 * 16 * MB
    ln = [0x100000000 + (400 + i) * 0x10000000 for i in range(4)]
    layer = []
    for l in range(2):
        layer += [norm(R, Yd, ln[2 * l], XN), proj(w(768, 512, 500 + 5 * l), XN, Yq),
                  proj(w(512, 384, 501 + 5 * l), A, Yo), norm(R, Yo, ln[2 * l + 1], XN),
                  proj(w(1024, 512, 502 + 5 * l), XN, H, up=w(1024, 512, 503 + 5 * l)),
                  proj(w(512, 1024, 504 + 5 * l), H, Yd)]
    assert waits(layer) == 4 + 5
    # invalid calls: the status
    bad = [proj(w(256, 512, 600), X1, Yq), proj(w(256, 512, 601), X1, Yq, rows=0)]
    assert waits(bad) == {v: k for k, v in nv.STATUS.items()}["NVFP4_E_ROWS"]
    del keep


def _dense(nv, W=FAKE, n=256, k=512, x=XF, rows=1, y=YF, dtype=0):
    return nv.lib().nvfp4_dense_gemv_bf16(W, n, k, x, rows, y, dtype, None)


def test_dense_gemv_argument_errors(nv):
    """Every argument check of the dense bf16 projection runs before any HIP
    call (these fake pointers are never dereferenced)."""
    E = {v: k for k, v in nv.STATUS.items()}
    assert _dense(nv, W=None) == E["NVFP4_E_NULL"]
    assert "W is NULL" in nv.nvfp4_last_error()
    assert _dense(nv, x=None) == E["NVFP4_E_NULL"]
    assert _dense(nv, y=None) == E["NVFP4_E_NULL"]
    assert _dense(nv, k=24) == E["NVFP4_E_SHAPE"]
    assert _dense(nv, n=0) == E["NVFP4_E_SHAPE"]
    assert _dense(nv, n=(1 << 20) + 1) == E["NVFP4_E_SHAPE"]
    assert _dense(nv, rows=0) == E["NVFP4_E_ROWS"]
    assert _dense(nv, rows=129) == E["NVFP4_E_ROWS"]
    assert _dense(nv, dtype=2) == E["NVFP4_E_DTYPE"]
    assert _dense(nv, W=FAKE + 8) == E["NVFP4_E_ALIGN"]
    assert _dense(nv, x=XF + 2) == E["NVFP4_E_ALIGN"]
    assert _dense(nv, y=YF + 2, dtype=1) == E["NVFP4_E_ALIGN"]
    assert _dense(nv, y=XF + 256) == E["NVFP4_E_OVERLAP"]        # y inside x
    assert "y overlaps x" in nv.nvfp4_last_error()
    assert _dense(nv, y=FAKE + 4096) == E["NVFP4_E_OVERLAP"]     # y inside W
    assert "y overlaps W" in nv.nvfp4_last_error()


def _mx(nv, c=FAKE, s=WF, n=256, k=512, x=XF, rows=1, y=YF, dtype=0):
    return nv.lib().nvfp4_mxfp4_gemv(c, s, n, k, x, rows, y, dtype, None)


def test_mxfp4_gemv_argument_errors(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    assert _mx(nv, c=None) == E["NVFP4_E_NULL"]
    assert _mx(nv, s=None) == E["NVFP4_E_NULL"]
    assert _mx(nv, x=None) == E["NVFP4_E_NULL"]
    assert _mx(nv, k=48) == E["NVFP4_E_SHAPE"]              # not a multiple of 32
    assert _mx(nv, n=0) == E["NVFP4_E_SHAPE"]
    assert _mx(nv, rows=129) == E["NVFP4_E_ROWS"]
    assert _mx(nv, c=FAKE + 8) == E["NVFP4_E_ALIGN"]
    assert _mx(nv, dtype=5) == E["NVFP4_E_DTYPE"]
    assert _mx(nv, y=XF + 64) == E["NVFP4_E_OVERLAP"]
    assert _mx(nv, y=FAKE + 1024) == E["NVFP4_E_OVERLAP"]


def _w8(nv, c=FAKE, s=WF, n=256, k=512, x=XF, rows=1, y=YF, dtype=0):
    return nv.lib().nvfp4_w8g32_gemv(c, s, n, k, x, rows, y, dtype, None)


def test_w8g32_gemv_argument_errors(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    assert _w8(nv, c=None) == E["NVFP4_E_NULL"]
    assert _w8(nv, s=None) == E["NVFP4_E_NULL"]
    assert _w8(nv, k=96) == E["NVFP4_E_SHAPE"]               # not a multiple of 128
    assert _w8(nv, n=(1 << 20) + 1) == E["NVFP4_E_SHAPE"]
    assert _w8(nv, rows=0) == E["NVFP4_E_ROWS"]
    assert _w8(nv, s=WF + 4) == E["NVFP4_E_ALIGN"]
    assert _w8(nv, c=FAKE + 8) == E["NVFP4_E_ALIGN"]
    assert _w8(nv, y=XF + 64) == E["NVFP4_E_OVERLAP"]
    assert _w8(nv, y=FAKE + 4096) == E["NVFP4_E_OVERLAP"]


def _norm(nv, r=XF, h=WF, w=FAKE, k=512, rows=2, eps=1e-6, gemma=0, ro=YF, x=YF + 0x100000):
    return nv.lib().nvfp4_residual_rmsnorm(r, h, w, k, rows, eps, gemma, ro, x, None)


def test_residual_rmsnorm_argument_errors(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    assert _norm(nv, r=None) == E["NVFP4_E_NULL"]
    assert _norm(nv, h=None) == E["NVFP4_E_NULL"]
    assert _norm(nv, w=None) == E["NVFP4_E_NULL"]
    assert _norm(nv, ro=None) == E["NVFP4_E_NULL"]
    assert _norm(nv, x=None) == E["NVFP4_E_NULL"]
    assert _norm(nv, k=24) == E["NVFP4_E_SHAPE"]
    assert _norm(nv, k=0) == E["NVFP4_E_SHAPE"]
    assert _norm(nv, k=65536 + 16) == E["NVFP4_E_SHAPE"]
    assert _norm(nv, rows=0) == E["NVFP4_E_ROWS"]
    assert _norm(nv, eps=-1.0) == E["NVFP4_E_SHAPE"]
    assert _norm(nv, eps=float("nan")) == E["NVFP4_E_SHAPE"]
    assert _norm(nv, h=WF + 8) == E["NVFP4_E_ALIGN"]
    assert _norm(nv, ro=XF + 512) == E["NVFP4_E_OVERLAP"]       # partly over the residual
    assert _norm(nv, x=WF) == E["NVFP4_E_OVERLAP"]              # over delta
    assert _norm(nv, x=YF) == E["NVFP4_E_OVERLAP"]              # over residual_out
    assert "x overlaps" in nv.nvfp4_last_error()


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="valid arguments would launch on a real device")
def test_no_device_is_refused(nv):
    E = {v: k for k, v in nv.STATUS.items()}
    assert _gemv(nv, _weight(nv)) == E["NVFP4_E_DEVICE"]
    assert "gfx950" in nv.nvfp4_last_error()


def test_python_binding_fails_loudly_without_library(monkeypatch, nv):
    import bit_weight_only_nvfp4_amd as pkg
    monkeypatch.setattr(pkg, "_lib", None)
    monkeypatch.setattr(pkg, "LIB_PATH", "/nonexistent/libnvfp4_hip.so")
    with pytest.raises(ImportError):
        pkg.lib()


def test_read_ceiling_argument_errors(nv):
    L = nv.lib()
    E = {v: k for k, v in nv.STATUS.items()}
    assert L.nvfp4_read_ceiling(None, 1024, YF, None) == E["NVFP4_E_NULL"]
    assert L.nvfp4_read_ceiling(FAKE, 0, YF, None) == E["NVFP4_E_SHAPE"]
    assert L.nvfp4_read_ceiling(FAKE, 1000, YF, None) == E["NVFP4_E_SHAPE"]
    assert L.nvfp4_read_ceiling(FAKE + 8, 1024, YF, None) == E["NVFP4_E_ALIGN"]


def test_read_ceiling_binding_stays_inside_the_buffer(nv):
    """The binding refuses a read past its tensor before calling the library
    (the C entry point takes a raw pointer and cannot tell)."""
    buf = torch.zeros(4096, dtype=torch.uint8)
    sink = torch.zeros(256, dtype=torch.int32)
    with pytest.raises(ValueError):
        nv.nvfp4_read_ceiling(buf, 8192, sink)
    with pytest.raises(ValueError):
        nv.nvfp4_read_ceiling(buf, 2048, sink, offset=3072)
    with pytest.raises(ValueError):
        nv.nvfp4_read_ceiling(buf, 1024, torch.zeros(16, dtype=torch.int32))
