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
    assert len(names) == 19, names
    L = ctypes.CDLL(nv.LIB_PATH)
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(nv.EXPORTS)


def test_version_and_strerror(nv):
    assert nv.nvfp4_abi_version() == 1
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
    # more than 16 rows run as row chunks, whose waits need the counters (65 KiB)
    assert nv.nvfp4_workspace_bytes(256, 512, 16) == 0
    assert nv.nvfp4_workspace_bytes(256, 512, 17) == 65 * 1024
    assert nv.nvfp4_workspace_bytes(256, 512, 128) == 65 * 1024
    assert nv.nvfp4_workspace_bytes(5120, 17408, 128) == nv.nvfp4_workspace_bytes(5120, 17408, 16)
    for bad in [(256, 512, 0), (256, 512, 129), (0, 512, 1), (256, 24, 1)]:
        assert nv.nvfp4_workspace_bytes(*bad) == 0
    assert nv.nvfp4_quantize_workspace_bytes(256, 512) > 0
    assert nv.nvfp4_quantize_workspace_bytes(256, 20) == 0


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
    # the largest partial sums (rows 8 of the 5120 x 17408 call) plus the counters
    assert need == nv.nvfp4_workspace_bytes(5120, 17408, 8)
    assert L.nvfp4_gemv_sequence(arr, 3, WF, need - 16, None, None) == E["NVFP4_E_WORKSPACE"]
    # several calls always need the counters, split-K or not
    arr[1].w = ctypes.pointer(good)
    assert L.nvfp4_sequence_workspace_bytes(arr, 3) == 65 * 1024
    assert L.nvfp4_sequence_workspace_bytes(arr, 1) == 0
    assert L.nvfp4_sequence_launches(arr, 0) == 0 and L.nvfp4_sequence_launches(None, 3) == 0
    assert 1 <= L.nvfp4_sequence_launches(arr, 3) <= 3
    # a call of 40 rows runs as three row chunks (14, 13, 13): one call alone
    # needs the counters, and up to three launches
    arr[0].rows = 40
    assert L.nvfp4_sequence_workspace_bytes(arr, 1) == 65 * 1024
    assert 2 <= L.nvfp4_sequence_launches(arr, 1) <= 3
    arr[0].rows = 1
    assert L.nvfp4_gemv_sequence(None, 3, None, 0, None, None) == E["NVFP4_E_NULL"]


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
