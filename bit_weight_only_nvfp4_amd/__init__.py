"""MI355X (gfx950) weight-only NVFP4 projection GEMV -- Python binding.

Thin ctypes layer over ``libnvfp4_hip.so`` (C ABI in ``include/nvfp4.h``).  It
only marshals arguments: torch owns device memory and streams, and every step
of the computation runs in the library's HIP kernels.  There is no CPU
fallback; calling into the library without a built ``libnvfp4_hip.so`` raises.

Entry points (same names as the C ABI):
  nvfp4_packed_bytes, nvfp4_pack, nvfp4_unpack, nvfp4_dequant,
  nvfp4_quantize_workspace_bytes, nvfp4_quantize,
  nvfp4_workspace_bytes, nvfp4_gemv, nvfp4_gemv_dual_silu,
  nvfp4_sequence_workspace_bytes, nvfp4_gemv_sequence, nvfp4_sequence_launches
  (projections, gate/up pairs and residual add + RMSNorm calls: Sequence, Norm),
  nvfp4_abi_version, nvfp4_strerror, nvfp4_last_error.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4_hip.so")

NVFP4_LAYOUT_MAGIC = 0x34465056
NVFP4_LAYOUT_VERSION = 3
NVFP4_ABI_VERSION = 2
NVFP4_MAX_ROWS = 128
NVFP4_OUT_BF16 = 0
NVFP4_OUT_F32 = 1
NVFP4_WS_WAIT_FLAG_OFFSET = 65536   # uint32 in a workspace: a bounded wait of a launch gave up

STATUS = {
    0: "NVFP4_OK", -1: "NVFP4_E_NULL", -2: "NVFP4_E_SHAPE", -3: "NVFP4_E_ROWS", -4: "NVFP4_E_ALIGN",
    -5: "NVFP4_E_DTYPE", -6: "NVFP4_E_WORKSPACE", -7: "NVFP4_E_LAYOUT", -8: "NVFP4_E_DEVICE",
    -9: "NVFP4_E_HIP", -10: "NVFP4_E_OVERLAP",
}

EXPORTS = (
    "nvfp4_abi_version", "nvfp4_strerror", "nvfp4_last_error", "nvfp4_packed_bytes", "nvfp4_pack",
    "nvfp4_unpack", "nvfp4_dequant", "nvfp4_quantize_workspace_bytes", "nvfp4_quantize",
    "nvfp4_workspace_bytes", "nvfp4_gemv", "nvfp4_gemv_dual_silu", "nvfp4_sequence_workspace_bytes",
    "nvfp4_gemv_sequence", "nvfp4_sequence_launches", "nvfp4_dense_gemv_bf16", "nvfp4_residual_rmsnorm",
    "nvfp4_mxfp4_gemv", "nvfp4_w8g32_gemv", "nvfp4_read_ceiling", "nvfp4_gemv_noalloc",
    "nvfp4_sequence_plan_bytes", "nvfp4_sequence_plan", "nvfp4_sequence_plan_launch", "nvfp4_sequence_waits",
)


class nvfp4_weight(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("layout", ctypes.c_uint32),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("data", ctypes.c_void_p),
    ]


class nvfp4_norm(ctypes.Structure):
    _fields_ = [
        ("residual", ctypes.c_void_p),
        ("delta", ctypes.c_void_p),
        ("weight", ctypes.c_void_p),
        ("residual_out", ctypes.c_void_p),
        ("k", ctypes.c_int64),
        ("eps", ctypes.c_float),
        ("gemma_offset", ctypes.c_int),
    ]


class nvfp4_call(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.POINTER(nvfp4_weight)),
        ("up", ctypes.POINTER(nvfp4_weight)),
        ("x", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("rows", ctypes.c_int),
        ("out_dtype", ctypes.c_int),
        ("norm", ctypes.POINTER(nvfp4_norm)),
    ]


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%d): %s" % (fn, STATUS.get(status, "?"), status, detail))


_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError("libnvfp4_hip.so is not built (%s); run __graft_entry__.build() or "
                              "python bit_weight_only_nvfp4_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        wp = ctypes.POINTER(nvfp4_weight)
        sig = {
            "nvfp4_abi_version": ([], ctypes.c_int),
            "nvfp4_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "nvfp4_last_error": ([], ctypes.c_char_p),
            "nvfp4_packed_bytes": ([i64, i64], sz),
            "nvfp4_pack": ([vp, vp, ctypes.c_float, i64, i64, vp, sz, wp, vp], ctypes.c_int),
            "nvfp4_unpack": ([wp, vp, vp, vp, vp], ctypes.c_int),
            "nvfp4_dequant": ([wp, vp, vp], ctypes.c_int),
            "nvfp4_quantize_workspace_bytes": ([i64, i64], sz),
            "nvfp4_quantize": ([vp, i64, i64, vp, sz, vp, sz, wp, vp], ctypes.c_int),
            "nvfp4_workspace_bytes": ([i64, i64, ctypes.c_int, ctypes.c_int], sz),
            "nvfp4_gemv": ([wp, vp, ctypes.c_int, vp, ctypes.c_int, vp, sz, vp], ctypes.c_int),
            "nvfp4_gemv_dual_silu": ([wp, wp, vp, ctypes.c_int, vp, ctypes.c_int, vp, sz, vp], ctypes.c_int),
            "nvfp4_sequence_workspace_bytes": ([ctypes.POINTER(nvfp4_call), ctypes.c_int], sz),
            "nvfp4_sequence_launches": ([ctypes.POINTER(nvfp4_call), ctypes.c_int], ctypes.c_int),
            "nvfp4_gemv_sequence": ([ctypes.POINTER(nvfp4_call), ctypes.c_int, vp, sz,
                                     ctypes.POINTER(ctypes.c_void_p), vp], ctypes.c_int),
            "nvfp4_dense_gemv_bf16": ([vp, i64, i64, vp, ctypes.c_int, vp, ctypes.c_int, vp], ctypes.c_int),
            "nvfp4_mxfp4_gemv": ([vp, vp, i64, i64, vp, ctypes.c_int, vp, ctypes.c_int, vp], ctypes.c_int),
            "nvfp4_w8g32_gemv": ([vp, vp, i64, i64, vp, ctypes.c_int, vp, ctypes.c_int, vp], ctypes.c_int),
            "nvfp4_residual_rmsnorm": ([vp, vp, vp, i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, vp, vp, vp],
                                       ctypes.c_int),
            "nvfp4_read_ceiling": ([vp, sz, vp, vp], ctypes.c_int),
            "nvfp4_gemv_noalloc": ([wp, vp, ctypes.c_int, vp, ctypes.c_int, vp], ctypes.c_int),
            "nvfp4_sequence_waits": ([ctypes.POINTER(nvfp4_call), ctypes.c_int], ctypes.c_int),
            "nvfp4_sequence_plan_bytes": ([ctypes.POINTER(nvfp4_call), ctypes.c_int], sz),
            "nvfp4_sequence_plan": ([ctypes.POINTER(nvfp4_call), ctypes.c_int, vp, sz], ctypes.c_int),
            "nvfp4_sequence_plan_launch": ([vp, vp, sz, vp], ctypes.c_int),
        }
        for name, (argt, rest) in sig.items():
            f = getattr(L, name)
            f.argtypes = argt
            f.restype = rest
        _lib = L
        return L


def _check(fn: str, status: int):
    if status != 0:
        raise Nvfp4Error(fn, status, lib().nvfp4_last_error().decode(errors="replace"))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def nvfp4_abi_version() -> int:
    return lib().nvfp4_abi_version()


def nvfp4_strerror(status: int) -> str:
    return lib().nvfp4_strerror(status).decode()


def nvfp4_last_error() -> str:
    return lib().nvfp4_last_error().decode(errors="replace")


class PackedWeight:
    """A packed NVFP4 weight: the device byte buffer plus its C descriptor."""

    def __init__(self, data: torch.Tensor, desc: nvfp4_weight):
        self.data = data
        self.desc = desc

    @property
    def n(self) -> int:
        return self.desc.n

    @property
    def k(self) -> int:
        return self.desc.k

    @property
    def device(self):
        return self.data.device

    def global_scale(self) -> float:
        """s_g as stored in the packed header (synchronizes)."""
        return float(self.data[:4].view(torch.float32).item())


def nvfp4_packed_bytes(n: int, k: int) -> int:
    return int(lib().nvfp4_packed_bytes(n, k))


def _alloc_packed(n, k, device, out):
    need = nvfp4_packed_bytes(n, k)
    if need == 0:
        raise ValueError("invalid NVFP4 shape n=%d k=%d (k must be a positive multiple of 16)" % (n, k))
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=device)
    return out, need


def nvfp4_pack(codes: torch.Tensor, scales: torch.Tensor, global_scale: float,
               out: torch.Tensor | None = None) -> PackedWeight:
    """codes uint8 [n, k/2], scales uint8 [n, k/16] (device) -> PackedWeight."""
    n, half = codes.shape
    k = 2 * half
    codes = codes.contiguous()
    scales = scales.contiguous()
    buf, need = _alloc_packed(n, k, codes.device, out)
    desc = nvfp4_weight()
    _check("nvfp4_pack", lib().nvfp4_pack(_ptr(codes), _ptr(scales), float(global_scale), n, k,
                                          _ptr(buf), buf.numel(), ctypes.byref(desc), _stream(codes.device)))
    return PackedWeight(buf, desc)


def nvfp4_unpack(w: PackedWeight):
    """-> (codes uint8 [n, k/2], scales uint8 [n, k/16], s_g float32 [1]) on the device."""
    codes = torch.empty((w.n, w.k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((w.n, w.k // 16), dtype=torch.uint8, device=w.device)
    sg = torch.empty(1, dtype=torch.float32, device=w.device)
    _check("nvfp4_unpack", lib().nvfp4_unpack(ctypes.byref(w.desc), _ptr(codes), _ptr(scales), _ptr(sg),
                                              _stream(w.device)))
    return codes, scales, sg


def nvfp4_dequant(w: PackedWeight) -> torch.Tensor:
    out = torch.empty((w.n, w.k), dtype=torch.float32, device=w.device)
    _check("nvfp4_dequant", lib().nvfp4_dequant(ctypes.byref(w.desc), _ptr(out), _stream(w.device)))
    return out


def nvfp4_quantize_workspace_bytes(n: int, k: int) -> int:
    return int(lib().nvfp4_quantize_workspace_bytes(n, k))


def nvfp4_quantize(W: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> PackedWeight:
    """fp32 weights [n, k] on the device -> PackedWeight (quantized on the GPU)."""
    if W.dtype != torch.float32:
        raise TypeError("W must be float32")
    W = W.contiguous()
    n, k = W.shape
    buf, need = _alloc_packed(n, k, W.device, out)
    wneed = nvfp4_quantize_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(wneed, dtype=torch.uint8, device=W.device)
    desc = nvfp4_weight()
    _check("nvfp4_quantize", lib().nvfp4_quantize(_ptr(W), n, k, _ptr(buf), buf.numel(), _ptr(workspace),
                                                  workspace.numel(), ctypes.byref(desc), _stream(W.device)))
    return PackedWeight(buf, desc)


def nvfp4_workspace_bytes(n: int, k: int, rows: int, dual: bool = False) -> int:
    return int(lib().nvfp4_workspace_bytes(n, k, rows, int(bool(dual))))


# Zeroed split-K workspaces, one per (device, stream): every call leaves its
# arrival counters at zero, so a workspace is reusable by later calls on the
# same stream.
_ws_cache: dict = {}
_ws_lock = threading.Lock()


def _workspace(device, need: int) -> torch.Tensor | None:
    if need == 0:
        return None
    key = (device, _stream(device))
    with _ws_lock:
        t = _ws_cache.get(key)
        if t is None or t.numel() < need:
            t = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
            _ws_cache[key] = t
        return t


_OUT = {torch.bfloat16: NVFP4_OUT_BF16, torch.float32: NVFP4_OUT_F32}


def _gemv_common(x, rows_k, out_dtype, out, n):
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if out_dtype not in _OUT:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    x = x.contiguous()
    rows = x.shape[0]
    if out is None:
        out = torch.empty((rows, n), dtype=out_dtype, device=x.device)
    return x, rows, out


def nvfp4_gemv(w: PackedWeight, x: torch.Tensor, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[rows, n] = x[rows, k] @ dequant(w)^T (fp32 accumulation)."""
    x, rows, out = _gemv_common(x, None, out_dtype, out, w.n)
    need = nvfp4_workspace_bytes(w.n, w.k, rows, False)
    if workspace is None:
        workspace = _workspace(x.device, need)
    _check("nvfp4_gemv", lib().nvfp4_gemv(ctypes.byref(w.desc), _ptr(x), rows, _ptr(out), _OUT[out.dtype],
                                          _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                          _stream(x.device)))
    return out


def nvfp4_gemv_noalloc(w: PackedWeight, x: torch.Tensor, out_dtype=torch.bfloat16,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_gemv with the library's static per-device scratch as its workspace
    (no device allocation by the library; ``out`` may be given so that nothing
    is allocated here either)."""
    x, rows, out = _gemv_common(x, None, out_dtype, out, w.n)
    _check("nvfp4_gemv_noalloc", lib().nvfp4_gemv_noalloc(ctypes.byref(w.desc), _ptr(x), rows, _ptr(out),
                                                          _OUT[out.dtype], _stream(x.device)))
    return out


def nvfp4_gemv_dual_silu(gate: PackedWeight, up: PackedWeight, x: torch.Tensor, out_dtype=torch.bfloat16,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """o[rows, n] = silu(x @ gate^T) * (x @ up^T)."""
    x, rows, out = _gemv_common(x, None, out_dtype, out, gate.n)
    need = nvfp4_workspace_bytes(gate.n, gate.k, rows, True)
    if workspace is None:
        workspace = _workspace(x.device, need)
    _check("nvfp4_gemv_dual_silu",
           lib().nvfp4_gemv_dual_silu(ctypes.byref(gate.desc), ctypes.byref(up.desc), _ptr(x), rows, _ptr(out),
                                      _OUT[out.dtype], _ptr(workspace),
                                      0 if workspace is None else workspace.numel(), _stream(x.device)))
    return out


def nvfp4_dense_gemv_bf16(W: torch.Tensor, x: torch.Tensor, out_dtype=torch.bfloat16,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """y[rows, n] = x[rows, k] @ W[n, k]^T with bf16 W (the lm head), fp32
    accumulation."""
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise TypeError("W must be a 2-D bfloat16 tensor")
    W = W.contiguous()
    n, k = W.shape
    x, rows, out = _gemv_common(x, None, out_dtype, out, n)
    _check("nvfp4_dense_gemv_bf16",
           lib().nvfp4_dense_gemv_bf16(_ptr(W), n, k, _ptr(x), rows, _ptr(out), _OUT[out.dtype],
                                       _stream(x.device)))
    return out


def nvfp4_mxfp4_gemv(codes: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, out_dtype=torch.bfloat16,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """MXFP4 projection: codes uint8 [n, k/2] (low nibble first), scales uint8
    [n, k/32] (E8M0), x bf16 [rows, k] -> y [rows, n]."""
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or codes.dim() != 2:
        raise TypeError("codes and scales must be 2-D uint8 tensors")
    codes, scales = codes.contiguous(), scales.contiguous()
    n, k = codes.shape[0], codes.shape[1] * 2
    if tuple(scales.shape) != (n, k // 32):
        raise ValueError("scales must be [n, k/32]")
    x, rows, out = _gemv_common(x, None, out_dtype, out, n)
    _check("nvfp4_mxfp4_gemv",
           lib().nvfp4_mxfp4_gemv(_ptr(codes), _ptr(scales), n, k, _ptr(x), rows, _ptr(out), _OUT[out.dtype],
                                  _stream(x.device)))
    return out


def nvfp4_w8g32_gemv(codes: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, out_dtype=torch.bfloat16,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """W8G32_F16S projection: codes int8 [n, k], scales float16 [n, k/32], x
    bf16 [rows, k] -> y [rows, n]."""
    if codes.dtype != torch.int8 or scales.dtype != torch.float16 or codes.dim() != 2:
        raise TypeError("codes must be a 2-D int8 tensor and scales float16")
    codes, scales = codes.contiguous(), scales.contiguous()
    n, k = codes.shape
    if tuple(scales.shape) != (n, k // 32):
        raise ValueError("scales must be [n, k/32]")
    x, rows, out = _gemv_common(x, None, out_dtype, out, n)
    _check("nvfp4_w8g32_gemv",
           lib().nvfp4_w8g32_gemv(_ptr(codes), _ptr(scales), n, k, _ptr(x), rows, _ptr(out), _OUT[out.dtype],
                                  _stream(x.device)))
    return out


def nvfp4_residual_rmsnorm(residual: torch.Tensor, delta: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6,
                           gemma_offset: bool = False, residual_out: torch.Tensor | None = None,
                           x: torch.Tensor | None = None):
    """residual_out = bf16(residual + delta); x = RMSNorm(residual_out) * w'
    (w' = weight, or 1 + weight with the Gemma offset).  Returns
    (residual_out, x); pass residual_out=residual to update it in place."""
    for name, t in (("residual", residual), ("delta", delta), ("weight", weight)):
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be bfloat16" % name)
    residual, delta, weight = residual.contiguous(), delta.contiguous(), weight.contiguous()
    rows, k = residual.shape
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if x is None:
        x = torch.empty_like(residual)
    _check("nvfp4_residual_rmsnorm",
           lib().nvfp4_residual_rmsnorm(_ptr(residual), _ptr(delta), _ptr(weight), k, rows, float(eps),
                                        int(bool(gemma_offset)), _ptr(residual_out), _ptr(x),
                                        _stream(residual.device)))
    return residual_out, x


def nvfp4_read_ceiling(buf: torch.Tensor, nbytes: int | None = None, sink: torch.Tensor | None = None,
                       offset: int = 0) -> torch.Tensor:
    """Read ``nbytes`` of ``buf`` (a device tensor) from byte ``offset`` once
    with the projection kernel's launch shape: the streaming-read ceiling.
    Returns the 256-word sink."""
    size = buf.numel() * buf.element_size()
    nb = size - offset if nbytes is None else nbytes
    if offset < 0 or nb < 0 or offset + nb > size:
        raise ValueError("nvfp4_read_ceiling: bytes [%d, %d) are not inside the %d-byte buffer"
                         % (offset, offset + nb, size))
    if sink is None:
        sink = torch.empty(256, dtype=torch.int32, device=buf.device)
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("nvfp4_read_ceiling: the sink must hold 256 32-bit words")
    _check("nvfp4_read_ceiling", lib().nvfp4_read_ceiling(buf.data_ptr() + offset, nb, sink.data_ptr(),
                                                          _stream(buf.device)))
    return sink


NVFP4_WS_STATE_BYTES = 161 << 10   # counters and wait words at the start of a workspace


def counters_clear(workspace: torch.Tensor) -> bool:
    """Whether the workspace's counters and wait words (its first
    NVFP4_WS_STATE_BYTES) are all zero, as every launch leaves them.
    Synchronizes with the device."""
    return not bool(workspace[:NVFP4_WS_STATE_BYTES].any())


def wait_flag(workspace: torch.Tensor) -> int:
    """The workspace's wait flag (nonzero: a bounded wait of a launch gave up,
    between its calls or between the waves of a workgroup); synchronizes with
    the device to read it."""
    off = NVFP4_WS_WAIT_FLAG_OFFSET
    if workspace.numel() < off + 4:
        return 0
    return int(workspace[off:off + 4].view(torch.int32).item())


class Norm:
    """A residual add + RMSNorm call of a Sequence: residual_out = bf16(residual
    + delta), x = RMSNorm(residual_out) * w' (w' = weight, or 1 + weight with
    the Gemma offset); residual_out defaults to residual (updated in place).
    All bf16 device tensors: residual, delta, residual_out, x [rows, k];
    weight [k]."""

    def __init__(self, residual: torch.Tensor, delta: torch.Tensor, weight: torch.Tensor, x: torch.Tensor,
                 residual_out: torch.Tensor | None = None, eps: float = 1e-6, gemma_offset: bool = False):
        self.residual, self.delta, self.weight, self.x = residual, delta, weight, x
        self.residual_out = residual if residual_out is None else residual_out
        for name in ("residual", "delta", "weight", "x", "residual_out"):
            t = getattr(self, name)
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise TypeError("%s must be a contiguous bfloat16 tensor" % name)
        self.desc = nvfp4_norm(residual.data_ptr(), delta.data_ptr(), weight.data_ptr(),
                               self.residual_out.data_ptr(), residual.shape[-1], float(eps),
                               int(bool(gemma_offset)))


class Sequence:
    """A prepared list of calls (the projections of a decode step, and the
    residual add + RMSNorm between them), built once and enqueued with one
    native call each time it runs.

    ``calls``: iterable of (weight, up_or_None, x, y) with x bf16 [rows, k] and y
    [rows, n] (bf16 or fp32) device tensors, or Norm objects; a call may take
    an earlier call's y as its x (a Norm: its x as a projection's x, its
    residual_out as a later Norm's residual, a projection's y as its delta).
    """

    def __init__(self, calls):
        calls = list(calls)
        self._keep = []
        self.n = len(calls)
        self._arr = (nvfp4_call * max(self.n, 1))()
        for i, item in enumerate(calls):
            c = self._arr[i]
            if isinstance(item, Norm):
                c.w = c.up = None
                c.x = None
                c.y = item.x.data_ptr()
                c.rows = item.residual.shape[0]
                c.out_dtype = NVFP4_OUT_BF16
                c.norm = ctypes.pointer(item.desc)
                self._keep.append((None, None, item.residual, item))
                continue
            w, up, x, y = item
            if x.dtype != torch.bfloat16 or y.dtype not in _OUT:
                raise TypeError("call %d: x must be bfloat16 and y bfloat16 or float32" % i)
            if x.dim() != 2 or x.shape[1] != w.k or tuple(y.shape) != (x.shape[0], w.n):
                raise ValueError("call %d: x must be [rows, %d] and y [rows, %d]" % (i, w.k, w.n))
            if not (x.is_contiguous() and y.is_contiguous()):
                raise ValueError("call %d: x and y must be contiguous" % i)
            c.w = ctypes.pointer(w.desc)
            c.up = ctypes.pointer(up.desc) if up is not None else None
            c.x = x.data_ptr()
            c.y = y.data_ptr()
            c.rows = x.shape[0]
            c.out_dtype = _OUT[y.dtype]
            c.norm = None
            self._keep.append((w, up, x, y))
        self.workspace_bytes = int(lib().nvfp4_sequence_workspace_bytes(self._arr, self.n))
        # kernel launches of one launch() without events, and the waits
        # between calls inside them (on a device with cooperative launches)
        self.launches = int(lib().nvfp4_sequence_launches(self._arr, self.n))
        self.waits = int(lib().nvfp4_sequence_waits(self._arr, self.n)) if self.n else 0
        # validated once: launch() enqueues the plan (nvfp4_sequence_plan_launch)
        self._plan = None
        if self.n:
            nb = int(lib().nvfp4_sequence_plan_bytes(self._arr, self.n))   # 0: a call is invalid
            self._plan = (ctypes.c_uint64 * (-(-nb // 8) + 2))()
            base = ctypes.addressof(self._plan)
            self._plan_ptr = base + (-base % 16)
            _check("nvfp4_sequence_plan", lib().nvfp4_sequence_plan(self._arr, self.n, self._plan_ptr, nb))

    def launch(self, workspace: torch.Tensor | None = None, events=None, stream=None):
        """Enqueue every call on ``stream`` (default: the current stream).
        ``events``: None or a list of 2*n raw hipEvent_t handles (or None); with
        events, every call gets a kernel launch of its own."""
        dev = self._keep[0][2].device if self._keep else torch.device("cuda")
        if workspace is None:
            workspace = _workspace(dev, self.workspace_bytes)
        ev = None
        if events is not None:
            if len(events) != 2 * self.n:
                raise ValueError("events must hold 2 entries per call")
            ev = (ctypes.c_void_p * (2 * self.n))(*[e if e else None for e in events])
        st = stream if stream is not None else _stream(dev)
        wsb = 0 if workspace is None else workspace.numel()
        if ev is None and self._plan is not None:
            _check("nvfp4_sequence_plan_launch",
                   lib().nvfp4_sequence_plan_launch(self._plan_ptr, _ptr(workspace), wsb, st))
            return
        _check("nvfp4_gemv_sequence", lib().nvfp4_gemv_sequence(self._arr, self.n, _ptr(workspace), wsb, ev, st))


def nvfp4_sequence_workspace_bytes(calls) -> int:
    return Sequence(calls).workspace_bytes


def nvfp4_sequence_launches(calls) -> int:
    return Sequence(calls).launches


def nvfp4_gemv_sequence(calls, workspace: torch.Tensor | None = None, events=None) -> None:
    """One-shot form of Sequence(calls).launch(...)."""
    Sequence(calls).launch(workspace, events)
