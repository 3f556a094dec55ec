"""MI355X (gfx950) NVFP4 weight-only GEMM library -- Python binding.

The compute lives in ``libnvfp4.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/nvfp4.h``).  This module only marshals torch tensors
(device memory and streams) into that ABI.  There is no fallback: if the
library is missing, importing the binding's functions raises.

Low-level functions carry the C names (``nvfp4_quantize``, ``nvfp4_gemm``,
``nvfp4_grouped_gemm``, ...) and take every buffer explicitly; ``quantize``,
``gemm`` and ``grouped_gemm`` allocate outputs and a cached workspace.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

OK = 0
STATUS_NAMES = {0: "NVFP4_OK", 1: "NVFP4_ERR_INVALID_ARGUMENT", 2: "NVFP4_ERR_MISALIGNED",
                3: "NVFP4_ERR_UNSUPPORTED", 4: "NVFP4_ERR_WORKSPACE", 5: "NVFP4_ERR_HIP"}
OUT_BF16 = 0
OUT_F32 = 1
DSTATUS_NONFINITE = 1
DSTATUS_BAD_OFFSETS = 2
DSTATUS_BAD_INDEX = 4
DSTATUS_WAIT_TIMEOUT = 8
MAX_EXPERTS = 1024

EXPORTED = [
    "nvfp4_quantize", "nvfp4_gemm", "nvfp4_grouped_gemm", "nvfp4_grouped_gemm_swiglu",
    "nvfp4_grouped_gemm_gather", "nvfp4_grouped_mlp", "nvfp4_grouped_mlp_workspace_size",
    "nvfp4_grouped_mlp_kernel_name", "nvfp4_moe_combine", "nvfp4_gemm_w4a4",
    "nvfp4_grouped_gemm_w4a4", "nvfp4_gemm_noalloc", "nvfp4_gemm_w4a4_workspace_size",
    "nvfp4_grouped_gemm_w4a4_workspace_size",
    "nvfp4_quantize_workspace_size",
    "nvfp4_gemm_workspace_size", "nvfp4_grouped_gemm_workspace_size",
    "nvfp4_workspace_counter_bytes", "nvfp4_workspace_init", "nvfp4_status_string",
    "nvfp4_kernel_name",
    "nvfp4_version",
]

_lib = None
_lock = threading.Lock()


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s" % (what, STATUS_NAMES.get(status, str(status))))
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libnvfp4.so and declare its C signatures.  Raises OSError if the
    library has not been built (``python -m block_scaled_fp4_nibble_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise OSError("libnvfp4.so not found at %s; build it with "
                          "`python -m block_scaled_fp4_nibble_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I64, SZ, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        lib.nvfp4_quantize.argtypes = [P, I64, I64, I64, P, P, P, P, P, SZ, P]
        lib.nvfp4_quantize.restype = I32
        lib.nvfp4_gemm.argtypes = [P, I64, I64, I64, P, P, P, P, I32, P, SZ, P]
        lib.nvfp4_gemm.restype = I32
        lib.nvfp4_grouped_gemm.argtypes = [P, I64, P, I64, I64, I64, P, P, P, P, I32, P, P, SZ, P]
        lib.nvfp4_grouped_gemm.restype = I32
        lib.nvfp4_grouped_gemm_swiglu.argtypes = [P, I64, P, I64, I64, I64, P, P, P, P, I32, P, P,
                                                  SZ, P]
        lib.nvfp4_grouped_gemm_swiglu.restype = I32
        lib.nvfp4_grouped_gemm_gather.argtypes = [P, I64, P, I64, P, I64, I64, I64, P, P, P, P,
                                                  I32, I32, P, P, SZ, P]
        lib.nvfp4_grouped_gemm_gather.restype = I32
        lib.nvfp4_grouped_mlp.argtypes = [P, I64, P, I64, I64, I64, P, P, P, P, P, P, P, P, I32,
                                          P, P, SZ, P]
        lib.nvfp4_grouped_mlp.restype = I32
        lib.nvfp4_grouped_mlp_workspace_size.argtypes = [I64, I64, I64, I64]
        lib.nvfp4_grouped_mlp_workspace_size.restype = SZ
        lib.nvfp4_grouped_mlp_kernel_name.argtypes = [I64, I64, I64, I64]
        lib.nvfp4_grouped_mlp_kernel_name.restype = ctypes.c_char_p
        lib.nvfp4_moe_combine.argtypes = [P, I32, I64, P, P, I64, I64, I64, P, I32, P, P]
        lib.nvfp4_moe_combine.restype = I32
        lib.nvfp4_gemm_w4a4.argtypes = [P, P, P, I64, I64, I64, P, P, P, P, I32, P, SZ, P]
        lib.nvfp4_gemm_w4a4.restype = I32
        lib.nvfp4_grouped_gemm_w4a4.argtypes = [P, P, P, I64, P, I64, I64, I64, P, P, P, P, I32,
                                                P, P, SZ, P]
        lib.nvfp4_grouped_gemm_w4a4.restype = I32
        lib.nvfp4_gemm_noalloc.argtypes = [P, I64, I64, I64, P, P, P, P, I32, P]
        lib.nvfp4_gemm_noalloc.restype = I32
        lib.nvfp4_gemm_w4a4_workspace_size.argtypes = [I64, I64, I64]
        lib.nvfp4_gemm_w4a4_workspace_size.restype = SZ
        lib.nvfp4_grouped_gemm_w4a4_workspace_size.argtypes = [I64, I64, I64, I64]
        lib.nvfp4_grouped_gemm_w4a4_workspace_size.restype = SZ
        lib.nvfp4_quantize_workspace_size.argtypes = [I64, I64, I64]
        lib.nvfp4_quantize_workspace_size.restype = SZ
        lib.nvfp4_gemm_workspace_size.argtypes = [I64, I64, I64]
        lib.nvfp4_gemm_workspace_size.restype = SZ
        lib.nvfp4_grouped_gemm_workspace_size.argtypes = [I64, I64, I64, I64]
        lib.nvfp4_grouped_gemm_workspace_size.restype = SZ
        lib.nvfp4_workspace_counter_bytes.argtypes = []
        lib.nvfp4_workspace_counter_bytes.restype = SZ
        lib.nvfp4_workspace_init.argtypes = [P, SZ, P]
        lib.nvfp4_workspace_init.restype = I32
        lib.nvfp4_kernel_name.argtypes = [I64, I64, I64, I64, I32, I32]
        lib.nvfp4_kernel_name.restype = ctypes.c_char_p
        lib.nvfp4_status_string.argtypes = [I32]
        lib.nvfp4_status_string.restype = ctypes.c_char_p
        lib.nvfp4_version.argtypes = []
        lib.nvfp4_version.restype = I32
        _lib = lib
        return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream=None):
    """The stream handle to pass: the given torch stream, else the current
    stream of the current device (through torch's raw-handle query, which
    costs a fraction of building a torch.cuda.Stream object per call)."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, what: str):
    if status != OK:
        raise NVFP4Error(status, what)


# ---- raw C entry points (explicit buffers) ---------------------------------

def nvfp4_quantize(w, batch, n, k, packed, scales, global_scale, d_status, workspace,
                   ws_bytes, stream=None):
    return load_library().nvfp4_quantize(_ptr(w), batch, n, k, _ptr(packed), _ptr(scales),
                                         _ptr(global_scale), _ptr(d_status), _ptr(workspace),
                                         ws_bytes, _stream(stream))


def nvfp4_gemm(x, m, n, k, packed, scales, global_scale, y, out, workspace, ws_bytes,
               stream=None):
    return load_library().nvfp4_gemm(_ptr(x), m, n, k, _ptr(packed), _ptr(scales),
                                     _ptr(global_scale), _ptr(y), out, _ptr(workspace), ws_bytes,
                                     _stream(stream))


def nvfp4_gemm_noalloc(x, m, n, k, packed, scales, global_scale, y, out, stream=None):
    return load_library().nvfp4_gemm_noalloc(_ptr(x), m, n, k, _ptr(packed), _ptr(scales),
                                             _ptr(global_scale), _ptr(y), out, _stream(stream))


def nvfp4_grouped_gemm(x, rows, offsets, num_experts, n, k, packed, scales, global_scales, y,
                       out, d_status, workspace, ws_bytes, stream=None):
    return load_library().nvfp4_grouped_gemm(_ptr(x), rows, _ptr(offsets), num_experts, n, k,
                                             _ptr(packed), _ptr(scales), _ptr(global_scales),
                                             _ptr(y), out, _ptr(d_status), _ptr(workspace),
                                             ws_bytes, _stream(stream))


def nvfp4_moe_combine(y, y_type, rows, token_rows, weights, tokens, topk, n, out, out_type,
                      d_status, stream=None):
    return load_library().nvfp4_moe_combine(_ptr(y), y_type, rows, _ptr(token_rows),
                                            _ptr(weights), tokens, topk, n, _ptr(out), out_type,
                                            _ptr(d_status), _stream(stream))


def nvfp4_grouped_gemm_gather(x, x_rows, row_index, rows, offsets, num_experts, n, k, packed,
                              scales, global_scales, y, out, act, d_status, workspace, ws_bytes,
                              stream=None):
    return load_library().nvfp4_grouped_gemm_gather(
        _ptr(x), x_rows, _ptr(row_index), rows, _ptr(offsets), num_experts, n, k, _ptr(packed),
        _ptr(scales), _ptr(global_scales), _ptr(y), out, act, _ptr(d_status), _ptr(workspace),
        ws_bytes, _stream(stream))


def nvfp4_grouped_gemm_swiglu(x, rows, offsets, num_experts, n, k, packed, scales,
                              global_scales, h, out, d_status, workspace, ws_bytes, stream=None):
    return load_library().nvfp4_grouped_gemm_swiglu(
        _ptr(x), rows, _ptr(offsets), num_experts, n, k, _ptr(packed), _ptr(scales),
        _ptr(global_scales), _ptr(h), out, _ptr(d_status), _ptr(workspace), ws_bytes,
        _stream(stream))


def nvfp4_grouped_mlp(x, rows, offsets, num_experts, d_model, d_ff, up_packed, up_scales,
                      up_global, down_packed, down_scales, down_global, h, y, out, d_status,
                      workspace, ws_bytes, stream=None):
    return load_library().nvfp4_grouped_mlp(
        _ptr(x), rows, _ptr(offsets), num_experts, d_model, d_ff, _ptr(up_packed),
        _ptr(up_scales), _ptr(up_global), _ptr(down_packed), _ptr(down_scales),
        _ptr(down_global), _ptr(h), _ptr(y), out, _ptr(d_status), _ptr(workspace), ws_bytes,
        _stream(stream))


def nvfp4_grouped_mlp_workspace_size(rows, num_experts, d_model, d_ff) -> int:
    return load_library().nvfp4_grouped_mlp_workspace_size(rows, num_experts, d_model, d_ff)


def nvfp4_grouped_mlp_kernel_name(rows, num_experts, d_model, d_ff) -> str:
    return load_library().nvfp4_grouped_mlp_kernel_name(rows, num_experts, d_model,
                                                        d_ff).decode()


def nvfp4_quantize_workspace_size(batch, n, k) -> int:
    return load_library().nvfp4_quantize_workspace_size(batch, n, k)


def nvfp4_gemm_workspace_size(m, n, k) -> int:
    return load_library().nvfp4_gemm_workspace_size(m, n, k)


def nvfp4_grouped_gemm_workspace_size(rows, num_experts, n, k) -> int:
    return load_library().nvfp4_grouped_gemm_workspace_size(rows, num_experts, n, k)


def nvfp4_gemm_w4a4_workspace_size(m, n, k) -> int:
    return load_library().nvfp4_gemm_w4a4_workspace_size(m, n, k)


def nvfp4_grouped_gemm_w4a4_workspace_size(rows, num_experts, n, k) -> int:
    return load_library().nvfp4_grouped_gemm_w4a4_workspace_size(rows, num_experts, n, k)


def nvfp4_gemm_w4a4(x_packed, x_scales, x_g, m, n, k, packed, scales, global_scale, y, out,
                    workspace, ws_bytes, stream=None):
    return load_library().nvfp4_gemm_w4a4(
        _ptr(x_packed), _ptr(x_scales), _ptr(x_g), m, n, k, _ptr(packed), _ptr(scales),
        _ptr(global_scale), _ptr(y), out, _ptr(workspace), ws_bytes, _stream(stream))


def nvfp4_grouped_gemm_w4a4(x_packed, x_scales, x_g, rows, offsets, num_experts, n, k, packed,
                            scales, global_scales, y, out, d_status, workspace, ws_bytes,
                            stream=None):
    return load_library().nvfp4_grouped_gemm_w4a4(
        _ptr(x_packed), _ptr(x_scales), _ptr(x_g), rows, _ptr(offsets), num_experts, n, k,
        _ptr(packed), _ptr(scales), _ptr(global_scales), _ptr(y), out, _ptr(d_status),
        _ptr(workspace), ws_bytes, _stream(stream))


def nvfp4_workspace_counter_bytes() -> int:
    return load_library().nvfp4_workspace_counter_bytes()


def nvfp4_workspace_init(workspace, ws_bytes, stream=None):
    return load_library().nvfp4_workspace_init(_ptr(workspace), ws_bytes, _stream(stream))


def nvfp4_kernel_name(rows, num_experts, n, k, grouped, gather=0) -> str:
    return load_library().nvfp4_kernel_name(rows, num_experts, n, k, int(grouped),
                                            int(gather)).decode()


def nvfp4_status_string(status: int) -> str:
    return load_library().nvfp4_status_string(status).decode()


def nvfp4_version() -> int:
    return load_library().nvfp4_version()


# ---- convenience layer --------------------------------------------------------

@dataclass
class QuantizedWeight:
    """NVFP4 weight: packed [.., n, k/2] uint8, scales [.., n, k/16] uint8
    (E4M3 bits), global_scale [batch] float32 -- all on one device."""
    packed: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor

    @property
    def n(self) -> int:
        return self.packed.shape[-2]

    @property
    def k(self) -> int:
        return self.packed.shape[-1] * 2


class Workspace:
    """Device workspaces for the convenience layer, one per (device, stream):
    calls on different streams never share split-K counters (the C contract:
    calls that may run concurrently need separate workspaces).

    Eager calls grow a stream's buffer as shapes grow and zero its counter
    region once at allocation (the kernels leave it zeroed after every call).
    An outgrown buffer is kept alive, because a HIP graph captured earlier may
    still hold its address.  Calls made while the stream is being captured get
    a fresh buffer of their own whose counter zeroing is recorded in the graph
    (a fill kernel, so it runs at every replay); such buffers are never handed
    to eager calls, whose counters could otherwise be read before the first
    replay zeroed them, and are kept alive as long as the process."""

    def __init__(self):
        self._buf = {}
        self._keep = []
        self._lock = threading.Lock()

    def get(self, nbytes: int, device, stream=None):
        if nbytes == 0:
            return None
        dev = torch.device(device).index
        handle = _stream(stream).value or 0
        if torch.cuda.is_current_stream_capturing():
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _check(nvfp4_workspace_init(buf, buf.numel(), stream), "nvfp4_workspace_init")
            with self._lock:
                self._keep.append(buf)
            return buf
        key = (dev, handle)
        with self._lock:
            buf = self._buf.get(key)
            if buf is None or buf.numel() < nbytes:
                new = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
                _check(nvfp4_workspace_init(new, new.numel(), stream), "nvfp4_workspace_init")
                if buf is not None:
                    self._keep.append(buf)
                self._buf[key] = buf = new
            return buf


_gemm_ws = Workspace()
_quant_ws = Workspace()


def _bf16_2d_or_3d(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError("%s must be a CUDA/HIP bfloat16 tensor" % name)
    return t.contiguous()


def quantize(w: torch.Tensor, d_status: torch.Tensor | None = None, stream=None) -> QuantizedWeight:
    """Encode BF16 weights [n, k] or [batch, n, k] to NVFP4 on the GPU."""
    w = _bf16_2d_or_3d(w, "w")
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    if w3.dim() != 3:
        raise ValueError("w must be [n, k] or [batch, n, k]")
    b, n, k = w3.shape
    dev = w.device
    packed = torch.empty((b, n, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((b, n, k // 16), dtype=torch.uint8, device=dev)
    g = torch.empty((b,), dtype=torch.float32, device=dev)
    nbytes = nvfp4_quantize_workspace_size(b, n, k)
    ws = _quant_ws.get(nbytes, dev, stream)
    _check(nvfp4_quantize(w3, b, n, k, packed, scales, g, d_status, ws, nbytes, stream),
           "nvfp4_quantize")
    if squeeze:
        return QuantizedWeight(packed[0], scales[0], g)
    return QuantizedWeight(packed, scales, g)


def gemm(x: torch.Tensor, qw: QuantizedWeight, out_dtype=torch.bfloat16,
         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [m, n] = x [m, k] (bf16) @ dequant(qw)^T."""
    x = _bf16_2d_or_3d(x, "x")
    m, k = x.shape
    n = qw.packed.shape[-2]
    if qw.packed.dim() != 2 or qw.k != k:
        raise ValueError("weight must be a single [n, k/2] tensor matching x")
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    nbytes = nvfp4_gemm_workspace_size(m, n, k)
    ws = _gemm_ws.get(nbytes, x.device, stream)
    _check(nvfp4_gemm(x, m, n, k, qw.packed, qw.scales, qw.global_scale, out, code, ws,
                      nbytes, stream), "nvfp4_gemm")
    return out


def grouped_gemm(x: torch.Tensor, offsets: torch.Tensor, qw: QuantizedWeight,
                 out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                 d_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Rows [offsets[e], offsets[e+1]) of x times expert e's weight.  Rows of
    the output that belong to no expert are left as allocated."""
    x = _bf16_2d_or_3d(x, "x")
    rows, k = x.shape
    if qw.packed.dim() != 3 or qw.k != k:
        raise ValueError("weight must be [E, n, k/2] matching x")
    E, n, _ = qw.packed.shape
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int32 tensor of E+1 entries")
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out is None:
        out = torch.empty((rows, n), dtype=out_dtype, device=x.device)
    nbytes = nvfp4_grouped_gemm_workspace_size(rows, E, n, k)
    ws = _gemm_ws.get(nbytes, x.device, stream)
    _check(nvfp4_grouped_gemm(x, rows, offsets.contiguous(), E, n, k, qw.packed, qw.scales,
                              qw.global_scale, out, code, d_status, ws, nbytes, stream),
           "nvfp4_grouped_gemm")
    return out


def grouped_gemm_swiglu(x: torch.Tensor, offsets: torch.Tensor, qw: QuantizedWeight,
                        out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                        d_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """h [rows, n/2] = SiLU(gate) * up of the grouped gate_up product, the
    weight's rows in 32-row groups of 16 gate rows then the 16 matching up
    rows (see nvfp4_grouped_gemm_swiglu in include/nvfp4.h)."""
    x = _bf16_2d_or_3d(x, "x")
    rows, k = x.shape
    if qw.packed.dim() != 3 or qw.k != k:
        raise ValueError("weight must be [E, n, k/2] matching x")
    E, n, _ = qw.packed.shape
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int32 tensor of E+1 entries")
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out is None:
        out = torch.empty((rows, n // 2), dtype=out_dtype, device=x.device)
    nbytes = nvfp4_grouped_gemm_workspace_size(rows, E, n, k)
    ws = _gemm_ws.get(nbytes, x.device, stream)
    _check(nvfp4_grouped_gemm_swiglu(x, rows, offsets.contiguous(), E, n, k, qw.packed,
                                     qw.scales, qw.global_scale, out, code, d_status, ws, nbytes,
                                     stream),
           "nvfp4_grouped_gemm_swiglu")
    return out


def grouped_mlp(x: torch.Tensor, offsets: torch.Tensor, qw_up: QuantizedWeight,
                qw_down: QuantizedWeight, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                h: torch.Tensor | None = None, d_status: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """y [rows, d_model] = grouped_gemm(grouped_gemm_swiglu(x, qw_up), qw_down) in
    one persistent launch (see nvfp4_grouped_mlp in include/nvfp4.h); the
    intermediate goes to h [rows, d_ff] (allocated when not given).  Raises
    NVFP4Error(UNSUPPORTED) for shapes the fused launch does not take."""
    x = _bf16_2d_or_3d(x, "x")
    rows, d_model = x.shape
    if qw_up.packed.dim() != 3 or qw_up.k != d_model or qw_down.packed.dim() != 3:
        raise ValueError("weights must be [E, n, k/2]; the up weight's k must match x")
    E, n_up, _ = qw_up.packed.shape
    d_ff = n_up // 2
    if qw_down.packed.shape[0] != E or qw_down.n != d_model or qw_down.k != d_ff:
        raise ValueError("down weight must be [E, d_model, d_ff/2]")
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int32 tensor of E+1 entries")
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out is None:
        out = torch.empty((rows, d_model), dtype=out_dtype, device=x.device)
    if h is None:
        h = torch.empty((rows, d_ff), dtype=torch.bfloat16, device=x.device)
    nbytes = nvfp4_grouped_mlp_workspace_size(rows, E, d_model, d_ff)
    ws = _gemm_ws.get(nbytes, x.device, stream)
    _check(nvfp4_grouped_mlp(x, rows, offsets.contiguous(), E, d_model, d_ff, qw_up.packed,
                             qw_up.scales, qw_up.global_scale, qw_down.packed, qw_down.scales,
                             qw_down.global_scale, h, out, code, d_status, ws, nbytes, stream),
           "nvfp4_grouped_mlp")
    return out


def grouped_gemm_gather(x: torch.Tensor, row_index: torch.Tensor, offsets: torch.Tensor,
                        qw: QuantizedWeight, act: str = "none", out_dtype=torch.bfloat16,
                        out: torch.Tensor | None = None, d_status: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Grouped GEMM over routed rows gathered from the token matrix x
    [tokens, k]: routed row r uses x[row_index[r]].  act="none" returns
    [rows, n]; act="swiglu" returns SiLU(gate) * up [rows, n/2]."""
    x = _bf16_2d_or_3d(x, "x")
    x_rows, k = x.shape
    if qw.packed.dim() != 3 or qw.k != k:
        raise ValueError("weight must be [E, n, k/2] matching x")
    E, n, _ = qw.packed.shape
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int32 tensor of E+1 entries")
    if row_index.dtype != torch.int32 or row_index.dim() != 1 or not row_index.is_cuda:
        raise ValueError("row_index must be a device int32 vector")
    rows = row_index.numel()
    if act not in ("none", "swiglu"):
        raise ValueError("act must be 'none' or 'swiglu'")
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    ncols = n // 2 if act == "swiglu" else n
    if out is None:
        out = torch.empty((rows, ncols), dtype=out_dtype, device=x.device)
    nbytes = nvfp4_grouped_gemm_workspace_size(rows, E, n, k)
    ws = _gemm_ws.get(nbytes, x.device, stream)
    _check(nvfp4_grouped_gemm_gather(x, x_rows, row_index.contiguous(), rows, offsets.contiguous(),
                                     E, n, k, qw.packed, qw.scales, qw.global_scale, out, code,
                                     1 if act == "swiglu" else 0, d_status, ws, nbytes, stream),
           "nvfp4_grouped_gemm_gather")
    return out


def moe_combine(y: torch.Tensor, token_rows: torch.Tensor, weights: torch.Tensor,
                out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                d_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out [tokens, n] = sum_j weights[t, j] * y[token_rows[t, j]] (router-weighted
    sum of each token's routed rows; negative ids are empty slots)."""
    if y.dtype not in (torch.bfloat16, torch.float32) or y.dim() != 2 or not y.is_cuda:
        raise ValueError("y must be a 2-D bf16 or float32 device tensor")
    if token_rows.dtype != torch.int32 or token_rows.dim() != 2 or not token_rows.is_cuda:
        raise ValueError("token_rows must be a [tokens, topk] device int32 tensor")
    if weights.dtype != torch.float32 or weights.shape != token_rows.shape or not weights.is_cuda:
        raise ValueError("weights must be a float32 device tensor shaped like token_rows")
    y = y.contiguous()
    rows, n = y.shape
    tokens, topk = token_rows.shape
    if out is None:
        out = torch.empty((tokens, n), dtype=out_dtype, device=y.device)
    _check(nvfp4_moe_combine(y, OUT_F32 if y.dtype == torch.float32 else OUT_BF16, rows,
                             token_rows.contiguous(), weights.contiguous(), tokens, topk, n, out,
                             OUT_F32 if out.dtype == torch.float32 else OUT_BF16, d_status,
                             stream), "nvfp4_moe_combine")
    return out


def gemm_w4a4(xq: QuantizedWeight, qw: QuantizedWeight, out_dtype=torch.bfloat16,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [m, n] = g_x g_w x_dec @ w_dec^T for activations in NVFP4 (xq, e.g.
    from quantize(x) of a [m, k] BF16 tensor) and an NVFP4 weight."""
    if xq.packed.dim() != 2 or qw.packed.dim() != 2 or xq.k != qw.k:
        raise ValueError("activations [m, k/2] and weight [n, k/2] with the same k")
    m, k, n = xq.packed.shape[0], xq.k, qw.n
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=xq.packed.device)
    nbytes = nvfp4_gemm_w4a4_workspace_size(m, n, k)
    ws = _gemm_ws.get(nbytes, xq.packed.device, stream)
    _check(nvfp4_gemm_w4a4(xq.packed, xq.scales, xq.global_scale, m, n, k, qw.packed, qw.scales,
                           qw.global_scale, out, code, ws, nbytes, stream), "nvfp4_gemm_w4a4")
    return out


def grouped_gemm_w4a4(xq: QuantizedWeight, offsets: torch.Tensor, qw: QuantizedWeight,
                      out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                      d_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Rows [offsets[e], offsets[e+1]) of the NVFP4 activations (one global
    scale for all rows) times expert e's NVFP4 weight."""
    if xq.packed.dim() != 2 or qw.packed.dim() != 3 or xq.k != qw.k:
        raise ValueError("activations [rows, k/2] and weight [E, n, k/2] with the same k")
    rows, k = xq.packed.shape[0], xq.k
    E, n, _ = qw.packed.shape
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int32 tensor of E+1 entries")
    code = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    if out is None:
        out = torch.empty((rows, n), dtype=out_dtype, device=xq.packed.device)
    nbytes = nvfp4_grouped_gemm_w4a4_workspace_size(rows, E, n, k)
    ws = _gemm_ws.get(nbytes, xq.packed.device, stream)
    _check(nvfp4_grouped_gemm_w4a4(xq.packed, xq.scales, xq.global_scale, rows,
                                   offsets.contiguous(), E, n, k, qw.packed, qw.scales,
                                   qw.global_scale, out, code, d_status, ws, nbytes, stream),
           "nvfp4_grouped_gemm_w4a4")
    return out

