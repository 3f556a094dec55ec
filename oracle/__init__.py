"""CPU oracle for the NVFP4 weight-only GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it,
and it imports nothing from the product package: the two share no code.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, IEEE binary32 for the
quantization decisions, double for the GEMM sums); this module only marshals
numpy arrays through ctypes.  The format facts it follows come from the page
"The Blackwell Architectural Split: NVFP4, Attention, and Consumer Silicon",
section "Preserving precision -- dual-tier scale handling" (1/2/1 bit split,
global scale plus one block scale per 16 values), and from the format
definition written out in the C file's header (E2M1 value set, E4M3 block
scale = block amax / 6, global scale = tensor amax / 2688).

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")

OK = 0
ERR_ARG = 1
ERR_NONFINITE = 2

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libnvfp4_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fno-finite-math-only", "-Wall", "-Wextra", "-shared", "-fPIC",
            _SRC, "-o", tmp, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [F]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e2m1_encode_mag.argtypes = [F]
    lib.orc_e2m1_encode_mag.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
    lib.orc_e2m1_encode_mag_array.argtypes = [P, I64, P]
    lib.orc_global_scale.argtypes = [F]
    lib.orc_global_scale.restype = F
    lib.orc_block_scale_code.argtypes = [F, F]
    lib.orc_block_scale_code.restype = ctypes.c_uint8
    lib.orc_element_code.argtypes = [F, F, F]
    lib.orc_element_code.restype = ctypes.c_uint8
    lib.orc_quantize.argtypes = [P, I64, I64, I64, P, P, P]
    lib.orc_quantize.restype = ctypes.c_int
    lib.orc_dequant.argtypes = [P, P, I64, I64, P]
    lib.orc_gemm.argtypes = [P, I64, I64, I64, P, P, F, P, P]
    lib.orc_gemm.restype = ctypes.c_int
    lib.orc_gemm_sampled.argtypes = [P, I64, I64, I64, P, P, F, P, P, I64, P, P]
    lib.orc_gemm_sampled.restype = ctypes.c_int
    lib.orc_grouped_gemm.argtypes = [P, I64, P, I64, I64, I64, P, P, P, P, P]
    lib.orc_grouped_gemm.restype = ctypes.c_int
    lib.orc_grouped_gemm_sampled.argtypes = [P, I64, P, I64, I64, I64, P, P, P, P, P, I64, P, P]
    lib.orc_grouped_gemm_sampled.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


# ---- format ---------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code (sign 0) of each non-negative float32: RNE, saturating."""
    x = _c(x, np.float32).reshape(-1)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def e2m1_encode_mag(q) -> np.ndarray:
    """3-bit E2M1 magnitude code of each non-negative float32: RNE, saturating."""
    q = _c(q, np.float32).reshape(-1)
    out = np.empty(q.shape, np.uint8)
    _load().orc_e2m1_encode_mag_array(_ptr(q), q.size, _ptr(out))
    return out


def global_scale(amax: float) -> float:
    return float(_load().orc_global_scale(float(amax)))


def block_scale_code(amax_b: float, g: float) -> int:
    return int(_load().orc_block_scale_code(float(amax_b), float(g)))


def element_code(w: float, s_dec: float, g: float) -> int:
    return int(_load().orc_element_code(float(w), float(s_dec), float(g)))


# ---- quantize / dequantize ------------------------------------------------

def quantize(w_bf16_bits: np.ndarray):
    """Quantize BF16 weights given as uint16 bit patterns, shape [n, k] or
    [batch, n, k].  Returns (packed uint8 [..., n, k/2], scales uint8
    [..., n, k/16], g float32 [batch] or scalar array)."""
    w = _c(w_bf16_bits, np.uint16)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    if w.ndim != 3:
        raise ValueError("weights must be [n, k] or [batch, n, k]")
    b, n, k = w.shape
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    packed = np.zeros((b, n, k // 2), np.uint8)
    scales = np.zeros((b, n, k // 16), np.uint8)
    g = np.zeros((b,), np.float32)
    st = _load().orc_quantize(_ptr(w), b, n, k, _ptr(packed), _ptr(scales), _ptr(g))
    if st == ERR_NONFINITE:
        raise OracleError("non-finite weight")
    if st != OK:
        raise OracleError("quantize failed: %d" % st)
    if squeeze:
        return packed[0], scales[0], g[0:1].copy()
    return packed, scales, g


def dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded weight without the global scale, float64 [n, k]."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    n, kh = packed.shape
    k = kh * 2
    if scales.shape != (n, k // 16):
        raise ValueError("scale shape mismatch")
    out = np.empty((n, k), np.float64)
    _load().orc_dequant(_ptr(packed), _ptr(scales), n, k, _ptr(out))
    return out


# ---- GEMM -----------------------------------------------------------------

def gemm(x_bf16_bits, packed, scales, g):
    """y = g * x @ w_dec^T and D = |g| * |x| @ |w_dec|^T, both float64 [m, n]."""
    x = _c(x_bf16_bits, np.uint16)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape != (n, k // 2) or scales.shape != (n, k // 16):
        raise ValueError("shape mismatch")
    y = np.zeros((m, n), np.float64)
    d = np.zeros((m, n), np.float64)
    st = _load().orc_gemm(_ptr(x), m, n, k, _ptr(packed), _ptr(scales), float(np.float32(g)),
                          _ptr(y), _ptr(d))
    if st != OK:
        raise OracleError("gemm failed: %d" % st)
    return y, d


def gemm_sampled(x_bf16_bits, packed, scales, g, rows, cols):
    x = _c(x_bf16_bits, np.uint16)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    m, k = x.shape
    n = packed.shape[0]
    y = np.zeros(rows.shape, np.float64)
    d = np.zeros(rows.shape, np.float64)
    st = _load().orc_gemm_sampled(_ptr(x), m, n, k, _ptr(packed), _ptr(scales),
                                  float(np.float32(g)), _ptr(rows), _ptr(cols), rows.size,
                                  _ptr(y), _ptr(d))
    if st != OK:
        raise OracleError("gemm_sampled failed: %d" % st)
    return y, d


def grouped_gemm(x_bf16_bits, offsets, packed, scales, g):
    """Rows [offsets[e], offsets[e+1]) of x use expert e.  packed [E, n, k/2],
    scales [E, n, k/16], g [E].  Rows of empty segments are never written and
    stay NaN in the returned y (and D)."""
    x = _c(x_bf16_bits, np.uint16)
    offsets = _c(offsets, np.int32)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    g = _c(g, np.float32)
    rows, k = x.shape
    E, n, _ = packed.shape
    y = np.full((rows, n), np.nan, np.float64)
    d = np.full((rows, n), np.nan, np.float64)
    st = _load().orc_grouped_gemm(_ptr(x), rows, _ptr(offsets), E, n, k, _ptr(packed),
                                  _ptr(scales), _ptr(g), _ptr(y), _ptr(d))
    if st != OK:
        raise OracleError("grouped_gemm failed: %d" % st)
    return y, d


def grouped_gemm_sampled(x_bf16_bits, offsets, packed, scales, g, rows_idx, cols_idx):
    x = _c(x_bf16_bits, np.uint16)
    offsets = _c(offsets, np.int32)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    g = _c(g, np.float32)
    rs = _c(rows_idx, np.int64)
    cs = _c(cols_idx, np.int64)
    rows, k = x.shape
    E, n, _ = packed.shape
    y = np.zeros(rs.shape, np.float64)
    d = np.zeros(rs.shape, np.float64)
    st = _load().orc_grouped_gemm_sampled(_ptr(x), rows, _ptr(offsets), E, n, k, _ptr(packed),
                                          _ptr(scales), _ptr(g), _ptr(rs), _ptr(cs), rs.size,
                                          _ptr(y), _ptr(d))
    if st != OK:
        raise OracleError("grouped_gemm_sampled failed: %d" % st)
    return y, d


# ---- gate_up with the SiLU(gate) * up epilogue -------------------------------
#
# "The FP4 Frontier", Finding 5 (persistent kernel recommendations) names the
# fused MoE MLP: the gate_up grouped GEMM followed by SiLU and the down GEMM.
# The pages define neither SiLU nor the fused weight's row order; the plain
# readings are SiLU(v) = v / (1 + e^-v) applied to the gate half and
# multiplied elementwise by the up half.  The fused weight [n = 2 i, k] holds
# its rows in 32-row groups: 16 gate rows, then the 16 up rows of the same
# output columns (output column c pairs weight rows 32 (c / 16) + c % 16 and
# that + 16).

SILU_SLOPE_MAX = 1.1  # bound on |d SiLU / dv| (its maximum is 1.0998 near v = 2.4)


def silu(v):
    """SiLU(v) = v / (1 + exp(-v)) in float64 (-0.0 for v -> -inf)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def gate_up_rows(n: int):
    """Weight rows (gate, up) feeding each of the n / 2 output columns."""
    if n % 32:
        raise ValueError("n must be a multiple of 32")
    c = np.arange(n // 2)
    gate = (c // 16) * 32 + c % 16
    return gate, gate + 16


def swiglu(y, d):
    """h = SiLU(y_gate) * y_up and its error scale D_h from the GEMM's
    (y, D) over the fused columns: a first-order bound on how errors
    of size e * D in y move h, D_h = 1.1 D_gate |y_up| + |SiLU(y_gate)| D_up."""
    y = np.asarray(y, np.float64)
    d = np.asarray(d, np.float64)
    gate, up = gate_up_rows(y.shape[-1])
    yg, yu = y[..., gate], y[..., up]
    sg = silu(yg)
    return sg * yu, SILU_SLOPE_MAX * d[..., gate] * np.abs(yu) + np.abs(sg) * d[..., up]


def grouped_gemm_swiglu(x_bf16_bits, offsets, packed, scales, g):
    """(h, D_h) of the grouped gate_up GEMM with the SiLU(gate) * up epilogue:
    h [rows, n / 2]; rows of empty segments stay NaN."""
    y, d = grouped_gemm(x_bf16_bits, offsets, packed, scales, g)
    return swiglu(y, d)


def grouped_gemm_swiglu_sampled(x_bf16_bits, offsets, packed, scales, g, rows_idx, cols_idx):
    """(h, D_h) at output positions (rows_idx, cols_idx) of the h matrix."""
    cols_idx = np.asarray(cols_idx, np.int64)
    gate, up = gate_up_rows(packed.shape[1])
    rr = np.concatenate([rows_idx, rows_idx])
    cc = np.concatenate([gate[cols_idx], up[cols_idx]])
    y, d = grouped_gemm_sampled(x_bf16_bits, offsets, packed, scales, g, rr, cc)
    m = len(cols_idx)
    yg, yu, dg, du = y[:m], y[m:], d[:m], d[m:]
    sg = silu(yg)
    return sg * yu, SILU_SLOPE_MAX * dg * np.abs(yu) + np.abs(sg) * du


# ---- MoE combine -----------------------------------------------------------------
#
# The scatter half of the routing-aware MoE layer ("The FP4 Frontier",
# Finding 5): each token's output is the router-weighted sum of the outputs of
# its top-k routed rows.  The pages give no formula; the plain reading is
# out[t] = sum_j w[t, j] * y[rows[t, j]], rows[t, j] < 0 meaning "no row".


def moe_combine(y, token_rows, weights):
    """out [tokens, n] and its error scale D = sum_j |w[t, j] * y[rows[t, j]]|,
    both float64; y [rows, n] as float64 values."""
    y = np.asarray(y, np.float64)
    token_rows = np.asarray(token_rows, np.int64)
    weights = np.asarray(weights, np.float64)
    tokens, topk = token_rows.shape
    out = np.zeros((tokens, y.shape[1]), np.float64)
    d = np.zeros_like(out)
    for t in range(tokens):
        for j in range(topk):
            r = token_rows[t, j]
            if r < 0:
                continue
            out[t] += weights[t, j] * y[r]
            d[t] += np.abs(weights[t, j] * y[r])
    return out, d


# ---- W4A4: both operands in NVFP4 -------------------------------------------
#
# The pages' FP4 GEMMs with block-scaled FP4 data and scale tiles for both
# operands ("The SM120 FP4 GEMM Kernel Investigation", section "The
# Comprehensive Synthesis: Message 6"; "The Tile That Didn't Fit: Diagnosing
# FP4 Kernel Underutilization on Blackwell SM120", section "Why Tile Size
# Matters for FP4 Performance").  Activations take the same encoding as the
# weights (two tiers, one E4M3 scale per 16 values along K, one FP32 scale
# per tensor), so the product is the plain definition over the two decoded
# operands: y = g_x * g_w * sum_k x_dec[m, k] * w_dec[n, k], in FP64.

def gemm_w4a4(x_packed, x_scales, g_x, packed, scales, g):
    """(y, D) float64 [m, n]: y = g_x * g * x_dec @ w_dec^T and
    D = |g_x * g| * |x_dec| @ |w_dec|^T, x_dec / w_dec the decoded operands
    without their global scales."""
    xd = dequant(x_packed, x_scales)
    wd = dequant(packed, scales)
    if xd.shape[1] != wd.shape[1]:
        raise ValueError("k mismatch")
    sg = float(np.float32(np.asarray(g_x).reshape(-1)[0])) * float(
        np.float32(np.asarray(g).reshape(-1)[0]))
    y = sg * (xd @ wd.T)
    d = abs(sg) * (np.abs(xd) @ np.abs(wd).T)
    return y, d


def grouped_gemm_w4a4(x_packed, x_scales, g_x, offsets, packed, scales, g):
    """Rows [offsets[e], offsets[e+1]) of the NVFP4 activations (one global
    scale g_x for all rows) times expert e's weight with g[e].  Rows of empty
    segments stay NaN."""
    x_packed = _c(x_packed, np.uint8)
    x_scales = _c(x_scales, np.uint8)
    offsets = _c(offsets, np.int64)
    g = _c(g, np.float32)
    rows = x_packed.shape[0]
    E, n, _ = np.asarray(packed).shape
    y = np.full((rows, n), np.nan, np.float64)
    d = np.full((rows, n), np.nan, np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b], d[a:b] = gemm_w4a4(x_packed[a:b], x_scales[a:b], g_x, packed[e], scales[e],
                                       g[e])
    return y, d

