"""Helpers for the GPU parity tests: device plumbing and the error metric.

Error metric (the tolerance the GEMMs are held to): for every output
element, |y - y_ref| / D with D = |g| * sum_k |x[m,k] * w_dec[n,k]| (the
oracle returns D next to y_ref).  FP32 output must stay within 1e-5, BF16
output within 4e-3; where D == 0 the output must be exactly 0.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

F32_TOL = 1e-5
BF16_TOL = 4e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp4_nibble_amd as nv
    nv.load_library()  # raises if the HIP library is missing: no fallback
    return nv


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy array -> device tensor with the same bytes (uint16 -> bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def output_values(y: torch.Tensor) -> np.ndarray:
    h = host(y)
    if h.dtype == np.uint16:
        return bf16_bits_to_f64(h)
    return h.astype(np.float64)


def normalized_error(y: np.ndarray, y_ref: np.ndarray, d: np.ndarray) -> float:
    y = np.asarray(y, np.float64)
    assert y.shape == y_ref.shape == d.shape
    assert np.isfinite(y).all(), "non-finite output (unwritten sentinel or overflow)"
    zero = d == 0
    assert (y[zero] == 0).all(), "output must be exactly 0 where every product is 0"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(y - y_ref)[~zero] / d[~zero]).max())


def check_close(y_t: torch.Tensor, y_ref: np.ndarray, d: np.ndarray, what: str = ""):
    tol = F32_TOL if y_t.dtype == torch.float32 else BF16_TOL
    err = normalized_error(output_values(y_t), y_ref, d)
    assert err <= tol, "%s: normalized error %.3e > %.1e" % (what, err, tol)
    return err


def sample_positions(rows: int, cols: int, count: int, seed: int):
    rng = np.random.default_rng(np.random.SeedSequence([1234, seed]))
    r = rng.integers(0, rows, size=count)
    c = rng.integers(0, cols, size=count)
    # always include the corners and the last row / column
    r = np.concatenate([r, [0, rows - 1, 0, rows - 1]])
    c = np.concatenate([c, [0, 0, cols - 1, cols - 1]])
    return r.astype(np.int64), c.astype(np.int64)


def stratified_positions(segments, cols, seed, blk_r=16, blk_c=64):
    """Sample output positions that hit every 16-row x 64-column block of every
    row segment (an expert's rows, or [(0, rows)] for a dense product) once,
    so every output tile, every persistent round and every wave's column range
    of any kernel configuration gets a sample.  The position inside the block
    cycles through the (row % 16, column % 64) classes of the accumulator
    layout, so all of them are covered across the blocks; each segment's last
    row and the last column are always included."""
    rng = np.random.default_rng(np.random.SeedSequence([4321, seed]))
    rows_out, cols_out = [], []
    k = int(rng.integers(0, 1 << 20))
    for a, b in segments:
        a, b = int(a), int(b)
        if b <= a:
            continue
        for r0 in range(a, b, blk_r):
            nr = min(blk_r, b - r0)
            for c0 in range(0, cols, blk_c):
                nc = min(blk_c, cols - c0)
                rows_out.append(r0 + (k % blk_r) % nr)
                cols_out.append(c0 + ((k // blk_r) % blk_c) % nc)
                k += 1
        rows_out += [b - 1, b - 1, a]
        cols_out += [cols - 1, 0, cols - 1]
    return np.asarray(rows_out, np.int64), np.asarray(cols_out, np.int64)


def segments_of(offsets):
    off = np.asarray(offsets)
    return [(int(off[e]), int(off[e + 1])) for e in range(len(off) - 1)]


class EnvOverride:
    """Set library tuning overrides (environment variables read per call) for
    a block and restore them afterwards."""

    def __init__(self, **kv):
        self.kv = {k: (None if v is None else str(v)) for k, v in kv.items()}
        self.old = {}

    def __enter__(self):
        import os
        for k, v in self.kv.items():
            self.old[k] = os.environ.get(k)
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        return self

    def __exit__(self, *exc):
        import os
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        return False
