"""CPU checks of the C ABI: the library loads, exports every function that
include/nvfp4.h declares, and rejects bad arguments on the host before
touching the GPU (no compute calls here).  Boundary lesson: a backend that
returned all zeros without an error ("The SM120 FP4 GEMM Kernel
Investigation", section "The Breaking Point: FlashInfer #2577") -- every bad
call here must return a non-OK status instead."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_nibble_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv.LIB_PATH):
        pytest.fail("libnvfp4.so is not built (run __graft_entry__.build())")
    return nv.load_library()


def test_header_lists_the_entry_points():
    fns = declared_functions()
    for f in ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_grouped_gemm"):
        assert f in fns
    assert sorted(nv.EXPORTED) == fns


def test_every_declared_symbol_is_exported(lib):
    for f in declared_functions():
        assert hasattr(lib, f), f


def test_exports_are_c_symbols():
    raw = ctypes.CDLL(nv.LIB_PATH)
    for f in declared_functions():
        ctypes.cast(getattr(raw, f), ctypes.c_void_p)  # resolvable unmangled


def test_status_strings(lib):
    for code, name in nv.STATUS_NAMES.items():
        assert nv.nvfp4_status_string(code) == name
    assert nv.nvfp4_status_string(99) == "NVFP4_ERR_UNKNOWN"
    assert nv.nvfp4_version() >= 100
    assert nv.nvfp4_workspace_counter_bytes() % 16 == 0


class FakePtr:
    """Stands in for a tensor: only an address, never dereferenced because
    every call below is rejected on the host."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


A = FakePtr(0x10000)        # aligned
MIS = FakePtr(0x10008)      # 8-byte aligned only


class FakeStream:
    cuda_stream = 0


S = FakeStream()


def gemm_call(x=A, m=4, n=8, k=32, packed=A, scales=A, g=A, y=A, out=nv.OUT_BF16):
    return nv.nvfp4_gemm(x, m, n, k, packed, scales, g, y, out, None, 0, S)


def test_gemm_host_validation(lib):
    assert gemm_call(k=24) == 1           # k % 16 != 0
    assert gemm_call(k=0) == 1
    assert gemm_call(n=0) == 1
    assert gemm_call(m=-1) == 1
    assert gemm_call(out=7) == 1
    assert gemm_call(x=None) == 1
    assert gemm_call(y=MIS) == 2          # misaligned
    assert gemm_call(packed=MIS) == 2
    assert gemm_call(m=0, x=None, y=None) == 0  # empty problem is a no-op


def test_gemm_noalloc_host_validation(lib):
    def call(x=A, m=4, n=8, k=32, y=A, out=nv.OUT_BF16):
        return nv.nvfp4_gemm_noalloc(x, m, n, k, A, A, A, y, out, S)
    assert call(k=24) == 1
    assert call(n=0) == 1
    assert call(out=7) == 1
    assert call(x=None) == 1
    assert call(y=MIS) == 2
    assert call(m=0, x=None, y=None) == 0


def test_grouped_host_validation(lib):
    def call(E=4, offsets=A, rows=8, k=32):
        return nv.nvfp4_grouped_gemm(A, rows, offsets, E, 8, k, A, A, A, A, nv.OUT_BF16, None,
                                     None, 0, S)
    assert call(E=0) == 1
    assert call(E=nv.MAX_EXPERTS + 1) == 3   # unsupported, never silent
    assert call(offsets=None) == 1
    assert call(offsets=FakePtr(0x10002)) == 2
    assert call(k=40) == 1
    assert call(rows=0, offsets=None) == 0


def test_grouped_swiglu_host_validation(lib):
    def call(E=4, offsets=A, rows=8, n=64, k=32):
        return nv.nvfp4_grouped_gemm_swiglu(A, rows, offsets, E, n, k, A, A, A, A, nv.OUT_BF16,
                                            None, None, 0, S)
    assert call(n=48) == 1                   # gate/up rows come in 32-row groups
    assert call(n=16) == 1
    assert call(E=0) == 1
    assert call(E=nv.MAX_EXPERTS + 1) == 3
    assert call(offsets=None) == 1
    assert call(offsets=FakePtr(0x10002)) == 2
    assert call(k=40) == 1
    assert call(rows=0, offsets=None) == 0


def test_grouped_gather_host_validation(lib):
    def call(E=4, offsets=A, idx=A, rows=8, x_rows=16, n=64, k=32, act=0):
        return nv.nvfp4_grouped_gemm_gather(A, x_rows, idx, rows, offsets, E, n, k, A, A, A, A,
                                            nv.OUT_BF16, act, None, None, 0, S)
    assert call(idx=None) == 1
    assert call(x_rows=0) == 1
    assert call(act=2) == 1
    assert call(act=1, n=48) == 1
    assert call(idx=FakePtr(0x10002)) == 2
    assert call(E=nv.MAX_EXPERTS + 1) == 3
    assert call(x_rows=1 << 20, k=4096) == 3   # activation offsets exceed 32 bits
    assert call(rows=0, offsets=None, idx=None) == 0


def test_moe_combine_host_validation(lib):
    def call(y=A, rows=8, tr=A, w=A, tokens=4, topk=2, n=64, out=A, yt=None, ot=None):
        yt = nv.OUT_BF16 if yt is None else yt
        ot = nv.OUT_BF16 if ot is None else ot
        return nv.nvfp4_moe_combine(y, yt, rows, tr, w, tokens, topk, n, out, ot, None, S)
    assert call(n=12) == 1                    # columns come in groups of 8
    assert call(topk=0) == 1
    assert call(topk=65) == 1
    assert call(tokens=-1) == 1
    assert call(yt=7) == 1
    assert call(tr=None) == 1
    assert call(y=MIS) == 2
    assert call(w=FakePtr(0x10002)) == 2
    assert call(tokens=0, y=None, tr=None, w=None, out=None) == 0


def test_w4a4_host_validation(lib):
    def call(xs=A, xg=A, m=4, ws=None, nbytes=0):
        return nv.nvfp4_gemm_w4a4(A, xs, xg, m, 64, 32, A, A, A, A, nv.OUT_BF16, ws, nbytes, S)
    assert call(xs=None) == 1
    assert call(xg=FakePtr(0x10002)) == 2
    assert call() == 4                      # the decoded activations need a workspace
    assert nv.nvfp4_gemm_w4a4_workspace_size(4, 64, 32) >= 4 * 32 * 2
    assert call(m=0, xs=None, xg=None) == 0

    def gcall(E=4, off=A, rows=8):
        return nv.nvfp4_grouped_gemm_w4a4(A, A, A, rows, off, E, 64, 32, A, A, A, A,
                                          nv.OUT_BF16, None, None, 0, S)
    assert gcall(off=None) == 1
    assert gcall(E=nv.MAX_EXPERTS + 1) == 3
    assert gcall() == 4
    assert gcall(rows=0, off=None) == 0


def test_grouped_mlp_host_validation(lib):
    def call(E=4, offsets=A, rows=8, d_model=128, d_ff=64, h=A, y=A, out=nv.OUT_BF16):
        return nv.nvfp4_grouped_mlp(A, rows, offsets, E, d_model, d_ff, A, A, A, A, A, A, h, y,
                                    out, None, None, 0, S)
    assert call(E=0) == 1
    assert call(E=nv.MAX_EXPERTS + 1) == 3
    assert call(d_model=40) == 1             # not a multiple of 16
    assert call(d_model=96) == 3             # 64-column tiles only: unsupported, never silent
    assert call(d_ff=32) == 3
    assert call(out=7) == 1
    assert call(h=None) == 1
    assert call(y=MIS) == 2
    assert call(offsets=None) == 1
    assert call(offsets=FakePtr(0x10002)) == 2
    assert call(rows=0, offsets=None) == 0
    assert nv.nvfp4_grouped_mlp_workspace_size(8, 4, 96, 64) == 0
    assert nv.nvfp4_grouped_mlp_kernel_name(8, 4, 96, 64) == ""


@pytest.mark.parametrize("rows,E,d_model,d_ff,bm", [
    (512 * 8, 64, 6144, 2048, 64),   # ~64 rows per expert
    (128 * 8, 64, 6144, 2048, 32),   # ~16 rows per expert
    (333, 8, 512, 256, 64),
    (200, 4, 256, 128, 64),
    (8, 1, 128, 64, 16),
])
def test_grouped_mlp_plan(lib, rows, E, d_model, d_ff, bm):
    """The fused launch takes the grouped GEMM's K-phase kernel for the row
    tile its average rows per expert select, and its workspace is the GEMM
    counter region plus one 32-bit count per possible row tile."""
    name = nv.nvfp4_grouped_mlp_kernel_name(rows, E, d_model, d_ff)
    assert name.startswith("nvfp4::gemm_kp_kernel<%d," % bm) and name.endswith("false, true>"), name
    ws = nv.nvfp4_grouped_mlp_workspace_size(rows, E, d_model, d_ff)
    row_tiles = -(-rows // bm) + min(E, rows)
    assert ws == nv.nvfp4_workspace_counter_bytes() + -(-(4 * row_tiles) // 256) * 256


def test_quantize_host_validation(lib):
    def call(batch=1, n=4, k=32, w=A, ws=None):
        return nv.nvfp4_quantize(w, batch, n, k, A, A, A, None, ws, 0, S)
    assert call(k=8) == 1
    assert call(n=0) == 1
    assert call(batch=-1) == 1
    assert call(w=MIS) == 2
    assert call(batch=0) == 0
