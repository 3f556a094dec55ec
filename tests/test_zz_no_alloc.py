"""nvfp4_gemm_noalloc, the dense GEMM for callers that cannot allocate: its
split-K counters and partial tiles live in the library's per-device scratch
array instead of a caller workspace.  Called through the C ABI and compared
bit for bit with nvfp4_gemm (same schedule and kernels) on two calls in a
row, the second one smaller, plus the oracle and the over-limit error."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import EnvOverride, check_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _case(m, n, k, seed):
    x = W.normal_bf16((m, k), 1.0, (9090, seed, 0))
    w = W.normal_bf16((n, k), 0.03, (9090, seed, 1))
    p, s, g = oracle.quantize(w)
    return x, p, s, np.atleast_1d(g).astype(np.float32)


def _with_workspace(nv, xd, m, n, k, qd, out_code, dt):
    y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
    nbytes = nv.nvfp4_gemm_workspace_size(m, n, k)
    ws = None
    if nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        assert nv.nvfp4_workspace_init(ws, nbytes) == 0
    st = nv.nvfp4_gemm(xd, m, n, k, qd[0], qd[1], qd[2], y, out_code, ws, nbytes)
    assert st == 0, nv.nvfp4_status_string(st)
    return y, nbytes


def _noalloc(nv, xd, m, n, k, qd, out_code, dt):
    y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
    st = nv.nvfp4_gemm_noalloc(xd, m, n, k, qd[0], qd[1], qd[2], y, out_code)
    assert st == 0, nv.nvfp4_status_string(st)
    return y


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_noalloc_matches_gemm_two_calls(dt):
    nv = require_gpu()
    code = nv.OUT_F32 if dt == torch.float32 else nv.OUT_BF16
    # a split-K decode shape, then a smaller one (fewer rows, columns and K),
    # then one that needs no scratch at all
    for m, n, k in [(64, 4096, 7168), (20, 1000, 2048), (3, 300, 512)]:
        x, p, s, g = _case(m, n, k, seed=m * 7 + n + k)
        xd = dev(x)
        qd = (dev(p), dev(s), dev(g))
        y_ref, nbytes = _with_workspace(nv, xd, m, n, k, qd, code, dt)
        y = _noalloc(nv, xd, m, n, k, qd, code, dt)
        torch.cuda.synchronize()
        assert np.array_equal(host(y).view(np.uint16 if dt == torch.bfloat16 else np.uint32),
                              host(y_ref).view(np.uint16 if dt == torch.bfloat16 else np.uint32)), \
            (m, n, k)
        o_ref, d = oracle.gemm(x, p, s, g[0])
        check_close(y, o_ref, d, "noalloc %dx%dx%d" % (m, n, k))
        if (m, n, k) == (64, 4096, 7168):
            assert nbytes > nv.nvfp4_workspace_counter_bytes()  # the scratch path ran


def test_noalloc_forced_splits_and_limit():
    nv = require_gpu()
    m, n, k = 40, 1024, 4096
    x, p, s, g = _case(m, n, k, seed=3)
    xd, qd = dev(x), (dev(p), dev(s), dev(g))
    for splits in (2, 7, 32):
        with EnvOverride(NVFP4_SPLITK=splits, NVFP4_GEMV=0):
            y_ref, _ = _with_workspace(nv, xd, m, n, k, qd, nv.OUT_F32, torch.float32)
            y1 = _noalloc(nv, xd, m, n, k, qd, nv.OUT_F32, torch.float32)
            y2 = _noalloc(nv, xd, m, n, k, qd, nv.OUT_F32, torch.float32)
            torch.cuda.synchronize()
        assert np.array_equal(host(y1).view(np.uint32), host(y_ref).view(np.uint32)), splits
        assert np.array_equal(host(y2).view(np.uint32), host(y_ref).view(np.uint32)), splits
    # a schedule needing more than the scratch holds is refused, nothing written
    m, n, k = 64, 8192, 7168
    x, p, s, g = _case(m, n, k, seed=4)
    xd, qd = dev(x), (dev(p), dev(s), dev(g))
    with EnvOverride(NVFP4_SPLITK=56, NVFP4_GEMV=0):
        assert nv.nvfp4_gemm_workspace_size(m, n, k) > 65536 + (16 << 20)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        st = nv.nvfp4_gemm_noalloc(xd, m, n, k, qd[0], qd[1], qd[2], y, nv.OUT_F32)
        torch.cuda.synchronize()
    assert st == 3  # NVFP4_ERR_UNSUPPORTED
    assert torch.isnan(y).all()
