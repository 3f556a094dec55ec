"""Persistent launches whose workgroups each walk several units, checked in
full against the oracle.

At the reduced sizes the other tests use, the grid covers every unit in one
round, so the paths only full-size launches reach -- a workgroup's second and
later units, the K-phase kernel's prefetch of the next unit's first stages
during the current unit's last iterations (units of at least five 128-deep
stages), the large-M kernel's tile loop -- would go unchecked.  NVFP4_GRID
caps the grid to a few workgroups, so small products run through exactly
those paths, every output compared with the oracle ("The FP4 Frontier",
Finding 5: one persistent grouped kernel over all experts)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import EnvOverride, check_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu

GRIDS = [1, 3, 8]


def grouped_case(counts, n, k, seed):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    x = W.normal_bf16((int(off[-1]), k), 1.0, (8080, seed, 0))
    w = W.normal_bf16((len(counts), n, k), 0.03, (8080, seed, 1))
    p, s, g = oracle.quantize(w)
    return x, off, p, s, g


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("counts,n,k,env", [
    ([17, 0, 29, 5, 64, 3], 384, 1024, {}),                   # 4-wave, 128 columns
    ([70, 0, 130, 9], 512, 768, {}),                          # 8 waves, 64-row tiles
    ([20, 33, 1], 384, 640, {"NVFP4_KPCFG": 8}),              # 8 waves on small tiles
    ([9, 15, 2, 16], 256, 1152, {"NVFP4_BM": 16}),            # 16-row tiles
    ([40, 0, 7], 300, 1088, {}),                              # ragged N and K tail
], ids=["kp4", "kp8", "kp8_forced", "bm16", "ragged"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_multi_round(counts, n, k, env, grid, out_dtype):
    nv = require_gpu()
    x, off, p, s, g = grouped_case(counts, n, k, seed=sum(counts) + n + k)
    y_ref, d = oracle.grouped_gemm(x, off, p, s, g)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    with EnvOverride(NVFP4_GRID=grid, **env):
        y = torch.full((int(off[-1]), n), float("nan"), dtype=out_dtype, device="cuda")
        nv.grouped_gemm(dev(x), dev(off), qw, out_dtype=out_dtype, out=y)
        torch.cuda.synchronize()
    check_close(y, y_ref, d, "grid %d %s" % (grid, counts))


@pytest.mark.parametrize("grid", GRIDS)
def test_swiglu_and_gather_multi_round(grid):
    nv = require_gpu()
    counts, n, k = [17, 0, 40, 5], 256, 1024
    x, off, p, s, g = grouped_case(counts, n, k, seed=77)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    h_ref, dh = oracle.grouped_gemm_swiglu(x, off, p, s, g)
    tokens = 30
    rng = np.random.default_rng(5)
    row_token = rng.integers(0, tokens, int(off[-1])).astype(np.int32)
    x_tok = W.normal_bf16((tokens, k), 1.0, (8080, 78, 0))
    y_ref, d = oracle.grouped_gemm(x_tok[row_token], off, p, s, g)
    with EnvOverride(NVFP4_GRID=grid):
        h = nv.grouped_gemm_swiglu(dev(x), dev(off), qw, out_dtype=torch.float32)
        y = nv.grouped_gemm_gather(dev(x_tok), dev(row_token), dev(off), qw,
                                   out_dtype=torch.float32)
        hg = nv.grouped_gemm_gather(dev(x_tok), dev(row_token), dev(off), qw, act="swiglu",
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()
    check_close(h, h_ref, dh, "swiglu grid %d" % grid)
    check_close(y, y_ref, d, "gather grid %d" % grid)
    hg_ref, dhg = oracle.grouped_gemm_swiglu(x_tok[row_token], off, p, s, g)
    check_close(hg, hg_ref, dhg, "gather swiglu grid %d" % grid)


@pytest.mark.parametrize("grid", [1, 2, 5])
@pytest.mark.parametrize("m,n,k", [(600, 600, 576), (513, 300, 1088)])
def test_large_m_multi_round(m, n, k, grid):
    """The 256 x 256 large-M kernel with several tiles per workgroup."""
    nv = require_gpu()
    x = W.normal_bf16((m, k), 1.0, (8081, m + n, 0))
    w = W.normal_bf16((n, k), 0.03, (8081, m + n, 1))
    p, s, g = oracle.quantize(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(np.atleast_1d(g).astype(np.float32)))
    with EnvOverride(NVFP4_GRID=grid, NVFP4_LM=2):
        for dt in (torch.float32, torch.bfloat16):
            y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            nv.gemm(dev(x), qw, out_dtype=dt, out=y)
            torch.cuda.synchronize()
            check_close(y, y_ref, d, "large-M grid %d %s" % (grid, dt))


@pytest.mark.parametrize("grid", [1, 4])
@pytest.mark.parametrize("splits", [2, 3])
def test_split_k_multi_round(grid, splits):
    """K split across units that one workgroup runs one after another."""
    nv = require_gpu()
    counts, n, k = [20, 0, 45], 300, 1536
    x, off, p, s, g = grouped_case(counts, n, k, seed=91 + splits)
    y_ref, d = oracle.grouped_gemm(x, off, p, s, g)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    with EnvOverride(NVFP4_GRID=grid, NVFP4_SPLITK=splits):
        y1 = nv.grouped_gemm(dev(x), dev(off), qw, out_dtype=torch.float32)
        y2 = nv.grouped_gemm(dev(x), dev(off), qw, out_dtype=torch.float32)
        torch.cuda.synchronize()
    check_close(y1, y_ref, d, "split %d grid %d" % (splits, grid))
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32))
