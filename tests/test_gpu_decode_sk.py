"""GPU parity of the split-K decode kernel (dense products of 7 to 64 rows,
and of 5 and 6 with NVFP4_DSK=2; k % 128 == 0) against the oracle.

The kernel (gemv.hip, decode_sk_kernel) splits K into units of at most 16
128-deep groups; wave w owns the groups j with j % 8 == w and stages their
token rows in an LDS region of its own (both of its groups up to 32 rows,
one at a time above), the eight waves' sums meet through LDS and the splits
through device-scope partial tiles in split order.  The cases cover both
region layouts, units with fewer groups than waves (waves with nothing to
multiply), uneven and single splits (no workspace), column counts that are
not a multiple of the 64-column unit, every row-fragment count and the
decode shape of "The FP4 Frontier" (N = 4096, K = 7168) in full.  Tolerances as in
the other GEMM tests (FP32 output 1e-5, BF16 4e-3 of sum_k |x w|)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import EnvOverride, check_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def kernel_name(nv, m, n, k):
    return nv.load_library().nvfp4_kernel_name(m, 1, n, k, 0, 0).decode()


@pytest.fixture(scope="module")
def decode_weight():
    p, s, g = oracle.quantize(W.decode_weight())
    return p, s, np.atleast_1d(g).astype(np.float32)


@pytest.mark.parametrize("m", [9, 16, 17, 32, 33, 48, 63, 64])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_shape_rows(decode_weight, m, out_dtype):
    nv = require_gpu()
    p, s, g = decode_weight
    assert kernel_name(nv, m, 4096, 7168).startswith("nvfp4::decode_sk_kernel<")
    x = W.decode_act(m)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    y = torch.full((m, 4096), float("nan"), dtype=out_dtype, device="cuda")
    nv.gemm(dev(x), qw, out=y, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y_ref, d = oracle.gemm(x, p, s, g[0])
    check_close(y, y_ref, d, "decode split-K m=%d" % m)


# (m, n, k): ragged columns, one to 16 groups per unit (so some waves own no
# group), both groups of a wave resident (up to 32 rows) or one at a time, a
# single split (at least as many column tiles as CUs), 32 splits of one group
SHAPES = [
    (5, 200, 384),
    (16, 64, 128),
    (20, 16448, 256),
    (33, 130, 1152),
    (32, 4096, 8192),
    (48, 1000, 2816),
    (64, 4160, 2304),
    (64, 96, 4096),
    (64, 4096, 8192),
]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_ragged_shapes(m, n, k):
    nv = require_gpu()
    seed = m * 7 + n + k
    x = W.normal_bf16((m, k), 1.0, (97, seed, 0))
    w = W.normal_bf16((n, k), 0.05, (97, seed, 1))
    p, s, g = oracle.quantize(w)
    g = np.atleast_1d(g).astype(np.float32)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    y_ref, d = oracle.gemm(x, p, s, g[0])
    with EnvOverride(NVFP4_DSK=2):  # the split-K decode kernel from 5 rows up
        assert kernel_name(nv, m, n, k).startswith("nvfp4::decode_sk_kernel<")
        for out_dtype in (torch.float32, torch.bfloat16):
            y = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda")
            nv.gemm(dev(x), qw, out=y, out_dtype=out_dtype)
            torch.cuda.synchronize()
            check_close(y, y_ref, d, "decode split-K %dx%dx%d" % (m, n, k))


def test_reproducible_bits(decode_weight):
    """The splits are summed in split order: repeated launches agree bit for
    bit."""
    nv = require_gpu()
    p, s, g = decode_weight
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    x = dev(W.decode_act(64))
    y0 = nv.gemm(x, qw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = host(y0).view(np.uint32).copy()
    for _ in range(5):
        y = nv.gemm(x, qw, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(host(y).view(np.uint32), want)


def test_switched_off_matches(decode_weight):
    """With the kernel switched off (NVFP4_DSK=0) the K-phase path computes
    the same product within the bound."""
    nv = require_gpu()
    p, s, g = decode_weight
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    x = W.decode_act(40)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    with EnvOverride(NVFP4_DSK=0):
        assert not kernel_name(nv, 40, 4096, 7168).startswith("nvfp4::decode_sk_kernel<")
        y = nv.gemm(dev(x), qw, out_dtype=torch.float32)
        torch.cuda.synchronize()
    check_close(y, y_ref, d, "decode m=40, K-phase path")
