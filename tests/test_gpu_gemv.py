"""GPU parity of the decode kernels for dense products of one to sixteen rows.

Decode products ("The FP4 Frontier", Finding 7: bandwidth-bound at small
batch) of one to six token rows whose K fits its LDS (rows x K x 2 bytes up
to 96 KB) run on a kernel that keeps the block scale out of the inner loop:
per 16-element block the exact E2M1 values are dotted with the activations
in FP32, and the block's E4M3 scale multiplies that partial sum.  Five
and six rows of longer K (k % 128 == 0) run on one MFMA row tile per 16
columns with whole K per workgroup and a permuted K order inside each MFMA
(the K = 16384 cases below); from seven rows the split-K decode kernel takes
over (its own tests are in test_gpu_decode_sk.py; the 8-, 13- and 16-row
cases here run on it, with up to 128 splits of one K group at K = 16384, and
again on the MFMA kernel, which NVFP4_DSK=0 extends to 16 rows).  Same tolerances as
every GEMM: FP32 output within 1e-5, BF16 within 4e-3 of sum_k |x * w|."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_close, dev, host, output_values, require_gpu

pytestmark = pytest.mark.gpu


def oracle_weight(w_bits):
    p, s, g = oracle.quantize(w_bits)
    return p, s, np.atleast_1d(g).astype(np.float32)


def to_qw(nv, p, s, g):
    return nv.QuantizedWeight(dev(p), dev(s), dev(g))


def run_gemm(nv, x_bits, qw, out_dtype):
    out = torch.full((x_bits.shape[0], qw.n), float("nan"), dtype=out_dtype, device="cuda")
    y = nv.gemm(dev(x_bits), qw, out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    return y


class env:
    """Set one library override for the duration of a block."""

    def __init__(self, name, value):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = os.environ.get(self.name)
        os.environ[self.name] = self.value

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop(self.name, None)
        else:
            os.environ[self.name] = self.old


SHAPES = [
    (1, 32),       # one 32-weight chunk per row
    (17, 96),      # ragged column tile, three chunks
    (300, 1056),   # chunks not a multiple of the 32 a workgroup covers per pass
    (64, 8192),    # a lane's second batch of chunks
]


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("n,k", SHAPES)
def test_against_oracle(m, n, k):
    nv = require_gpu()
    name = nv.load_library().nvfp4_kernel_name(m, 1, n, k, 0, 0).decode()
    assert name == "nvfp4::gemv_kernel<%d>" % m, name
    key = m * 1000003 + n * 1009 + k
    w = W.normal_bf16((n, k), 0.05, (81, key, 0))
    x = W.normal_bf16((m, k), 1.0, (81, key, 1))
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    check_close(run_gemm(nv, x, qw, torch.float32), y_ref, d, "f32 %dx%dx%d" % (m, n, k))
    check_close(run_gemm(nv, x, qw, torch.bfloat16), y_ref, d, "bf16 %dx%dx%d" % (m, n, k))


SHAPES_128 = [
    (1, 128),      # one 128-deep K group: seven of the eight waves idle
    (17, 384),     # ragged column tile
    (300, 1152),   # K groups not a multiple of the eight waves
    (64, 16384),   # a wave's second batch of K groups
]


@pytest.mark.parametrize("m", [5, 6, 8, 13, 16])
@pytest.mark.parametrize("n,k", SHAPES_128)
def test_mfma_rows_against_oracle(m, n, k):
    nv = require_gpu()
    key = m * 1000003 + n * 1009 + k
    w = W.normal_bf16((n, k), 0.05, (83, key, 0))
    x = W.normal_bf16((m, k), 1.0, (83, key, 1))
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    check_close(run_gemm(nv, x, qw, torch.float32), y_ref, d, "f32 %dx%dx%d" % (m, n, k))
    check_close(run_gemm(nv, x, qw, torch.bfloat16), y_ref, d, "bf16 %dx%dx%d" % (m, n, k))
    if m <= 6 and m * k * 2 <= 98304:
        return  # the dot-product kernel's (staged rows fit its LDS)
    with env("NVFP4_DSK", "0"):  # the whole-K MFMA kernel up to 16 rows
        name = nv.load_library().nvfp4_kernel_name(m, 1, n, k, 0, 0).decode()
        assert name.startswith("nvfp4::decode_mfma_kernel<"), name
        check_close(run_gemm(nv, x, qw, torch.float32), y_ref, d, "mfma f32 %dx%dx%d" % (m, n, k))


@pytest.fixture(scope="module")
def decode_weight():
    return oracle_weight(W.decode_weight())


@pytest.mark.parametrize("m", [1, 4, 5, 16])
def test_decode_weight_both_paths(decode_weight, m):
    """N = 4096, K = 7168 with 0.1 % outliers: the decode kernel and the
    K-phase kernel (override NVFP4_GEMV=0) both within tolerance; the former
    reproducible bit for bit."""
    nv = require_gpu()
    p, s, g = decode_weight
    x = W.decode_act(m)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    y1 = run_gemm(nv, x, qw, torch.float32)
    y2 = run_gemm(nv, x, qw, torch.float32)
    check_close(y1, y_ref, d, "dot-product m=%d" % m)
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32))
    with env("NVFP4_GEMV", "0"):
        y3 = run_gemm(nv, x, qw, torch.float32)
    check_close(y3, y_ref, d, "K-phase m=%d" % m)


def test_zero_weight_gives_exact_zero():
    nv = require_gpu()
    w = np.zeros((40, 256), np.uint16)
    x = W.normal_bf16((1, 256), 1.0, (81, 1, 1))
    p, s, g = oracle_weight(w)
    y = run_gemm(nv, x, to_qw(nv, p, s, g), torch.float32)
    assert (host(y) == 0).all()


def test_rows_beyond_lds_limit_use_the_kphase_kernel():
    # 4 rows x K = 16384 is 128 KB of activations, above the 96 KB the
    # dot-product kernel stages; the product still comes out right
    nv = require_gpu()
    w = W.normal_bf16((96, 16384), 0.05, (81, 2, 0))
    x = W.normal_bf16((4, 16384), 1.0, (81, 2, 1))
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    check_close(run_gemm(nv, x, to_qw(nv, p, s, g), torch.float32), y_ref, d, "4x96x16384")


def test_signed_zero_and_extreme_codes():
    """Every nibble code (both zeros, all magnitudes, both signs) and the
    largest and smallest scale codes, with activations of mixed sign."""
    nv = require_gpu()
    rng = np.random.default_rng(82)
    n, k = 48, 512
    p = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    s = rng.integers(0, 0x7F, size=(n, k // 16), dtype=np.uint8)  # every finite code
    s[0, :] = 0x7E
    s[1, :] = 0x01
    s[2, :] = 0x00
    g = np.array([0.75], np.float32)
    x = W.normal_bf16((2, k), 1.0, (82, 0, 1))
    y_ref, d = oracle.gemm(x, p, s, g[0])
    y = run_gemm(nv, x, to_qw(nv, p, s, g), torch.float32)
    check_close(y, y_ref, d, "all codes")
    assert (output_values(y)[:, 2] == 0).all()  # a row of zero scales
