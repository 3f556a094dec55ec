"""GPU parity of the dense W4A16 GEMM against the oracle.

y = g * x @ w_dec^T with BF16 activations and NVFP4 weights ("The SM120 FP4
GEMM Kernel Investigation", section "The Context").  The weights fed to the
GPU are the oracle's own encoding (quantize parity is tested separately), so
these tests isolate the GEMM.  Tolerances: FP32 output 1e-5, BF16 output
4e-3, normalized by sum_k |x * w| (see gpu_helpers)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_close, dev, host, output_values, require_gpu, sample_positions

pytestmark = pytest.mark.gpu


def oracle_weight(w_bits):
    p, s, g = oracle.quantize(w_bits)
    return p, s, np.atleast_1d(g).astype(np.float32)


def to_qw(nv, p, s, g):
    return nv.QuantizedWeight(dev(p), dev(s), dev(g))


def run_gemm(nv, x_bits, qw, out_dtype, sentinel=True):
    m = x_bits.shape[0]
    out = torch.full((m, qw.n), float("nan"), dtype=out_dtype, device="cuda") if sentinel else None
    y = nv.gemm(dev(x_bits), qw, out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    return y


@pytest.fixture
def splitk(request):
    """Force a K split through the library's tuning override, on the K-phase
    kernel also for products of 1 to 64 rows (the decode kernels, which
    otherwise take them, are switched off: they split K by their own plan or
    not at all)."""
    old = {v: os.environ.get(v) for v in ("NVFP4_SPLITK", "NVFP4_GEMV")}
    os.environ["NVFP4_SPLITK"] = str(request.param)
    os.environ["NVFP4_GEMV"] = "0"
    yield request.param
    for v, o in old.items():
        if o is None:
            os.environ.pop(v, None)
        else:
            os.environ[v] = o


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_small_dense(out_dtype):
    nv = require_gpu()
    x, w = W.small_dense()
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    y = run_gemm(nv, x, to_qw(nv, p, s, g), out_dtype)
    check_close(y, y_ref, d, "16x256x512")
    assert np.abs(output_values(y)).max() > 0  # never a silent all-zero result


@pytest.fixture(scope="module")
def decode_weight():
    return oracle_weight(W.decode_weight())


@pytest.mark.parametrize("m", [1, 16, 64])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_shapes(decode_weight, m, out_dtype):
    nv = require_gpu()
    p, s, g = decode_weight
    x = W.decode_act(m)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    y = run_gemm(nv, x, to_qw(nv, p, s, g), out_dtype)
    check_close(y, y_ref, d, "decode m=%d" % m)


RAGGED = [
    (1, 1, 16), (2, 17, 48), (15, 255, 64), (17, 257, 320), (33, 300, 576), (63, 100, 1040),
    (65, 511, 256), (130, 129, 208), (5, 1000, 2048), (100, 33, 96),
]


@pytest.mark.parametrize("m,n,k", RAGGED)
def test_ragged_shapes(m, n, k):
    nv = require_gpu()
    key = m * 1000003 + n * 1009 + k
    w = W.normal_bf16((n, k), 0.05, (77, key, 0))
    x = W.normal_bf16((m, k), 1.0, (77, key, 1))
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    check_close(run_gemm(nv, x, qw, torch.float32), y_ref, d, "f32 %dx%dx%d" % (m, n, k))
    check_close(run_gemm(nv, x, qw, torch.bfloat16), y_ref, d, "bf16 %dx%dx%d" % (m, n, k))


LARGE_M = [(256, 256, 64), (257, 300, 576), (300, 513, 1088), (511, 1024, 2048), (1000, 129, 4096)]


@pytest.fixture
def lm_mode(request):
    """NVFP4_LM=2 forces the 256 x 256 large-M kernel for any dense product of
    256 rows or more (by default it runs only when its tiles fill the CUs)."""
    old = os.environ.get("NVFP4_LM")
    if request.param is None:
        os.environ.pop("NVFP4_LM", None)
    else:
        os.environ["NVFP4_LM"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("NVFP4_LM", None)
    else:
        os.environ["NVFP4_LM"] = old


@pytest.mark.parametrize("lm_mode", ["2", None], indirect=True)
@pytest.mark.parametrize("m,n,k", LARGE_M)
def test_large_m_shapes(m, n, k, lm_mode):
    """Row counts of 256 and more: the 256 x 256 tile path (forced) and the
    default choice; ragged M, N and one-step K included."""
    nv = require_gpu()
    key = m * 1000003 + n * 1009 + k
    w = W.normal_bf16((n, k), 0.05, (79, key, 0))
    x = W.normal_bf16((m, k), 1.0, (79, key, 1))
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    check_close(run_gemm(nv, x, qw, torch.float32), y_ref, d, "f32 %dx%dx%d" % (m, n, k))
    check_close(run_gemm(nv, x, qw, torch.bfloat16), y_ref, d, "bf16 %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("splitk", [1, 2, 3, 7], indirect=True)
@pytest.mark.parametrize("m,n,k", [(16, 256, 1024), (3, 300, 1088), (64, 513, 960), (20, 64, 80)])
def test_forced_split_k(splitk, m, n, k):
    nv = require_gpu()
    key = m * 7919 + n * 31 + k
    w = W.normal_bf16((n, k), 0.05, (78, key, 0))
    x = W.normal_bf16((m, k), 1.0, (78, key, 1))
    p, s, g = oracle_weight(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    y1 = run_gemm(nv, x, qw, torch.float32)
    check_close(y1, y_ref, d, "split %d %dx%dx%d" % (splitk, m, n, k))
    y2 = run_gemm(nv, x, qw, torch.float32)
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32)), "not reproducible"


@pytest.mark.parametrize("splitk", [9, 28, 56], indirect=True)
@pytest.mark.parametrize("m", [1, 64])
def test_decode_deep_split(decode_weight, splitk, m):
    # many K splits per output tile (down to one 128-deep stage each): the
    # partial-tile hand-off between workgroups on different XCDs, summed in
    # split order
    nv = require_gpu()
    p, s, g = decode_weight
    x = W.decode_act(m)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = to_qw(nv, p, s, g)
    y1 = run_gemm(nv, x, qw, torch.float32)
    check_close(y1, y_ref, d, "decode m=%d split %d" % (m, splitk))
    y2 = run_gemm(nv, x, qw, torch.float32)
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32)), "not reproducible"


def test_default_schedule_reproducible(decode_weight):
    nv = require_gpu()
    p, s, g = decode_weight
    x = W.decode_act(16)
    qw = to_qw(nv, p, s, g)
    ys = [host(run_gemm(nv, x, qw, torch.float32)).view(np.uint32) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_zero_rows_is_noop():
    nv = require_gpu()
    x, w = W.small_dense()
    p, s, g = oracle_weight(w)
    y = nv.gemm(dev(x[:0]), to_qw(nv, p, s, g))
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_zero_weight_gives_exact_zero():
    nv = require_gpu()
    x, _ = W.small_dense()
    w = np.zeros((256, 512), np.uint16)
    p, s, g = oracle_weight(w)
    y = run_gemm(nv, x, to_qw(nv, p, s, g), torch.float32)
    assert (host(y) == 0).all()


def test_large_stratified_and_full_tiles():
    """8192 x 8192 x 8192 on the 256 x 256 large-M kernel (four persistent
    rounds of 256 tiles): one output in every 16 x 64 block (all tiles,
    rounds and accumulator positions), every output written, and four whole
    256 x 256 tiles -- one from each round -- against the oracle."""
    nv = require_gpu()
    from gpu_helpers import BF16_TOL, normalized_error, stratified_positions
    x, w = W.large_dense()
    p, s, g = oracle_weight(w)
    y = run_gemm(nv, x, to_qw(nv, p, s, g), torch.bfloat16)
    yv = output_values(y)
    assert np.isfinite(yv).all()  # every element written
    rows, cols = stratified_positions([(0, 8192)], 8192, seed=5)
    y_ref, d = oracle.gemm_sampled(x, p, s, g[0], rows, cols)
    err = normalized_error(yv[rows, cols], y_ref, d)
    assert err <= BF16_TOL, err
    # tile t covers rows 256 (t // 32), columns 256 (t % 32); round r of a
    # 256-workgroup grid takes tiles [256 r, 256 r + 256)
    for rnd in range(4):
        t = 256 * rnd + (37 * rnd + 11) % 256
        r0, c0 = 256 * (t // 32), 256 * (t % 32)
        y_ref, d = oracle.gemm(x[r0:r0 + 256], p[c0:c0 + 256], s[c0:c0 + 256], g[0])
        err = normalized_error(yv[r0:r0 + 256, c0:c0 + 256], y_ref, d)
        assert err <= BF16_TOL, "tile %d: %.3e" % (t, err)
