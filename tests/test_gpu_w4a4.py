"""GPU parity of the W4A4 products (activations and weights both NVFP4).

Both operands carry the two-tier encoding ("The SM120 FP4 GEMM Kernel
Investigation", section "The Comprehensive Synthesis: Message 6").  The
activations are quantized by the library (bit-exact with the oracle's
encoder, checked here too), decoded once per call to BF16 and multiplied on
the W4A16 kernels with the product of the two global scales.  Parity is
against the oracle's FP64 product of the decoded operands, with the usual
tolerances (FP32 output 1e-5, BF16 4e-3 of the error scale D).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (BF16_TOL, F32_TOL, check_close, dev, host, normalized_error,
                         output_values, require_gpu, sample_positions)

pytestmark = pytest.mark.gpu


def to_q(nv, p, s, g):
    return nv.QuantizedWeight(dev(p), dev(s), dev(np.atleast_1d(g).astype(np.float32)))


def quantized_pair(nv, x, w):
    """Library-quantized activations (checked bit for bit against the
    oracle) and oracle-quantized weights."""
    xp, xs, xg = oracle.quantize(x)
    xq = nv.quantize(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(host(xq.packed), xp) and np.array_equal(host(xq.scales), xs)
    assert host(xq.global_scale)[0] == xg[0]
    wp, ws, wg = oracle.quantize(w)
    return xq, (xp, xs, xg), to_q(nv, wp, ws, wg), (wp, ws, wg)


@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (3, 100, 96), (16, 300, 1024), (37, 129, 256),
                                   (300, 257, 576), (64, 4096, 7168)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dense_against_oracle(m, n, k, out_dtype):
    nv = require_gpu()
    key = m * 1000003 + n * 1009 + k
    x = W.normal_bf16((m, k), 1.0, (84, key, 1))
    w = W.normal_bf16((n, k), 0.05, (84, key, 2))
    xq, (xp, xs, xg), qw, (wp, ws, wg) = quantized_pair(nv, x, w)
    y_ref, d = oracle.gemm_w4a4(xp, xs, xg, wp, ws, wg)
    y = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda")
    nv.gemm_w4a4(xq, qw, out_dtype=out_dtype, out=y)
    torch.cuda.synchronize()
    check_close(y, y_ref, d, "w4a4 %dx%dx%d" % (m, n, k))


def test_exact_activations_equal_w4a16_launch():
    """Activations the encoding represents exactly: the W4A4 launch equals
    the W4A16 launch on the same BF16 activations, bit for bit."""
    nv = require_gpu()
    rng = np.random.default_rng(85)
    m, k = 24, 256
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    c = rng.integers(0, 16, size=(m, k))
    blocks = c.reshape(m, k // 16, 16)
    blocks[:, :, 0] = 7
    sc = rng.integers(0x30, 0x60, size=(m, k // 16))
    sc[0, 0] = 0x7E  # the tensor's largest block scale: g comes out as exactly 0.25
    e = (sc >> 3) & 15
    sval = (1 + (sc & 7) / 8.0) * np.exp2(e - 7.0)
    xv = 0.25 * e2m1[blocks.reshape(m, k)] * np.repeat(sval, 16, axis=1)
    x = W.f32_to_bf16_bits(xv.astype(np.float32))
    w = W.normal_bf16((200, k), 0.05, (85, 0, 2))
    xq, _, qw, _ = quantized_pair(nv, x, w)
    assert host(xq.global_scale)[0] == np.float32(0.25)
    y4 = nv.gemm_w4a4(xq, qw, out_dtype=torch.float32)
    y16 = nv.gemm(dev(x), qw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(y4).view(np.uint32), host(y16).view(np.uint32))


@pytest.mark.parametrize("counts,n,k", [([5, 0, 17, 1, 40], 192, 512), ([16] * 6, 320, 1024),
                                        ([70, 0, 3], 256, 2048)])
def test_grouped_against_oracle(counts, n, k):
    nv = require_gpu()
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    x = W.normal_bf16((int(off[-1]), k), 1.0, (86, n, 1))
    w = W.normal_bf16((E, n, k), 0.05, (86, n, 2))
    xq, (xp, xs, xg), qw, (wp, ws, wg) = quantized_pair(nv, x, w)
    y_ref, d = oracle.grouped_gemm_w4a4(xp, xs, xg, off, wp, ws, wg)
    for out_dtype in (torch.float32, torch.bfloat16):
        y = torch.full((int(off[-1]), n), float("nan"), dtype=out_dtype, device="cuda")
        nv.grouped_gemm_w4a4(xq, dev(off), qw, out_dtype=out_dtype, out=y)
        torch.cuda.synchronize()
        check_close(y, y_ref, d, "grouped w4a4 %s" % counts)


def test_uniform_16_tokens_per_expert_sampled():
    """The ~16 tok/expert up projection (N = 4096, K = 6144) with NVFP4
    activations: sampled outputs against the oracle."""
    nv = require_gpu()
    r, x, w = W.moe_uniform_inputs()
    xq, (xp, xs, xg), qw, (wp, ws, wg) = quantized_pair(nv, x, w)
    y = nv.grouped_gemm_w4a4(xq, dev(r.offsets.astype(np.int32)), qw)
    torch.cuda.synchronize()
    yv = output_values(y)
    rows, cols = sample_positions(r.rows, yv.shape[1], 1500, seed=51)
    xd = oracle.dequant(xp, xs)
    y_ref = np.empty(rows.shape)
    d = np.empty(rows.shape)
    e_of = np.searchsorted(r.offsets, rows, side="right") - 1
    for i, (rr, cc, e) in enumerate(zip(rows, cols, e_of)):
        wd = oracle.dequant(wp[e, cc:cc + 1], ws[e, cc:cc + 1])[0]
        sg = float(xg[0]) * float(wg[e])
        y_ref[i] = sg * float(xd[rr] @ wd)
        d[i] = abs(sg) * float(np.abs(xd[rr]) @ np.abs(wd))
    assert normalized_error(yv[rows, cols], y_ref, d) <= BF16_TOL


def test_shared_workspace_keeps_split_counters_zero():
    """A W4A4 call that does not split K, then split-K launches reusing the
    same workspace: the decoded activations never land on the counters."""
    nv = require_gpu()
    x = W.normal_bf16((300, 576), 1.0, (87, 0, 1))
    w = W.normal_bf16((257, 576), 0.05, (87, 0, 2))
    xq, _, qw, _ = quantized_pair(nv, x, w)
    nv.gemm_w4a4(xq, qw)
    wp, ws, wg = oracle.quantize(W.normal_bf16((512, 2048), 0.05, (87, 1, 2)))
    x2 = W.normal_bf16((64, 2048), 1.0, (87, 1, 1))
    y_ref, d = oracle.gemm(x2, wp, ws, wg[0])
    for _ in range(2):
        y = torch.full((64, 512), float("nan"), dtype=torch.float32, device="cuda")
        nv.gemm(dev(x2), to_q(nv, wp, ws, wg), out_dtype=torch.float32, out=y)
        torch.cuda.synchronize()
        check_close(y, y_ref, d, "split-K after W4A4")
