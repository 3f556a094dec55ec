"""Pins of the oracle's GEMM and grouped GEMM.

The product is the plain definition y[m, n] = g * sum_k x[m, k] * w_dec[n, k]
with BF16 activations ("The SM120 FP4 GEMM Kernel Investigation", section
"The Context": 4-bit weights, BF16 activations) and one expert per token
segment ("The FP4 Frontier", Finding 5: one grouped GEMM over all experts).
Pins: exact rational arithmetic on tiny dyadic cases (decoded through the
golden E2M1 table and torch's E4M3 cast, not the oracle's decoders), the
unit-scale special case against torch.matmul, symmetry, and the grouped
structure.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 16, 0), (3, 5, 32, 1), (8, 8, 48, 2),
                                        (2, 7, 16, 3), (8, 3, 48, 4)])
def test_tiny_dyadic_exact(m, n, k, seed):
    rng = np.random.default_rng(np.random.SeedSequence([7, seed]))
    codes = rng.integers(0, 16, size=(n, k))
    sc = rng.integers(0x28, 0x48, size=(n, k // 16))
    g = np.float32(2.0 ** int(rng.integers(-6, 3)))
    xv = rng.integers(-64, 65, size=(m, k)) * 2.0 ** -5   # exact in bf16
    x = bits(xv)
    y, d = oracle.gemm(x, pack(codes), sc.astype(np.uint8), g)
    s_dec = torch_e4m3(sc)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            mag = Fraction(0)
            for c in range(k):
                p = Fraction(xv[i, c]) * Fraction(E2M1[codes[j, c]]) * Fraction(s_dec[j, c // 16])
                acc += p
                mag += abs(p)
            assert y[i, j] == float(Fraction(float(g)) * acc), (i, j)
            assert d[i, j] == float(Fraction(float(g)) * mag), (i, j)


def test_unit_scale_reduces_to_matmul():
    """All block scales 0x38 (= 1.0) and g = 1: the product is x @ e2m1^T."""
    rng = np.random.default_rng(np.random.SeedSequence([7, 100]))
    m, n, k = 9, 33, 128
    codes = rng.integers(0, 16, size=(n, k))
    x = W.normal_bf16((m, k), 1.0, (7, 101))
    sc = np.full((n, k // 16), 0x38, np.uint8)
    y, _ = oracle.gemm(x, pack(codes), sc, np.float32(1.0))
    xt = torch.from_numpy(W.bf16_bits_to_f32(x).astype(np.float64))
    wt = torch.tensor(E2M1, dtype=torch.float64)[torch.from_numpy(codes)]
    ref = (xt @ wt.T).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_negation_symmetry_and_error_scale():
    x, w = W.small_dense()
    p, s, g = oracle.quantize(w)
    y, d = oracle.gemm(x, p, s, g[0])
    y2, d2 = oracle.gemm(x ^ np.uint16(0x8000), p, s, g[0])
    assert np.array_equal(y2, -y) and np.array_equal(d2, d)
    # D = |g| * |x| @ |w_dec|^T (library matmul in double)
    wd = oracle.dequant(p, s)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    dref = abs(float(g[0])) * (np.abs(xf) @ np.abs(wd).T)
    assert np.allclose(d, dref, rtol=1e-12)
    yref = float(g[0]) * (xf @ wd.T)
    assert np.allclose(y, yref, rtol=1e-9, atol=1e-9 * dref.max())
    assert (np.abs(y) <= d * (1 + 1e-12)).all()


def test_sampled_matches_full():
    x, w = W.small_dense()
    p, s, g = oracle.quantize(w)
    y, d = oracle.gemm(x, p, s, g[0])
    rows = np.array([0, 15, 7, 3])
    cols = np.array([255, 0, 100, 17])
    ys, ds = oracle.gemm_sampled(x, p, s, g[0], rows, cols)
    assert np.array_equal(ys, y[rows, cols]) and np.array_equal(ds, d[rows, cols])


def _grouped_case(counts, n=48, k=64, seed=0):
    E = len(counts)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    x = W.normal_bf16((int(offsets[-1]), k), 1.0, (8, seed, 1))
    w = W.normal_bf16((E, n, k), 0.02, (8, seed, 2))
    p, s, g = oracle.quantize(w)
    return x, offsets, p, s, g


def test_grouped_segments_are_dense_gemms():
    counts = [3, 0, 5, 1, 0, 7]
    x, off, p, s, g = _grouped_case(counts)
    y, d = oracle.grouped_gemm(x, off, p, s, g)
    for e in range(len(counts)):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        ye, de = oracle.gemm(x[r0:r1], p[e], s[e], g[e])
        assert np.array_equal(y[r0:r1], ye) and np.array_equal(d[r0:r1], de)
    assert not np.isnan(y).any()  # every routed row is written


def test_grouped_single_hot_expert_equals_dense():
    counts = [0, 0, 12, 0]
    x, off, p, s, g = _grouped_case(counts, seed=1)
    y, _ = oracle.grouped_gemm(x, off, p, s, g)
    yd, _ = oracle.gemm(x, p[2], s[2], g[2])
    assert np.array_equal(y, yd)


def test_grouped_rejects_bad_offsets():
    x, off, p, s, g = _grouped_case([2, 2])
    bad = off.copy()
    bad[1] = 5  # above the total
    with pytest.raises(oracle.OracleError):
        oracle.grouped_gemm(x, bad, p, s, g)
    bad = off.copy()
    bad[0] = 1
    with pytest.raises(oracle.OracleError):
        oracle.grouped_gemm(x, bad, p, s, g)


def test_grouped_sampled_matches_full():
    counts = [4, 0, 6, 2]
    x, off, p, s, g = _grouped_case(counts, seed=2)
    y, d = oracle.grouped_gemm(x, off, p, s, g)
    rs = np.array([0, 3, 4, 9, 11])
    cs = np.array([1, 47, 0, 20, 33])
    ys, ds = oracle.grouped_gemm_sampled(x, off, p, s, g, rs, cs)
    assert np.array_equal(ys, y[rs, cs]) and np.array_equal(ds, d[rs, cs])
