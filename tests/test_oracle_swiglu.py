"""Pins of the oracle's gate_up GEMM with the SiLU(gate) * up epilogue.

The fused MoE MLP ("The FP4 Frontier", Finding 5) applies SiLU to the gate
half of the gate_up product and multiplies it by the up half.  Pins: SiLU
against scipy's logistic function, the row pairing against GEMMs over gate
and up rows separated by an explicit block loop (not the oracle's index
arithmetic), the error scale D_h as a bound under perturbations of the
GEMM output, and the sampled form against the full one.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads as W


def test_silu_matches_library_logistic():
    v = np.concatenate([np.linspace(-60, 60, 4801), [-1e5, -745.0, -700.0, -1e-300, 0.0, 1e-300,
                                                    700.0, 1e5, 3.0e38]])
    got = oracle.silu(v)
    want = v * expit(v)
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)  # two roundings apart
    assert np.signbit(oracle.silu(-1e5)) and oracle.silu(-1e5) == 0.0
    assert oracle.silu(0.0) == 0.0


def test_silu_slope_bound():
    v = np.linspace(-20, 20, 400001)
    s = oracle.silu(v)
    slope = np.abs(np.diff(s) / np.diff(v))
    assert slope.max() <= oracle.SILU_SLOPE_MAX
    assert slope.max() > 1.09  # the bound is close to the true maximum


def fused_from_halves(gate, up):
    """[E, 2 i, k] weight from gate and up [E, i, k], 16-row blocks alternating."""
    E, i, k = gate.shape
    fused = np.empty((E, 2 * i, k), gate.dtype)
    for b in range(i // 16):
        fused[:, 32 * b:32 * b + 16] = gate[:, 16 * b:16 * b + 16]
        fused[:, 32 * b + 16:32 * b + 32] = up[:, 16 * b:16 * b + 16]
    return fused


def halves_of_fused(a):
    """Inverse of fused_from_halves on axis 1 (explicit block loop)."""
    n = a.shape[1]
    gate = np.concatenate([a[:, 32 * b:32 * b + 16] for b in range(n // 32)], axis=1)
    up = np.concatenate([a[:, 32 * b + 16:32 * b + 32] for b in range(n // 32)], axis=1)
    return gate, up


@pytest.mark.parametrize("counts,i,k", [([2, 0, 3], 32, 32), ([5, 7], 64, 48)])
def test_pairing_against_separate_gemms(counts, i, k):
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    x = W.normal_bf16((int(off[-1]), k), 1.0, (95, i, 1))
    gate = W.normal_bf16((E, i, k), 0.05, (95, i, 2))
    up = W.normal_bf16((E, i, k), 0.05, (95, i, 3))
    p, s, g = oracle.quantize(fused_from_halves(gate, up))
    h, dh = oracle.grouped_gemm_swiglu(x, off, p, s, g)
    pg, pu = halves_of_fused(p)
    sg, su = halves_of_fused(s)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r0 == r1:
            assert np.isnan(h[r0:r1]).all()
            continue
        yg, dg = oracle.gemm(x[r0:r1], pg[e], sg[e], g[e])
        yu, du = oracle.gemm(x[r0:r1], pu[e], su[e], g[e])
        want = yg * expit(yg) * yu
        np.testing.assert_allclose(h[r0:r1], want, rtol=1e-13, atol=1e-300)
        assert (dh[r0:r1] >= np.abs(h[r0:r1]) * 0.99).all()


def test_error_scale_bounds_perturbations():
    rng = np.random.default_rng(96)
    y = rng.standard_normal((200, 64)) * 4
    d = np.abs(rng.standard_normal((200, 64))) * 3 + np.abs(y)
    h, dh = oracle.swiglu(y, d)
    eps = 1e-6
    for _ in range(20):
        yp = y + eps * d * rng.uniform(-1, 1, y.shape)
        hp, _ = oracle.swiglu(yp, d)
        assert (np.abs(hp - h) <= eps * dh * (1 + 1e-3) + 1e-300).all()


def test_sampled_matches_full():
    counts = [3, 0, 9, 4]
    E, i, k = len(counts), 48, 64
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    x = W.normal_bf16((int(off[-1]), k), 1.0, (97, 0, 1))
    w = W.normal_bf16((E, 2 * i, k), 0.05, (97, 0, 2))
    p, s, g = oracle.quantize(w)
    h, dh = oracle.grouped_gemm_swiglu(x, off, p, s, g)
    rows = np.array([0, 2, 3, 11, 15, 12])
    cols = np.array([0, 47, 16, 31, 5, 40])
    hs, dhs = oracle.grouped_gemm_swiglu_sampled(x, off, p, s, g, rows, cols)
    np.testing.assert_allclose(hs, h[rows, cols], rtol=1e-15, atol=0)
    np.testing.assert_allclose(dhs, dh[rows, cols], rtol=1e-15, atol=0)
