"""Pins of the oracle's W4A4 product (both operands NVFP4).

Both operands carry the two-tier encoding ("The SM120 FP4 GEMM Kernel
Investigation", section "The Comprehensive Synthesis: Message 6": FP4 data and
scale tiles for both operands).  The pins: activations that the encoding
represents exactly make W4A4 equal the W4A16 oracle; swapping the operands
transposes the result; a tiny case by brute force over the E2M1 / E4M3 value
tables; the grouped form equals per-expert dense products.
"""
import numpy as np
import pytest

import oracle
import workloads as W

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0,
                 -4.0, -6.0])


def e4m3_dec(code):
    code = np.asarray(code, np.int64)
    e = (code >> 3) & 15
    m = code & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))


def exact_activations(m, k, seed, g_exp=-3):
    """BF16 activations g0 * e2m1(c) * s(sc) with a +-6 in every block: the
    encoding reproduces them exactly (codes, scales and g0)."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 98, seed]))
    c = rng.integers(0, 16, size=(m, k))
    sc = rng.integers(0x20, 0x7F, size=(m, k // 16))
    blocks = c.reshape(m, k // 16, 16)
    pos = rng.integers(0, 16, size=(m, k // 16))
    np.put_along_axis(blocks, pos[..., None], 7, axis=2)
    sc[0, 0] = 0x7E
    xv = 2.0 ** g_exp * E2M1[blocks.reshape(m, k)] * np.repeat(e4m3_dec(sc), 16, axis=1)
    return W.f32_to_bf16_bits(xv.astype(np.float32))


def test_exact_activations_match_w4a16():
    x = exact_activations(9, 96, seed=1)
    w = W.normal_bf16((40, 96), 0.05, (98, 1, 2))
    wp, ws, wg = oracle.quantize(w)
    xp, xs, xg = oracle.quantize(x)
    assert xg[0] == np.float32(2.0 ** -3)
    y4, d4 = oracle.gemm_w4a4(xp, xs, xg, wp, ws, wg)
    y16, d16 = oracle.gemm(x, wp, ws, wg[0])
    assert np.allclose(y4, y16, rtol=1e-13, atol=0)
    assert np.allclose(d4, d16, rtol=1e-13, atol=0)


def test_swapping_operands_transposes():
    x = W.normal_bf16((7, 64), 1.0, (98, 2, 1))
    w = W.normal_bf16((11, 64), 0.05, (98, 2, 2))
    xp, xs, xg = oracle.quantize(x)
    wp, ws, wg = oracle.quantize(w)
    y, d = oracle.gemm_w4a4(xp, xs, xg, wp, ws, wg)
    yt, dt = oracle.gemm_w4a4(wp, ws, wg, xp, xs, xg)
    assert np.array_equal(y, yt.T) and np.array_equal(d, dt.T)


def test_brute_force_tiny():
    rng = np.random.default_rng(5)
    m, n, k = 3, 4, 32
    xp = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    xs = rng.integers(0, 0x7F, size=(m, k // 16), dtype=np.uint8)
    ws = rng.integers(0, 0x7F, size=(n, k // 16), dtype=np.uint8)
    gx, gw = np.float32(0.375), np.float32(-1.25)
    y, d = oracle.gemm_w4a4(xp, xs, np.array([gx]), wp, ws, np.array([gw]))

    def val(p, s, r, kk):
        byte = int(p[r, kk // 2])
        code = byte & 15 if kk % 2 == 0 else byte >> 4
        return E2M1[code] * float(e4m3_dec(s[r, kk // 16]))

    for i in range(m):
        for j in range(n):
            acc = sum(val(xp, xs, i, kk) * val(wp, ws, j, kk) for kk in range(k))
            assert y[i, j] == pytest.approx(float(gx) * float(gw) * acc, rel=1e-14, abs=1e-300)


def test_grouped_is_per_expert_dense():
    counts = [3, 0, 5, 1]
    off = np.zeros(5, np.int64)
    off[1:] = np.cumsum(counts)
    x = W.normal_bf16((9, 48), 1.0, (98, 3, 1))
    w = W.normal_bf16((4, 24, 48), 0.05, (98, 3, 2))
    xp, xs, xg = oracle.quantize(x)
    wp, ws, wg = oracle.quantize(w)
    y, _ = oracle.grouped_gemm_w4a4(xp, xs, xg, off, wp, ws, wg)
    for e in range(4):
        a, b = off[e], off[e + 1]
        if b > a:
            ye, _ = oracle.gemm_w4a4(xp[a:b], xs[a:b], xg, wp[e], ws[e], wg[e])
            assert np.array_equal(y[a:b], ye)
