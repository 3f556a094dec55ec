"""Pins of the oracle's quantizer: fixed points, invariants and a hand-worked
example.  Two-tier scaling (global scale plus one E4M3 scale per 16 values):
"The Blackwell Architectural Split: NVFP4, Attention, and Consumer Silicon",
section "Preserving precision -- dual-tier scale handling"; about 4.5 stored
bits per weight: "The FP4 Frontier", Finding 6.
"""
import numpy as np
import pytest

import oracle
import workloads as W

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0,
                 -4.0, -6.0])


def e4m3_dec(code):
    """Independent E4M3FN decode (bias 7, 3 mantissa bits) used only to build
    test tensors."""
    code = np.asarray(code, np.int64)
    e = (code >> 3) & 15
    m = code & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(code >> 7, -v, v)


def unpack(packed):
    lo = packed & 15
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_storage_is_4p5_bits_per_weight():
    x, w = W.small_dense()
    p, s, g = oracle.quantize(w)
    n, k = w.shape
    assert (p.nbytes + s.nbytes) * 8 == 4.5 * n * k
    assert g.nbytes == 4


def test_hand_worked_block():
    """One row of 48 values (three blocks), worked by hand.

    amax of the tensor is 10.5, so g = 10.5 / 2688 = 2^-8 exactly.
    Block 0, amax 3: 3/6 = 0.5, 0.5 / 2^-8 = 128 = E4M3 0x70; step d = 0.5.
      3 -> 6 (code 7); -1.5 -> -3 (0xD); 0.75 -> 1.5 (3); 0.25 -> 0.5 (1);
      0.125 -> 0.25, a tie between 0 and 0.5 -> 0 (even); 0.375 -> 0.75, tie
      -> 1.0 (2); 0.625 -> 1.25, tie -> 1.0 (2); 0.875 -> 1.75, tie -> 2.0
      (4); 1.25 -> 2.5, tie -> 2.0 (4); 1.75 -> 3.5, tie -> 4.0 (6);
      2.5 -> 5, tie -> 4.0 (6); -2.75 -> -5.5 -> -6 (0xF); 0 -> 0; -0 -> 8.
    Block 1, amax 10.5: 1.75 / 2^-8 = 448 = 0x7E; d = 1.75.
      10.5 -> 6 (7); -5.25 -> -3 (0xD); 0.875 -> 0.5 (1).
    Block 2, amax 2.90625: 0.484375 / 2^-8 = 124, a tie between 120 (0x6F)
      and 128 (0x70) -> 0x70 (even); d = 0.5.
      2.90625 -> 5.8125 -> 6 (7); 1 -> 2 (4); -0.0625 -> -0.125 -> -0 (8).
    """
    row = np.zeros(48, np.float32)
    row[:14] = [3.0, -1.5, 0.75, 0.25, 0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5, -2.75,
                0.0, -0.0]
    row[16:19] = [10.5, -5.25, 0.875]
    row[32:35] = [2.90625, 1.0, -0.0625]
    w = bits(row)[None, :]
    p, s, g = oracle.quantize(w)
    assert g[0] == np.float32(2.0 ** -8)
    assert list(s[0]) == [0x70, 0x7E, 0x70]
    codes = [int(c) for c in unpack(p)[0]]
    assert codes[:16] == [7, 0xD, 3, 1, 0, 2, 2, 4, 4, 6, 6, 0xF, 0, 8, 0, 0]
    assert codes[16:32] == [7, 0xD, 1] + [0] * 13
    assert codes[32:48] == [7, 4, 8] + [0] * 13


@pytest.mark.parametrize("g_exp", [-12, -3, 0, 4])
def test_fixed_point(g_exp):
    """W = g0 * e2m1(c) * s(sc) with g0 a power of two, every block holding a
    +-6 and one block with sc = 0x7E quantizes back to exactly (c, sc, g0)."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 99, g_exp + 100]))
    n, k = 24, 96
    c = rng.integers(0, 16, size=(n, k))
    sc = rng.integers(0x20, 0x7F, size=(n, k // 16))
    blocks = c.reshape(n, k // 16, 16)
    pos = rng.integers(0, 16, size=(n, k // 16))
    sign = rng.integers(0, 2, size=(n, k // 16))
    np.put_along_axis(blocks, pos[..., None], (7 | (sign << 3))[..., None], axis=2)
    sc[rng.integers(0, n), rng.integers(0, k // 16)] = 0x7E
    c = blocks.reshape(n, k)
    g0 = 2.0 ** g_exp
    wv = g0 * E2M1[c] * np.repeat(e4m3_dec(sc), 16, axis=1)
    w = bits(wv)
    assert np.array_equal(W.bf16_bits_to_f32(w), wv.astype(np.float32))  # exact
    p, s, g = oracle.quantize(w)
    assert g[0] == np.float32(g0)
    assert np.array_equal(s, sc.astype(np.uint8))
    assert np.array_equal(unpack(p), c.astype(np.uint8))


@pytest.mark.parametrize("j", [-9, -2, 3, 11])
def test_power_of_two_scaling(j):
    _, w = W.small_dense()
    p0, s0, g0 = oracle.quantize(w)
    w2 = bits(W.bf16_bits_to_f32(w) * np.float32(2.0 ** j))
    p1, s1, g1 = oracle.quantize(w2)
    assert np.array_equal(p0, p1) and np.array_equal(s0, s1)
    assert g1[0] == g0[0] * np.float32(2.0 ** j)


def test_sign_flip():
    _, w = W.small_dense()
    p0, s0, g0 = oracle.quantize(w)
    p1, s1, g1 = oracle.quantize(w ^ np.uint16(0x8000))
    assert np.array_equal(s0, s1) and g0[0] == g1[0]
    assert np.array_equal(p1, p0 ^ np.uint8(0x88))


def test_block_max_encodes_to_six():
    w = W.decode_weight(256, 1024)
    p, s, g = oracle.quantize(w)
    codes = unpack(p).reshape(256, 64, 16)
    mags = np.abs(W.bf16_bits_to_f32(w)).reshape(256, 64, 16)
    amax_pos = mags.argmax(axis=2)
    top = np.take_along_axis(codes, amax_pos[..., None], axis=2)[..., 0] & 7
    normal = s >= 0x08
    assert normal.any()
    assert (top[normal] == 7).all()


def test_reconstruction_error_bound():
    """|w - g*w_dec| <= (half the E2M1 gap at the chosen code) * s_dec * g,
    outside the saturated region (q > 6)."""
    _, w = W.small_dense()
    p, s, g = oracle.quantize(w)
    wd = oracle.dequant(p, s) * float(g[0])
    wf = W.bf16_bits_to_f32(w).astype(np.float64)
    d = np.repeat(e4m3_dec(s), 16, axis=1) * float(g[0])
    q = np.abs(wf) / d
    gaps = np.array([0.25, 0.25, 0.25, 0.25, 0.5, 0.5, 1.0, 1.0])  # half-gaps around each code
    code = unpack(p) & 7
    err = np.abs(wf - wd)
    ok = (q <= 6.0)
    assert (err[ok] <= gaps[code[ok]] * d[ok] * (1 + 1e-6)).all()
    # saturated elements are clamped to 6 * d
    assert (np.abs(wd[~ok]) == 6.0 * d[~ok]).all()


def test_all_zero_tensor():
    w = np.zeros((4, 32), np.uint16)
    w[1, 3] = 0x8000
    p, s, g = oracle.quantize(w)
    assert g[0] == 0 and (s == 0).all()
    codes = unpack(p)
    assert codes[1, 3] == 8 and codes.sum() == 8


def test_nonfinite_rejected():
    w = np.zeros((2, 16), np.uint16)
    w[0, 5] = 0x7F80  # +inf
    with pytest.raises(oracle.OracleError):
        oracle.quantize(w)
    w[0, 5] = 0x7FC1  # NaN
    with pytest.raises(oracle.OracleError):
        oracle.quantize(w)


def test_batch_matches_individual():
    ws = np.stack([W.fuzz_weight(32, 64, "normal", i) for i in range(3)])
    pb, sb, gb = oracle.quantize(ws)
    for i in range(3):
        p, s, g = oracle.quantize(ws[i])
        assert np.array_equal(pb[i], p) and np.array_equal(sb[i], s) and gb[i] == g[0]


def test_subnormal_inputs_survive():
    """BF16 subnormals are not flushed: a tensor of tiny values still gets a
    non-zero global scale and non-zero codes."""
    w = W.fuzz_weight(16, 64, "subnormal")
    p, s, g = oracle.quantize(w)
    assert g[0] > 0 and (unpack(p) & 7).any()
