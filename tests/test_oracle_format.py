"""Pins of the oracle's format layer (E2M1 / E4M3 decode and RNE encode).

Each test ties the oracle to something outside it: the E2M1 value table
(golden file), PyTorch's float8_e4m3fn conversion (a library routine), the
hand-listed E2M1 rounding midpoints, and structural counts of the E4M3 code
space.  Format facts: "The Blackwell Architectural Split: NVFP4, Attention,
and Consumer Silicon", section "Preserving precision -- dual-tier scale
handling" (1 sign, 2 exponent, 1 mantissa bit; one block scale per 16 values).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e2m1():
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            table[int(c)] = float(v)
    return table


def test_e2m1_decode_matches_table():
    table = _golden_e2m1()
    assert sorted(table) == list(range(16))
    for c, v in table.items():
        got = oracle.e2m1_value(c)
        assert got == v, (c, got, v)
        assert math.copysign(1.0, got) == math.copysign(1.0, v), c  # -0 for code 8


def test_e2m1_bit_split():
    # sign is bit 3; codes c and c|8 are negatives of each other
    for c in range(8):
        assert oracle.e2m1_value(c | 8) == -oracle.e2m1_value(c)
    # exponent field (bits 2..1) doubles the value for every step once normal
    for e in range(1, 3):
        for m in range(2):
            assert oracle.e2m1_value(((e + 1) << 1) | m) == 2 * oracle.e2m1_value((e << 1) | m)


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all()
    assert np.array_equal(got[~nan_got], ref[~nan_ref])
    assert np.array_equal(np.signbit(got[~nan_got]), np.signbit(ref[~nan_ref]))


def test_e4m3_code_space_structure():
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.isnan(vals).sum() == 2 and np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert (vals == 0).sum() == 2
    pos = vals[:0x7F]
    assert (pos[1:] > 0).sum() == 126
    assert (pos[1:8] < 2.0 ** -6).all() and (pos[8:] >= 2.0 ** -6).all()  # 7 subnormals
    assert (np.diff(pos) > 0).all()
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9


def _float_range(lo_bits, hi_bits, chunk=1 << 26):
    for s in range(lo_bits, hi_bits, chunk):
        e = min(hi_bits, s + chunk)
        yield np.arange(s, e, dtype=np.uint32).view(np.float32)


def test_e4m3_encode_every_float_vs_torch():
    """Every float32 bit pattern in [0, 464] against torch's RNE cast; above
    464 torch returns NaN while the oracle saturates to 448 (code 0x7E)."""
    hi = int(np.array([464.0], np.float32).view(np.uint32)[0]) + 1
    for x in _float_range(0, hi):
        got = oracle.e4m3_encode(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])
    above = np.array([464.00003, 465.0, 480.0, 1e6, 3.4e38], np.float32)
    assert (oracle.e4m3_encode(above) == 0x7E).all()


def test_e4m3_encode_roundtrip_and_ties():
    for c in range(0x7F):
        assert oracle.e4m3_encode(np.float32(oracle.e4m3_value(c)))[0] == c
    # below half of the smallest subnormal -> 0; exactly half is a tie -> 0 (even)
    assert oracle.e4m3_encode(np.float32(2.0 ** -10))[0] == 0
    assert oracle.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))[0] == 1
    # 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): tie -> even 0x38
    assert oracle.e4m3_encode(np.float32(1.0625))[0] == 0x38
    # 1.1875 lies between 1.125 (0x39) and 1.25 (0x3A): tie -> even 0x3A
    assert oracle.e4m3_encode(np.float32(1.1875))[0] == 0x3A


# E2M1 magnitudes and the rounding midpoints between neighbours, with the
# winner of each tie (the code whose mantissa bit is 0), listed by hand.
E2M1_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E2M1_TIES = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]


def _e2m1_reference(q):
    mids = np.array([t for t, _ in E2M1_TIES], np.float32)
    idx = np.searchsorted(mids, q, side="left")  # number of midpoints strictly below q
    out = idx.astype(np.uint8)
    at_tie = np.isin(q, mids)
    tie_idx = np.searchsorted(mids, q[at_tie])
    out[at_tie] = np.array([w for _, w in E2M1_TIES], np.uint8)[tie_idx]
    return out


def test_e2m1_encode_every_float_in_range():
    """Every float32 bit pattern in [0, 8] against the midpoint rule."""
    hi = int(np.array([8.0], np.float32).view(np.uint32)[0]) + 1
    for q in _float_range(0, hi):
        got = oracle.e2m1_encode_mag(q)
        ref = _e2m1_reference(q)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (q[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e2m1_encode_saturates_and_neighbours():
    big = np.array([6.0, 6.5, 7.0, 100.0, 3.0e38, np.inf], np.float32)
    assert (oracle.e2m1_encode_mag(big) == 7).all()
    for t, w in E2M1_TIES:
        t32 = np.float32(t)
        below = np.nextafter(t32, np.float32(0))
        above = np.nextafter(t32, np.float32(10))
        lo_code = E2M1_MAGS.index(max(v for v in E2M1_MAGS if v < t))
        hi_code = E2M1_MAGS.index(min(v for v in E2M1_MAGS if v > t))
        assert oracle.e2m1_encode_mag([below])[0] == lo_code
        assert oracle.e2m1_encode_mag([t32])[0] == w
        assert oracle.e2m1_encode_mag([above])[0] == hi_code


def test_decoded_products_exact_in_bf16():
    """Every e2m1 * E4M3 product is exactly representable in BF16: at most six
    significant bits, magnitude between 2^-10 and 2688."""
    for c in range(16):
        for s in range(0x7F):
            v = oracle.e2m1_value(c) * oracle.e4m3_value(s)
            b = torch.tensor([v], dtype=torch.float64).to(torch.bfloat16).to(torch.float64)
            assert b.item() == v, (c, s, v)
