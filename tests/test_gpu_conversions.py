"""The gfx950 conversions the quantizer and the dequantizer rely on, checked
exhaustively on the GPU against the oracle's definitions of the formats (page
"The Blackwell Architectural Split: NVFP4, Attention, and Consumer Silicon",
section "Preserving precision -- dual-tier scale handling": E2M1 elements, one
E4M3 scale per 16 of them).  The kernels (tests/gpu_probe/conv_probe.hip) call
the same device helpers as the product kernels:

  - pack_e2m1_pair: FP32 -> E2M1 code (sign, then the nearest magnitude, ties
    to even, saturating at 6), over every non-negative FP32 pattern up to
    +inf and each one's negative;
  - encode_e4m3: the block-scale encoder, over every FP32 pattern from 0 to
    2^9 (every value that rounds to a finite code, then saturation);
  - decode_e4m3: all 256 codes, in each byte position of a dword;
  - element_quotient: the encoder's correctly rounded |x| / d, against IEEE
    binary32 division (numpy) on random and edge operands;
  - dequant8: every E2M1 code in every nibble position times every finite
    E4M3 scale, exact as BF16.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import probe_lib
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


def _chunks(lo, hi):
    b = lo
    while b < hi:
        n = min(CHUNK, hi - b)
        yield b, n
        b += n


def test_e2m1_pack_every_fp32_pattern():
    require_gpu()
    lib = probe_lib.load()
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    st = probe_lib.stream()
    top = 0x7F800000 + 1  # every finite non-negative pattern and +inf
    checked = 0
    for base, n in _chunks(0, top):
        assert lib.probe_e2m1_pack(base, n, probe_lib.ptr(out), st) == 0
        torch.cuda.synchronize()
        got = out[:n].cpu().numpy()
        x = np.arange(base, base + n, dtype=np.uint32).view(np.float32)
        mag = oracle.e2m1_encode_mag(x)
        want = mag | ((0x8 | mag) << 4)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "pattern 0x%08x: got 0x%02x want 0x%02x" % (
            base + bad[0], got[bad[0]], want[bad[0]])
        checked += n
    assert checked == top


def test_e4m3_encoder_every_fp32_pattern_to_512():
    require_gpu()
    lib = probe_lib.load()
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    st = probe_lib.stream()
    top = int(np.float32(512.0).view(np.uint32)) + 1
    for base, n in _chunks(0, top):
        assert lib.probe_e4m3_encode(base, n, probe_lib.ptr(out), st) == 0
        torch.cuda.synchronize()
        got = out[:n].cpu().numpy()
        want = oracle.e4m3_encode(np.arange(base, base + n, dtype=np.uint32).view(np.float32))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, "pattern 0x%08x: got 0x%02x want 0x%02x" % (
            base + bad[0], got[bad[0]], want[bad[0]])


def test_e4m3_decode_all_codes():
    require_gpu()
    lib = probe_lib.load()
    out = torch.empty(1024, dtype=torch.float32, device="cuda")
    assert lib.probe_e4m3_decode(probe_lib.ptr(out), probe_lib.stream()) == 0
    got = out.cpu().numpy().reshape(256, 4)
    for c in range(256):
        want = oracle.e4m3_value(c)
        for sel in range(4):
            g = float(got[c, sel])
            if np.isnan(want):
                assert np.isnan(g), (c, sel)
            else:
                assert g == want and np.signbit(g) == np.signbit(want), (c, sel, g, want)


def _quotient_cases(rng, n):
    # divisors d = decoded scale * g over the whole FP32 range the encoder can
    # see, dividends over every binade, plus exact multiples and edges
    d = (rng.random(n) + 0.5) * np.exp2(rng.integers(-140, 128, n).astype(np.float64))
    x = (rng.random(n) + 0.5) * np.exp2(rng.integers(-149, 128, n).astype(np.float64))
    d = d.astype(np.float32)
    x = x.astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        exact = (d * np.float32(3.0)).astype(np.float32)
    edge_d = np.array([2.0**-98, 2.0**100, 2.0**-98 * 1.5, 2.0**100 * 0.75, 1.0, 3.0, 6.0,
                       2.0**-126, 2.0**-149, 448.0 * 2.0**-10], np.float32)
    edge_x = np.array([0.0, 2.0**-149, 2.0**-126, 1.0, 6.0, 3.0e38, 0.25, 0.75, 5.0, 1.0e-30],
                      np.float32)
    ex, ed = np.meshgrid(edge_x, edge_d)
    xs = np.concatenate([x, exact, ex.ravel(), -x[:1000]])
    ds = np.concatenate([d, d, ed.ravel(), d[:1000]])
    keep = np.isfinite(xs) & np.isfinite(ds) & (ds > 0)
    return xs[keep], ds[keep]


def test_element_quotient_matches_ieee_division():
    require_gpu()
    lib = probe_lib.load()
    rng = np.random.default_rng(np.random.SeedSequence([5150, 1]))
    x, d = _quotient_cases(rng, 1 << 22)
    tx, td = torch.from_numpy(x).cuda(), torch.from_numpy(d).cuda()
    tq = torch.empty_like(tx)
    assert lib.probe_quotient(probe_lib.ptr(tx), probe_lib.ptr(td), probe_lib.ptr(tq),
                              x.size, probe_lib.stream()) == 0
    got = tq.cpu().numpy()
    with np.errstate(over="ignore", under="ignore", divide="ignore"):
        want = (np.abs(x) / d).astype(np.float32)  # IEEE binary32 division
    # bit for bit wherever the encoder relies on it: a dividend of at least
    # 2^-100 (else the residual step loses bits to underflow, and the
    # quotient, below d / 4, only has to stay under the first E2M1 rounding
    # threshold 0.25) and a normal quotient (the encoder's never exceed ~12)
    ax = np.abs(x)
    exact_region = np.isfinite(want) & (want >= 2.0**-126) & (ax >= 2.0**-100)
    assert (got[~exact_region & (want < 0.125)] < 0.25).all()
    assert exact_region.sum() > x.size // 2
    got, want, x, d = got[exact_region], want[exact_region], x[exact_region], d[exact_region]
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, "x=%r d=%r got %r want %r" % (x[bad[0]], d[bad[0]], got[bad[0]],
                                                          want[bad[0]])


def test_dequant8_every_code_and_scale():
    require_gpu()
    lib = probe_lib.load()
    # every code in every nibble position, then random words
    words = [int("%x" % c * 8, 16) for c in range(16)]
    words += [int(sum(((c + p) % 16) << (4 * p) for p in range(8))) for c in range(16)]
    rng = np.random.default_rng(np.random.SeedSequence([5150, 2]))
    words = np.concatenate([np.array(words, np.uint32),
                            rng.integers(0, 2**32, 2048, dtype=np.uint64).astype(np.uint32)])
    tw = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.empty(127 * words.size * 8, dtype=torch.float32, device="cuda")
    assert lib.probe_dequant(probe_lib.ptr(tw), words.size, probe_lib.ptr(out),
                             probe_lib.stream()) == 0
    got = out.cpu().numpy().reshape(127, words.size, 8)
    e2m1 = np.array([oracle.e2m1_value(c) for c in range(16)])
    codes = (words[:, None] >> (4 * np.arange(8)[None, :])) & 0xF
    for s in range(127):
        want = e2m1[codes] * oracle.e4m3_value(s)
        assert np.array_equal(got[s], want), "scale code 0x%02x" % s
        assert np.array_equal(np.signbit(got[s]), np.signbit(want)), "sign, scale 0x%02x" % s
