"""GPU parity: nvfp4_quantize must match the oracle bit for bit (packed nibbles,
E4M3 scale bytes and the FP32 global scale) on every workload's weights and on
encoder stress inputs.  Two-tier scaling per "The Blackwell Architectural
Split: NVFP4, Attention, and Consumer Silicon", section "Preserving precision
-- dual-tier scale handling"."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import dev, host, require_gpu

pytestmark = pytest.mark.gpu


def gpu_quantize(w_bits, d_status=None):
    nv = require_gpu()
    qw = nv.quantize(dev(w_bits), d_status=d_status)
    torch.cuda.synchronize()
    return host(qw.packed), host(qw.scales), host(qw.global_scale)


def assert_same(w_bits, what):
    p_ref, s_ref, g_ref = oracle.quantize(w_bits)
    p, s, g = gpu_quantize(w_bits)
    g_ref = np.atleast_1d(g_ref)
    assert g.view(np.uint32).tolist() == g_ref.view(np.uint32).tolist(), what + ": global scale"
    bad_s = np.argwhere(s != s_ref)
    assert bad_s.size == 0, "%s: %d scale bytes differ, first at %s" % (what, len(bad_s), bad_s[:3])
    bad_p = np.argwhere(p != p_ref)
    assert bad_p.size == 0, "%s: %d packed bytes differ, first at %s" % (what, len(bad_p), bad_p[:3])


def test_small_dense_weight():
    _, w = W.small_dense()
    assert_same(w, "256x512 N(0,1)")


def test_decode_weight_with_outliers():
    assert_same(W.decode_weight(), "4096x7168 N(0,0.02) + outliers")


@pytest.mark.parametrize("case", ["normal", "subnormal", "zeros", "outlier", "ties", "wide"])
@pytest.mark.parametrize("n,k", [(64, 1024), (37, 48), (5, 80), (300, 592)])
def test_fuzz(case, n, k):
    assert_same(W.fuzz_weight(n, k, case, key_extra=n * 10000 + k), "%s %dx%d" % (case, n, k))


def test_batched_experts_full_size():
    """64 experts of 4096 x 6144 (the MoE up-projection weights)."""
    _, _, w = W.moe_uniform_inputs()
    assert_same(w, "64x4096x6144 experts")


def test_zipf_up_weights_full_size():
    """64 experts of 4096 x 6144 (the ~64 tok/expert up-projection weights)."""
    _, _, w = W.moe_zipf_up_inputs()
    assert_same(w, "zipf up 64x4096x6144")


def test_zipf_down_weights_full_size():
    """64 experts of 6144 x 2048 (the ~64 tok/expert down-projection weights)."""
    _, _, w = W.moe_zipf_down_inputs()
    assert_same(w, "zipf down 64x6144x2048")


def test_large_weight():
    _, w = W.large_dense()
    assert_same(w, "8192x8192")


def test_nonfinite_sets_status_other_tensors_intact():
    nv = require_gpu()
    ws = np.stack([W.fuzz_weight(32, 64, "normal", i) for i in range(3)])
    ws[1, 4, 7] = 0x7FC0  # NaN in tensor 1
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    qw = nv.quantize(dev(ws), d_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & nv.DSTATUS_NONFINITE
    for t in (0, 2):
        p_ref, s_ref, g_ref = oracle.quantize(ws[t])
        assert np.array_equal(host(qw.packed)[t], p_ref)
        assert np.array_equal(host(qw.scales)[t], s_ref)
        assert host(qw.global_scale)[t] == g_ref[0]
    ws[1, 4, 7] = 0xFF80  # -inf
    status.zero_()
    nv.quantize(dev(ws), d_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & nv.DSTATUS_NONFINITE


def test_all_zero_and_signed_zero():
    w = np.zeros((16, 64), np.uint16)
    w[3, 5] = 0x8000
    w[7, 63] = 0x8000
    assert_same(w, "all zero")
    p, s, g = gpu_quantize(w)
    assert g[0] == 0 and (s == 0).all()


def test_deterministic_reruns():
    w = W.decode_weight(512, 1024)
    a = gpu_quantize(w)
    b = gpu_quantize(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
