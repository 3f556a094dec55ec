"""Activation fuzz through every GEMM kernel kind, against the oracle.

The products y = g * sum_k x[m,k] * w_dec[n,k] take BF16 activations
("The SM120 FP4 GEMM Kernel Investigation", section "The Context"); every
value of the format must pass through unchanged, subnormals and signed zeros
included.  Each family below is run through each kernel the planner can pick,
forced with the library's tuning overrides, with FP32 output (tolerance 1e-5
of sum_k |x w|):

  kind 6  dot-product kernel (1-6 dense rows, rows x K x 2 bytes <= 96 KB)
  kind 7  MFMA decode kernel (5-6 dense rows of longer K, k % 128 == 0;
          up to 16 rows with NVFP4_DSK=0)
  kind 8  split-K decode kernel (7-64 dense rows, k % 128 == 0)
  kind 4  K-phase kernel, 64-column tiles (dense <= 16 rows, NVFP4_GEMV=0)
  kind 1  K-phase kernel, 4 waves x 128 columns (65-128 dense rows, 17-64
          with NVFP4_DSK=0, or a grouped launch with <= 32 rows per expert)
  kind 2  K-phase kernel, 8 waves x 256 columns (NVFP4_KPCFG=8 / 64-row tiles)
  kind 3  large-M kernel (NVFP4_LM=2, >= 256 rows)
  kind 0  register kernel (k % 64 != 0)
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import EnvOverride, check_close, dev, require_gpu

pytestmark = pytest.mark.gpu

FAMILIES = ["subnormal", "wide", "signed_zeros", "mixed"]


def act(m, k, family, seed):
    """BF16 activation bit patterns of one family."""
    rng = np.random.default_rng(np.random.SeedSequence([7070, seed]))
    if family == "subnormal":
        # BF16 subnormals and the smallest normals (exponent field 0..2)
        bits = rng.integers(1, 3 << 7, size=(m, k), dtype=np.uint32)
        sign = rng.integers(0, 2, size=(m, k), dtype=np.uint32) << 15
        return (bits | sign).astype(np.uint16)
    if family == "wide":
        # every element its own binade, over ~120 binades
        e = rng.integers(-60, 60, size=(m, k)).astype(np.float32)
        v = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(e)
        return W.f32_to_bf16_bits(v)
    if family == "signed_zeros":
        v = W.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        z = rng.random((m, k)) < 0.5
        v[z] = np.where(rng.random(z.sum()) < 0.5, 0x0000, 0x8000).astype(np.uint16)
        v[0, :] = 0x8000  # a row of negative zeros: y must be exactly 0
        return v
    if family == "mixed":
        # normal values with subnormal and huge outliers in every row
        v = rng.standard_normal((m, k)).astype(np.float32)
        tiny = rng.random((m, k)) < 0.2
        v[tiny] *= np.float32(2.0**-130)
        huge = rng.random((m, k)) < 0.01
        v[huge] *= np.float32(2.0**60)
        return W.f32_to_bf16_bits(v)
    raise ValueError(family)


# (kind, m, n, k, overrides)
DENSE_KINDS = [
    (6, 3, 200, 512, {}),
    (7, 7, 200, 1024, {"NVFP4_DSK": 0}),
    (8, 11, 200, 1024, {}),
    (8, 40, 300, 1024, {}),
    (4, 9, 200, 1024, {"NVFP4_GEMV": 0}),
    (1, 40, 300, 1024, {"NVFP4_DSK": 0}),
    (2, 40, 300, 1024, {"NVFP4_DSK": 0, "NVFP4_KPCFG": 8}),
    (3, 300, 300, 512, {"NVFP4_LM": 2}),
    (0, 20, 200, 208, {}),
]
# kernel name prefix of each kind (the planner's choice is checked, so a
# change of the planner cannot silently move a case off its kernel)
KIND_NAME = {6: "nvfp4::gemv_kernel<", 7: "nvfp4::decode_mfma_kernel<",
             8: "nvfp4::decode_sk_kernel<", 4: "nvfp4::gemm_kp_kernel<16, 5, 4, 64,",
             1: "nvfp4::gemm_kp_kernel<32, 4, 4, 128,", 2: "nvfp4::gemm_kp_kernel<32, 5, 8, 256,",
             3: "nvfp4::gemm_lm_kernel", 0: "nvfp4::gemm_reg_kernel<"}


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("kind,m,n,k,env", DENSE_KINDS,
                         ids=["kind%d_m%d" % (c[0], c[1]) for c in DENSE_KINDS])
def test_dense(kind, m, n, k, env, family):
    nv = require_gpu()
    seed = kind * 100 + FAMILIES.index(family)
    x = act(m, k, family, seed)
    w = W.normal_bf16((n, k), 0.05, (7070, seed, 1))
    p, s, g = oracle.quantize(w)
    y_ref, d = oracle.gemm(x, p, s, g[0])
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(np.atleast_1d(g).astype(np.float32)))
    with EnvOverride(**env):
        name = nv.load_library().nvfp4_kernel_name(m, 1, n, k, 0, 0).decode()
        assert name.startswith(KIND_NAME[kind]), name
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        nv.gemm(dev(x), qw, out_dtype=torch.float32, out=y)
        torch.cuda.synchronize()
    check_close(y, y_ref, d, "kind %d %s" % (kind, family))
    if family == "signed_zeros":
        assert (y[0] == 0).all()


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("counts,env", [([20, 0, 9, 31], {}), ([70, 3, 64], {}),
                                        ([20, 0, 9, 31], {"NVFP4_KPCFG": 8})],
                         ids=["kp4", "kp8_bm64", "kp8_forced"])
def test_grouped(counts, env, family):
    nv = require_gpu()
    seed = sum(counts) * 7 + FAMILIES.index(family)
    n, k = 256, 1024
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    x = act(int(off[-1]), k, family, seed)
    w = W.normal_bf16((len(counts), n, k), 0.05, (7071, seed, 1))
    p, s, g = oracle.quantize(w)
    y_ref, d = oracle.grouped_gemm(x, off, p, s, g)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    with EnvOverride(**env):
        y = torch.full((int(off[-1]), n), float("nan"), dtype=torch.float32, device="cuda")
        nv.grouped_gemm(dev(x), dev(off), qw, out_dtype=torch.float32, out=y)
        torch.cuda.synchronize()
    check_close(y, y_ref, d, "grouped %s %s" % (counts, family))
