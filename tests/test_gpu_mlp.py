"""The MoE MLP in one persistent launch (nvfp4_grouped_mlp) against the
oracle's chain and against the two separate launches.

"The FP4 Frontier", Finding 5 recommends fusing the gate_up GEMM, SiLU and the
down GEMM into a single persistent kernel.  Here the launch's workgroups first
compute every gate_up tile (h = SiLU(gate) * up, stored with device-scope
stores), then every down tile; a down tile waits, by bounded polling, until
all gate_up tiles of its row tile are stored.  The kernels and summation
orders are those of nvfp4_grouped_gemm_swiglu followed by nvfp4_grouped_gemm
without a K split, so h and y must equal that two-launch result bit for bit; both are also
checked against the oracle (the down product's reference takes the GPU's h,
as the chain test of the combine does).  Tolerances: FP32 output 1e-5, BF16
4e-3 of the error scale.

The give-up path of the bounded wait is forced from the host (a wait target
no count reaches and a tiny poll limit): the launch must end normally and
report NVFP4_DSTATUS_WAIT_TIMEOUT, with h still complete.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (BF16_TOL, EnvOverride, check_close, dev, host, normalized_error,
                         output_values, require_gpu, segments_of, stratified_positions)

pytestmark = pytest.mark.gpu


def bits(t):
    return host(t).view(np.uint16 if t.dtype == torch.bfloat16 else np.uint32).copy()


def make_case(counts, d_model, d_ff, seed):
    counts = list(counts)
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    rows = int(off[-1])
    x = W.normal_bf16((rows, d_model), 1.0, (313, seed, 0))
    wu = W.normal_bf16((E, 2 * d_ff, d_model), 0.05, (313, seed, 1))
    wd = W.normal_bf16((E, d_model, d_ff), 0.05, (313, seed, 2))
    pu, su, gu = oracle.quantize(wu)
    pd, sd, gd = oracle.quantize(wd)
    return dict(off=off, rows=rows, x=x, pu=pu, su=su, gu=gu, pd=pd, sd=sd, gd=gd,
                d_model=d_model, d_ff=d_ff, E=E)


def run_both(nv, c, out_dtype):
    qu = nv.QuantizedWeight(dev(c["pu"]), dev(c["su"]), dev(c["gu"]))
    qd = nv.QuantizedWeight(dev(c["pd"]), dev(c["sd"]), dev(c["gd"]))
    x, offs = dev(c["x"]), dev(c["off"])
    rows, d_model, d_ff = c["rows"], c["d_model"], c["d_ff"]
    h = torch.full((rows, d_ff), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((rows, d_model), float("nan"), dtype=out_dtype, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    nv.grouped_mlp(x, offs, qu, qd, out=y, h=h, out_dtype=out_dtype, d_status=st)
    # the fused launch never splits K; the separate launches, told not to
    # either, run the same kernel with the same summation order
    with EnvOverride(NVFP4_SPLITK=1):
        h2 = nv.grouped_gemm_swiglu(x, offs, qu)
        y2 = nv.grouped_gemm(h2, offs, qd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return h, y, h2, y2, int(host(st)[0])


CASES = [
    # counts, d_model, d_ff: ~64 rows/expert with one empty expert (64-row
    # tiles, 8 waves x 256 columns); ~16 rows/expert (32-row tiles, 4 waves x
    # 128 columns); one expert holding every row; ragged tiles
    ([70, 0, 5, 33, 120, 64, 1, 40], 512, 256),
    ([16, 17, 15, 14, 18, 16, 0, 16, 20, 12, 16, 16], 512, 256),
    ([0, 0, 200, 0], 256, 128),
    ([3, 66, 129, 7], 384, 192),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("counts,d_model,d_ff", CASES, ids=["c%d" % i for i in range(len(CASES))])
def test_fused_equals_two_launches_and_oracle(counts, d_model, d_ff, out_dtype):
    nv = require_gpu()
    c = make_case(counts, d_model, d_ff, seed=sum(counts) + d_model)
    assert nv.nvfp4_grouped_mlp_kernel_name(c["rows"], c["E"], d_model, d_ff).startswith(
        "nvfp4::gemm_kp_kernel<")
    h, y, h2, y2, st = run_both(nv, c, out_dtype)
    assert st == 0
    assert np.array_equal(bits(h), bits(h2)), "h differs from the SiLU(gate) * up launch"
    assert np.array_equal(bits(y), bits(y2)), "y differs from the down launch"
    h_ref, dh = oracle.grouped_gemm_swiglu(c["x"], c["off"], c["pu"], c["su"], c["gu"])
    check_close(h, h_ref, dh, "fused h")
    y_ref, dy = oracle.grouped_gemm(host(h), c["off"], c["pd"], c["sd"], c["gd"])
    check_close(y, y_ref, dy, "fused y")


@pytest.mark.parametrize("grid", [1, 3, 8])
def test_multi_round(grid):
    """Few workgroups: each walks many gate_up and down units (rounds, the
    cross-unit prefetch, waits on tiles of its own earlier rounds)."""
    nv = require_gpu()
    c = make_case([70, 0, 5, 33, 120, 64, 1, 40], 512, 256, seed=grid)
    with EnvOverride(NVFP4_GRID=grid):
        h, y, h2, y2, st = run_both(nv, c, torch.float32)
    assert st == 0
    assert np.array_equal(bits(h), bits(h2))
    assert np.array_equal(bits(y), bits(y2))
    y_ref, dy = oracle.grouped_gemm(host(h), c["off"], c["pd"], c["sd"], c["gd"])
    check_close(y, y_ref, dy, "fused y, grid %d" % grid)


def test_full_size_zipf():
    """The skewed MoE layer at full size (64 experts, 512 tokens top-8 with
    Zipf(1.2) counts, d_model 6144, d_ff 2048, the workload generators' own
    inputs and weights): bit-identical to the two launches, and one output
    in every 16 x 64 block of every expert's rows of h and y against the
    oracle."""
    nv = require_gpu()
    r, x, wu = W.moe_zipf_up_inputs()
    pu, su, gu = oracle.quantize(wu)
    del wu
    _, _, wd = W.moe_zipf_down_inputs()
    pd, sd, gd = oracle.quantize(wd)
    del wd
    off = r.offsets.astype(np.int32)
    c = dict(off=off, rows=r.rows, x=x, pu=pu, su=su, gu=gu, pd=pd, sd=sd, gd=gd,
             d_model=6144, d_ff=2048, E=r.num_experts)
    h, y, h2, y2, st = run_both(nv, c, torch.bfloat16)
    assert st == 0
    assert np.array_equal(bits(h), bits(h2))
    assert np.array_equal(bits(y), bits(y2))
    hv, yv = output_values(h), output_values(y)
    assert np.isfinite(hv).all() and np.isfinite(yv).all(), "a routed row was not written"
    rr, cc = stratified_positions(segments_of(off), 2048, seed=5)
    h_ref, dh = oracle.grouped_gemm_swiglu_sampled(x, off, pu, su, gu, rr, cc)
    assert normalized_error(hv[rr, cc], h_ref, dh) <= BF16_TOL, "h samples"
    rr, cc = stratified_positions(segments_of(off), 6144, seed=6)
    y_ref, dy = oracle.grouped_gemm_sampled(host(h), off, pd, sd, gd, rr, cc)
    assert normalized_error(yv[rr, cc], y_ref, dy) <= BF16_TOL, "y samples"


def test_wait_give_up_path_ends_and_reports():
    """Forced from the host: every down tile waits for one more gate_up tile
    than exists, with a poll limit of 16.  The launch ends, the status word
    carries NVFP4_DSTATUS_WAIT_TIMEOUT, and h (written before any wait) is
    complete."""
    nv = require_gpu()
    c = make_case([70, 0, 5, 33, 120, 64, 1, 40], 512, 256, seed=77)
    with EnvOverride(NVFP4_MLP_WAIT_EXTRA=1, NVFP4_MLP_SPIN=16):
        h, y, h2, y2, st = run_both(nv, c, torch.float32)
    assert st & nv.DSTATUS_WAIT_TIMEOUT
    assert np.array_equal(bits(h), bits(h2))
    # the next call, with the normal target, is clean again
    h, y, h2, y2, st = run_both(nv, c, torch.float32)
    assert st == 0 and np.array_equal(bits(y), bits(y2))


def test_unsupported_shape_raises():
    nv = require_gpu()
    c = make_case([8, 8], 96, 64, seed=3)  # d_model % 64 != 0
    qu = nv.QuantizedWeight(dev(c["pu"]), dev(c["su"]), dev(c["gu"]))
    qd = nv.QuantizedWeight(dev(c["pd"]), dev(c["sd"]), dev(c["gd"]))
    with pytest.raises(nv.NVFP4Error) as e:
        nv.grouped_mlp(dev(c["x"]), dev(c["off"]), qu, qd)
    assert e.value.status == 3  # NVFP4_ERR_UNSUPPORTED


def test_graph_replay():
    """Captured in a HIP graph, the fused launch (its count zeroing is a fill
    kernel, no memset node) replays to the eager bits, with eager work in
    between, and every replay matches the oracle."""
    from test_gpu_graph import replay_and_compare
    nv = require_gpu()
    c = make_case([70, 0, 5, 33, 120, 64, 1, 40], 512, 256, seed=91)
    qu = nv.QuantizedWeight(dev(c["pu"]), dev(c["su"]), dev(c["gu"]))
    qd = nv.QuantizedWeight(dev(c["pd"]), dev(c["sd"]), dev(c["gd"]))
    x, offs = dev(c["x"]), dev(c["off"])
    h = torch.empty((c["rows"], 256), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((c["rows"], 512), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    h_ref, dh = oracle.grouped_gemm_swiglu(c["x"], c["off"], c["pu"], c["su"], c["gu"])
    y_ref = []

    def fn():
        nv.grouped_mlp(x, offs, qu, qd, out=y, h=h, out_dtype=torch.float32, d_status=st)

    def check(outs):
        check_close(h, h_ref, dh, "replayed h")
        if not y_ref:
            y_ref.extend(oracle.grouped_gemm(host(h), c["off"], c["pd"], c["sd"], c["gd"]))
        check_close(y, y_ref[0], y_ref[1], "replayed y")
        assert int(host(st)[0]) == 0
    replay_and_compare(fn, [h, y], check)
