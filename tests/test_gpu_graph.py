"""Launches captured in a HIP graph (torch.cuda.CUDAGraph) replay to the same
bits as eager launches.

Launch overhead dominates small GEMMs and the pages chain layers with
programmatic launch control ("The FP4 Frontier", Finding 5); the HIP analogue
is to capture a sequence of launches once and replay it.  The library
allocates nothing and enqueues no memset node (workspaces are caller-provided
and zeroed once by a fill kernel), and the split-K counters return to zero at
the end of every launch, so a captured launch can be replayed.  Each test
replays several times with eager work and synchronizations in between and
checks every replay against the eager result.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import dev, host, require_gpu

pytestmark = pytest.mark.gpu


def bits(t):
    return host(t).view(np.uint16 if t.dtype == torch.bfloat16 else np.uint32).copy()


def replay_and_compare(fn, outs, reps=4):
    """fn() enqueues the launches writing `outs`; compare graph replays with
    the eager result."""
    fn()  # eager (also allocates the cached workspace before capture)
    torch.cuda.synchronize()
    want = [bits(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for i in range(reps):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0x5A)
        _ = torch.ones(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(bits(o), w), "replay %d differs from the eager launch" % i


@pytest.mark.parametrize("m,gemv", [(1, "1"), (1, "0"), (16, "1")])
def test_dense_decode_replay(m, gemv):
    # M = 1 takes the dot-product kernel; with it switched off (and at
    # M = 16) the decode runs split-K: partial tiles and arrival counters in
    # the workspace, reset by the last split of each tile
    nv = require_gpu()
    w = W.decode_weight()
    p, s, g = oracle.quantize(w)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(np.atleast_1d(g).astype(np.float32)))
    x = dev(W.decode_act(m))
    y = torch.empty((m, qw.n), dtype=torch.bfloat16, device="cuda")
    old = os.environ.get("NVFP4_GEMV")
    os.environ["NVFP4_GEMV"] = gemv
    try:
        replay_and_compare(lambda: nv.gemm(x, qw, out=y), [y])
    finally:
        if old is None:
            os.environ.pop("NVFP4_GEMV", None)
        else:
            os.environ["NVFP4_GEMV"] = old


def test_grouped_and_swiglu_chain_replay():
    # a small MoE step: gate_up with SiLU(gate) * up, then a grouped launch
    # reading its output, captured as one graph
    nv = require_gpu()
    counts = [5, 0, 19, 2, 33, 1]
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    rows = int(off[-1])
    x = dev(W.normal_bf16((rows, 512), 1.0, (99, 0, 1)))
    wu = W.normal_bf16((E, 256, 512), 0.05, (99, 0, 2))
    wd = W.normal_bf16((E, 384, 128), 0.05, (99, 0, 3))
    pu, su, gu = oracle.quantize(wu)
    pd, sd, gd = oracle.quantize(wd)
    qu = nv.QuantizedWeight(dev(pu), dev(su), dev(gu))
    qd = nv.QuantizedWeight(dev(pd), dev(sd), dev(gd))
    offs = dev(off)
    h = torch.empty((rows, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, 384), dtype=torch.bfloat16, device="cuda")

    def step():
        nv.grouped_gemm_swiglu(x, offs, qu, out=h)
        nv.grouped_gemm(h, offs, qd, out=y)
    replay_and_compare(step, [h, y])


def test_quantize_replay():
    nv = require_gpu()
    b, n, k = 3, 128, 256
    w = dev(W.normal_bf16((b, n, k), 0.05, (99, 1, 0)))
    packed = torch.empty((b, n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((b, n, k // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty((b,), dtype=torch.float32, device="cuda")
    nbytes = nv.nvfp4_quantize_workspace_size(b, n, k)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def run():
        assert nv.nvfp4_quantize(w, b, n, k, packed, scales, g, None, ws, nbytes) == 0
    replay_and_compare(run, [packed, scales, g])
