"""Launches captured in a HIP graph (torch.cuda.CUDAGraph) replay to the same
bits as eager launches, and every replay matches the oracle.

Launch overhead dominates small GEMMs and the pages chain layers with
programmatic launch control ("The FP4 Frontier", Finding 5); the HIP analogue
is to capture a sequence of launches once and replay it.  The library
allocates nothing and enqueues no memset node (workspaces are caller-provided
and zeroed by a fill kernel), and the split-K counters return to zero at the
end of every launch, so a captured launch can be replayed.  Each test replays
several times with eager work and synchronizations in between and checks
every replay against the eager result and against the oracle.  The binding's
workspaces are per (device, stream); a capture that needs a larger one gets a
fresh buffer zeroed inside the graph, and buffers a graph may hold are never
freed (tests at the end).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import EnvOverride, check_close, dev, host, output_values, require_gpu
from test_gpu_combine import routing

pytestmark = pytest.mark.gpu


def bits(t):
    return host(t).view(np.uint16 if t.dtype == torch.bfloat16 else np.uint32).copy()


def capture(fn, warm=True):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    if warm:
        with torch.cuda.stream(s):
            fn()  # warm-up on a side stream
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_compare(fn, outs, check, reps=4):
    """fn() enqueues the launches writing `outs`; every graph replay must
    equal the eager result bit for bit and pass check(outs) (the oracle)."""
    fn()
    torch.cuda.synchronize()
    check(outs)
    want = [bits(o) for o in outs]
    g = capture(fn)
    for i in range(reps):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0x5A)
        _ = torch.ones(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(bits(o), w), "replay %d differs from the eager launch" % i
        check(outs)


@pytest.mark.parametrize("m,gemv", [(1, "1"), (1, "0"), (16, "1"), (64, "1")])
def test_dense_decode_replay(m, gemv):
    # M = 1 takes the dot-product kernel; with it switched off (and at
    # M = 64) the decode runs split-K: partial tiles and arrival counters in
    # the workspace, reset by the last split of each tile
    nv = require_gpu()
    w = W.decode_weight()
    p, s, g = oracle.quantize(w)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(np.atleast_1d(g).astype(np.float32)))
    xh = W.decode_act(m)
    x = dev(xh)
    y = torch.empty((m, qw.n), dtype=torch.bfloat16, device="cuda")
    y_ref, d = oracle.gemm(xh, p, s, np.float32(np.atleast_1d(g)[0]))
    with EnvOverride(NVFP4_GEMV=gemv):
        replay_and_compare(lambda: nv.gemm(x, qw, out=y), [y],
                           lambda o: check_close(o[0], y_ref, d, "decode m=%d" % m))


def test_moe_layer_chain_replay():
    """A routed MoE layer captured as one graph: gather + gate_up with
    SiLU(gate) * up -> grouped down projection -> router-weighted combine;
    every replay against the oracle's chain (each stage fed the previous
    stage's eager output, which the replay reproduces bit for bit)."""
    nv = require_gpu()
    tokens, topk, E, d_model, d_ff = 48, 4, 8, 512, 256
    row_token, off, token_rows, wts = routing(tokens, topk, E, seed=777)
    x_tok = W.normal_bf16((tokens, d_model), 1.0, (99, 2, 1))
    wu = W.normal_bf16((E, 2 * d_ff, d_model), 0.05, (99, 2, 2))
    wd = W.normal_bf16((E, d_model, d_ff), 0.05, (99, 2, 3))
    pu, su, gu = oracle.quantize(wu)
    pd, sd, gd = oracle.quantize(wd)
    qu = nv.QuantizedWeight(dev(pu), dev(su), dev(gu))
    qd = nv.QuantizedWeight(dev(pd), dev(sd), dev(gd))
    offs, xt, rt, tr, wt = dev(off), dev(x_tok), dev(row_token), dev(token_rows), dev(wts)
    rows = int(off[-1])
    h = torch.empty((rows, d_ff), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, d_model), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((tokens, d_model), dtype=torch.bfloat16, device="cuda")

    def step():
        nv.grouped_gemm_gather(xt, rt, offs, qu, act="swiglu", out=h)
        nv.grouped_gemm(h, offs, qd, out=y)
        nv.moe_combine(y, tr, wt, out=out)

    h_ref, dh = oracle.grouped_gemm_swiglu(x_tok[row_token], off, pu, su, gu)

    def check(o):
        hh, yy, oo = o
        check_close(hh, h_ref, dh, "chain gate_up")
        y_ref, dy = oracle.grouped_gemm(host(hh), off, pd, sd, gd)
        check_close(yy, y_ref, dy, "chain down")
        o_ref, do = oracle.moe_combine(output_values(yy), token_rows, wts)
        check_close(oo, o_ref, do, "chain combine")
    replay_and_compare(step, [h, y, out], check)


def test_quantize_replay():
    nv = require_gpu()
    b, n, k = 3, 128, 256
    wh = W.normal_bf16((b, n, k), 0.05, (99, 1, 0))
    w = dev(wh)
    packed = torch.empty((b, n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((b, n, k // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty((b,), dtype=torch.float32, device="cuda")
    nbytes = nv.nvfp4_quantize_workspace_size(b, n, k)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    p_ref, s_ref, g_ref = oracle.quantize(wh)

    def run():
        assert nv.nvfp4_quantize(w, b, n, k, packed, scales, g, None, ws, nbytes) == 0

    def check(o):
        assert np.array_equal(host(o[0]), p_ref)
        assert np.array_equal(host(o[1]), s_ref)
        assert np.array_equal(host(o[2]).view(np.uint32), g_ref.view(np.uint32))
    replay_and_compare(run, [packed, scales, g], check)


def _decode_case(nv, m, n, k, seed):
    x = W.normal_bf16((m, k), 1.0, (98, seed, 0))
    w = W.normal_bf16((n, k), 0.03, (98, seed, 1))
    p, s, g = oracle.quantize(w)
    g = np.atleast_1d(g).astype(np.float32)
    qw = nv.QuantizedWeight(dev(p), dev(s), dev(g))
    y_ref, d = oracle.gemm(x, p, s, g[0])
    return dev(x), qw, y_ref, d


def test_capture_first_then_eager_growth_then_replay():
    """A split-K launch captured with no eager call on its stream first gets a
    workspace zeroed inside the graph; eager launches of a larger shape (which
    grow the eager workspaces) and on the capture stream itself do not disturb
    the replays."""
    nv = require_gpu()
    xs, qs, ys_ref, ds = _decode_case(nv, 48, 2048, 4096, seed=1)
    xl, ql, yl_ref, dl = _decode_case(nv, 64, 4096, 7168, seed=2)
    ys = torch.empty((48, 2048), dtype=torch.float32, device="cuda")
    yl = torch.empty((64, 4096), dtype=torch.float32, device="cuda")
    with EnvOverride(NVFP4_GEMV=0):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=side):
            nv.gemm(xs, qs, out=ys, out_dtype=torch.float32)
        torch.cuda.synchronize()
        for i in range(3):
            nv.gemm(xl, ql, out=yl, out_dtype=torch.float32)  # eager, larger shape
            with torch.cuda.stream(side):
                nv.gemm(xl, ql, out=yl, out_dtype=torch.float32)  # eager on the capture stream
            torch.cuda.synchronize()
            check_close(yl, yl_ref, dl, "eager large %d" % i)
            ys.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            check_close(ys, ys_ref, ds, "replay %d" % i)


def test_streams_keep_separate_workspaces():
    """Split-K launches issued concurrently on two streams through the
    binding use separate workspaces (separate tile counters)."""
    nv = require_gpu()
    xa, qa, ya_ref, da = _decode_case(nv, 40, 1024, 4096, seed=3)
    xb, qb, yb_ref, db = _decode_case(nv, 24, 1024, 4096, seed=4)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ya = torch.empty((40, 1024), dtype=torch.float32, device="cuda")
    yb = torch.empty((24, 1024), dtype=torch.float32, device="cuda")
    with EnvOverride(NVFP4_GEMV=0, NVFP4_SPLITK=4):
        for _ in range(20):
            with torch.cuda.stream(sa):
                nv.gemm(xa, qa, out=ya, out_dtype=torch.float32)
            with torch.cuda.stream(sb):
                nv.gemm(xb, qb, out=yb, out_dtype=torch.float32)
        torch.cuda.synchronize()
    check_close(ya, ya_ref, da, "stream a")
    check_close(yb, yb_ref, db, "stream b")
