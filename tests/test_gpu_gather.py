"""GPU parity of the grouped GEMM that gathers its rows through an index.

The routing-aware form of the grouped GEMM ("The FP4 Frontier", Finding 5:
one grouped GEMM over all experts of the MoE layer): routed row r reads
token row x[row_index[r]] instead of a pre-permuted copy.  The oracle side is
the definition itself -- gather with numpy indexing, then the grouped GEMM
oracle.  Because the kernel sees the same bytes in the same order, the
gathered launch must also equal, bit for bit, the plain launch on the
pre-permuted activations.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (BF16_TOL, F32_TOL, check_close, dev, host, normalized_error,
                         output_values, require_gpu, segments_of,
                         stratified_positions)

pytestmark = pytest.mark.gpu


def routed(tokens, topk, E, k, seed, n=None):
    """Token matrix, routing (row_token, offsets) and weights for a small case."""
    rng = np.random.default_rng(np.random.SeedSequence([100, seed]))
    choices = np.stack([rng.choice(E, topk, replace=False) for _ in range(tokens)])
    tok = np.repeat(np.arange(tokens), topk)
    exp = choices.reshape(-1)
    order = np.lexsort((tok, exp))
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(np.bincount(exp, minlength=E))
    row_token = tok[order].astype(np.int32)
    x_tok = W.normal_bf16((tokens, k), 1.0, (100, seed, 1))
    return x_tok, row_token, off


def run_gather(nv, x_tok, row_token, off, qw, out_dtype, act="none", d_status=None):
    n = qw.n // 2 if act == "swiglu" else qw.n
    out = torch.full((len(row_token), n), float("nan"), dtype=out_dtype, device="cuda")
    y = nv.grouped_gemm_gather(dev(x_tok), dev(row_token), dev(off), qw, act=act,
                               out_dtype=out_dtype, out=out, d_status=d_status)
    torch.cuda.synchronize()
    return y


def to_qw(nv, p, s, g):
    return nv.QuantizedWeight(dev(p), dev(s), dev(g))


CASES = [
    # tokens, topk, experts, n, k
    (20, 4, 8, 128, 512),      # ~10 rows / expert: 16-row tiles
    (48, 4, 8, 320, 640),      # ~24 rows / expert: 32-row tiles, ragged column tile
    (96, 6, 8, 256, 1024),     # ~72 rows / expert: 64-row tiles
    (30, 2, 4, 96, 80),        # k % 64 != 0: fallback kernel
]


@pytest.mark.parametrize("tokens,topk,E,n,k", CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_against_oracle(tokens, topk, E, n, k, out_dtype):
    nv = require_gpu()
    x_tok, row_token, off = routed(tokens, topk, E, k, seed=tokens + n)
    w = W.normal_bf16((E, n, k), 0.05, (100, tokens + n, 2))
    p, s, g = oracle.quantize(w)
    y_ref, d = oracle.grouped_gemm(x_tok[row_token], off, p, s, g)
    y = run_gather(nv, x_tok, row_token, off, to_qw(nv, p, s, g), out_dtype)
    check_close(y, y_ref, d, "gather %d tokens n=%d k=%d" % (tokens, n, k))


@pytest.mark.parametrize("tokens,topk,E,n,k", CASES)
def test_swiglu_against_oracle(tokens, topk, E, n, k):
    nv = require_gpu()
    x_tok, row_token, off = routed(tokens, topk, E, k, seed=tokens + n + 1)
    w = W.normal_bf16((E, n, k), 0.05, (100, tokens + n, 3))
    p, s, g = oracle.quantize(w)
    h_ref, dh = oracle.grouped_gemm_swiglu(x_tok[row_token], off, p, s, g)
    h = run_gather(nv, x_tok, row_token, off, to_qw(nv, p, s, g), torch.float32, act="swiglu")
    check_close(h, h_ref, dh, "gather swiglu %d tokens" % tokens)


@pytest.mark.parametrize("env", [None, "NVFP4_SPLITK=3", "NVFP4_KPCFG=8"])
def test_bitwise_equal_to_prepermuted(env):
    nv = require_gpu()
    x_tok, row_token, off = routed(64, 4, 8, 1536, seed=7)
    w = W.normal_bf16((8, 384, 1536), 0.05, (100, 7, 2))
    p, s, g = oracle.quantize(w)
    qw = to_qw(nv, p, s, g)
    name, val = env.split("=") if env else (None, None)
    old = os.environ.get(name) if name else None
    if name:
        os.environ[name] = val
    try:
        y_g = run_gather(nv, x_tok, row_token, off, qw, torch.float32)
        y_p = nv.grouped_gemm(dev(x_tok[row_token]), dev(off), qw, out_dtype=torch.float32)
        torch.cuda.synchronize()
    finally:
        if name:
            if old is None:
                os.environ.pop(name, None)
            else:
                os.environ[name] = old
    assert np.array_equal(host(y_g).view(np.uint32), host(y_p).view(np.uint32))


def test_out_of_range_index_sets_status_and_reads_zero():
    nv = require_gpu()
    x_tok, row_token, off = routed(24, 3, 6, 576, seed=9)
    bad = row_token.copy()
    bad[5] = len(x_tok)      # one past the end
    bad[17] = -1             # negative
    w = W.normal_bf16((6, 128, 576), 0.05, (100, 9, 2))
    p, s, g = oracle.quantize(w)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = output_values(run_gather(nv, x_tok, bad, off, to_qw(nv, p, s, g), torch.float32,
                                 d_status=status))
    assert int(status.item()) & nv.DSTATUS_BAD_INDEX
    assert (y[5] == 0).all() and (y[17] == 0).all()
    y_ref, d = oracle.grouped_gemm(x_tok[row_token], off, p, s, g)
    keep = np.ones(len(bad), bool)
    keep[[5, 17]] = False
    assert normalized_error(y[keep], y_ref[keep], d[keep]) <= F32_TOL


def test_uniform_16_tokens_per_expert_full_size():
    """The ~16 tok/expert up projection (128 tokens x top-8, N = 4096,
    K = 6144) gathered from the 128-token matrix: bitwise equal to the plain
    launch on the permuted rows, and outputs of every 16 x 64 block against the
    oracle."""
    nv = require_gpu()
    r = W.moe_uniform_routing()
    _, x, w = W.moe_uniform_inputs()
    x_tok = np.empty((r.tokens, x.shape[1]), np.uint16)
    x_tok[r.row_token] = x
    p, s, g = oracle.quantize(w)
    qw = to_qw(nv, p, s, g)
    rt = r.row_token.astype(np.int32)
    y_g = run_gather(nv, x_tok, rt, r.offsets, qw, torch.bfloat16)
    y_p = nv.grouped_gemm(dev(x), dev(r.offsets.astype(np.int32)), qw)
    torch.cuda.synchronize()
    assert np.array_equal(host(y_g), host(y_p))
    yv = output_values(y_g)
    rows, cols = stratified_positions(segments_of(r.offsets), yv.shape[1], seed=31)
    y_ref, d = oracle.grouped_gemm_sampled(x, r.offsets, p, s, g, rows, cols)
    assert normalized_error(yv[rows, cols], y_ref, d) <= BF16_TOL
