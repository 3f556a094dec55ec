"""GPU parity of the MoE combine and of the whole routed MoE MLP chain.

The combine is the scatter half of the routing-aware MoE layer ("The FP4
Frontier", Finding 5): every token's output is the router-weighted sum of
the down projection's outputs of its top-k routed rows.  The oracle is the
definition (oracle.moe_combine, FP64); the error is normalized by
D = sum_j |w * y| as for the GEMMs: FP32 output within 1e-5, BF16 within 4e-3.
The chain test runs gather + SiLU(gate) * up, the down projection and the
combine, and checks every stage against the oracle fed with the previous
stage's device output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_close, dev, host, output_values, require_gpu

pytestmark = pytest.mark.gpu


def routing(tokens, topk, E, seed):
    """Expert-ordered routing: row_token (routed row -> token), offsets, and
    token_rows [tokens, topk] (token, slot -> routed row) with FP32 weights."""
    rng = np.random.default_rng(np.random.SeedSequence([101, seed]))
    choices = np.stack([rng.choice(E, topk, replace=False) for _ in range(tokens)])
    tok = np.repeat(np.arange(tokens), topk)
    order = np.lexsort((tok, choices.reshape(-1)))
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(np.bincount(choices.reshape(-1), minlength=E))
    token_rows = np.empty(tokens * topk, np.int32)
    token_rows[order] = np.arange(tokens * topk, dtype=np.int32)
    wts = rng.random((tokens, topk)).astype(np.float32)
    wts /= wts.sum(axis=1, keepdims=True)
    return tok[order].astype(np.int32), off, token_rows.reshape(tokens, topk), wts


def run_combine(nv, y, token_rows, wts, out_dtype, d_status=None):
    out = torch.full((token_rows.shape[0], y.shape[1]), float("nan"), dtype=out_dtype,
                     device="cuda")
    r = nv.moe_combine(y, dev(token_rows), dev(wts), out=out, d_status=d_status)
    torch.cuda.synchronize()
    return r


def y_values(y):
    return output_values(y)


CASES = [
    # tokens, topk, n, y dtype
    (1, 1, 8, torch.bfloat16),
    (7, 2, 96, torch.float32),
    (33, 8, 2048, torch.bfloat16),        # one full column chunk
    (20, 6, 2056, torch.float32),         # a second, ragged chunk of 8 columns
    (5, 64, 4104, torch.bfloat16),        # topk at the limit, three chunks
]


@pytest.mark.parametrize("tokens,topk,n,ydt", CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_against_oracle(tokens, topk, n, ydt, out_dtype):
    nv = require_gpu()
    _, _, token_rows, wts = routing(tokens, topk, max(topk, 8), seed=tokens * 100 + topk)
    yb = W.normal_bf16((tokens * topk, n), 1.0, (101, tokens, n))
    y = dev(yb) if ydt == torch.bfloat16 else dev(yb).float()
    out = run_combine(nv, y, token_rows, wts, out_dtype)
    ref, d = oracle.moe_combine(y_values(y), token_rows, wts)
    check_close(out, ref, d, "combine %d x top-%d n=%d" % (tokens, topk, n))


def test_empty_slots_and_reused_rows():
    # negative ids are empty slots; a row may feed several tokens and slots
    nv = require_gpu()
    rng = np.random.default_rng(5)
    token_rows = rng.integers(-1, 12, size=(40, 5)).astype(np.int32)
    token_rows[3] = -1          # a token with no routed row: exact zeros
    wts = rng.standard_normal((40, 5)).astype(np.float32)
    y = dev(W.normal_bf16((12, 264), 1.0, (101, 5, 1))).float()
    out = run_combine(nv, y, token_rows, wts, torch.float32)
    ref, d = oracle.moe_combine(y_values(y), token_rows, wts)
    check_close(out, ref, d, "empty slots")
    assert (output_values(out)[3] == 0).all()


def test_out_of_range_row_sets_status():
    nv = require_gpu()
    _, _, token_rows, wts = routing(16, 4, 8, seed=3)
    bad = token_rows.copy()
    bad[2, 1] = 64              # rows == 64: one past the end
    y = dev(W.normal_bf16((64, 128), 1.0, (101, 3, 1)))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_combine(nv, y, bad, wts, torch.float32, d_status=status)
    assert int(status.item()) & nv.DSTATUS_BAD_INDEX
    skip = bad.copy()
    skip[2, 1] = -1             # the bad slot contributes nothing
    ref, d = oracle.moe_combine(y_values(y), skip, wts)
    check_close(out, ref, d, "bad index")


def test_bitwise_reproducible():
    nv = require_gpu()
    _, _, token_rows, wts = routing(128, 8, 64, seed=4)
    y = dev(W.normal_bf16((1024, 2048), 1.0, (101, 4, 1)))
    a = host(run_combine(nv, y, token_rows, wts, torch.bfloat16)).copy()
    b = host(run_combine(nv, y, token_rows, wts, torch.bfloat16))
    assert np.array_equal(a, b)


def test_zero_tokens_is_a_no_op():
    nv = require_gpu()
    y = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((0, 16), dtype=torch.bfloat16, device="cuda")
    nv.moe_combine(y, torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                   torch.zeros((0, 2), dtype=torch.float32, device="cuda"), out=out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("tokens,topk,E,d_model,d_ff", [
    (24, 4, 8, 256, 128),        # small: every stage checked in full
    (128, 8, 64, 1024, 512),     # ~16 routed rows per expert, decode-like
])
def test_moe_mlp_chain(tokens, topk, E, d_model, d_ff):
    """gather + gate_up with SiLU(gate) * up -> down projection -> combine,
    each stage against the oracle fed the previous stage's device output."""
    nv = require_gpu()
    row_token, off, token_rows, wts = routing(tokens, topk, E, seed=tokens + E)
    x_tok = W.normal_bf16((tokens, d_model), 1.0, (101, tokens, 1))
    wu = W.normal_bf16((E, 2 * d_ff, d_model), 0.05, (101, tokens, 2))
    wd = W.normal_bf16((E, d_model, d_ff), 0.05, (101, tokens, 3))
    pu, su, gu = oracle.quantize(wu)
    pd, sd, gd = oracle.quantize(wd)
    qu = nv.QuantizedWeight(dev(pu), dev(su), dev(gu))
    qd = nv.QuantizedWeight(dev(pd), dev(sd), dev(gd))
    offs = dev(off)
    h = nv.grouped_gemm_gather(dev(x_tok), dev(row_token), offs, qu, act="swiglu")
    y = nv.grouped_gemm(h, offs, qd)
    out = nv.moe_combine(y, dev(token_rows), dev(wts))
    torch.cuda.synchronize()
    h_ref, dh = oracle.grouped_gemm_swiglu(x_tok[row_token], off, pu, su, gu)
    check_close(h, h_ref, dh, "chain gate_up")
    y_ref, dy = oracle.grouped_gemm(host(h), off, pd, sd, gd)
    check_close(y, y_ref, dy, "chain down")
    o_ref, do = oracle.moe_combine(y_values(y), token_rows, wts)
    check_close(out, o_ref, do, "chain combine")
