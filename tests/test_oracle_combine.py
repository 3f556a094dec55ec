"""Pins of the oracle's MoE combine (out[t] = sum_j w[t, j] y[rows[t, j]]):
against a dense combine matrix multiplied with numpy's matmul, against
torch's index_add, and its error scale against the triangle inequality."""
import numpy as np
import torch

import oracle


def case(seed, tokens=37, topk=4, rows=150, n=24):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((rows, n))
    token_rows = np.stack([rng.choice(rows, topk, replace=False) for _ in range(tokens)])
    token_rows[3, 1] = -1  # a slot with no row
    w = rng.random((tokens, topk))
    return y, token_rows, w


def test_matches_dense_combine_matrix():
    y, tr, w = case(1)
    c = np.zeros((tr.shape[0], y.shape[0]))
    for t in range(tr.shape[0]):
        for j in range(tr.shape[1]):
            if tr[t, j] >= 0:
                c[t, tr[t, j]] += w[t, j]
    out, _ = oracle.moe_combine(y, tr, w)
    np.testing.assert_allclose(out, c @ y, rtol=1e-12, atol=1e-12)


def test_matches_torch_index_add():
    y, tr, w = case(2)
    tokens, topk = tr.shape
    src = torch.zeros((tokens * topk, y.shape[1]), dtype=torch.float64)
    idx = torch.arange(tokens).repeat_interleave(topk)
    for t in range(tokens):
        for j in range(topk):
            if tr[t, j] >= 0:
                src[t * topk + j] = torch.from_numpy(y[tr[t, j]]) * w[t, j]
    want = torch.zeros((tokens, y.shape[1]), dtype=torch.float64).index_add_(0, idx, src)
    out, _ = oracle.moe_combine(y, tr, w)
    np.testing.assert_allclose(out, want.numpy(), rtol=1e-12, atol=1e-12)


def test_error_scale_bounds_output():
    y, tr, w = case(3)
    out, d = oracle.moe_combine(y, tr, w)
    assert (np.abs(out) <= d * (1 + 1e-12)).all()
    assert (d[3] > 0).all()  # the token with an empty slot still sums its other rows
