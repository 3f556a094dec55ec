"""Seeded synthetic inputs for the NVFP4 W4A16 GEMM workloads.

This module holds no part of the method's arithmetic: it draws random numbers,
rounds them to BF16 bit patterns and builds MoE routings.  Tests feed the same
arrays to the CPU oracle and to the HIP library; the benchmark uses it too.

Workload shapes (from the pages): decode batches of 16-64 tokens per expert
("The FP4 Frontier", section "The Context"), hidden size 7168 and
intermediate sizes 2048 / 6144 ("The FP4 Frontier", Finding 4; "The Tile That
Didn't Fit", section "Broader Implications"), MoE grouped GEMM over all
experts ("The FP4 Frontier", Finding 5).

Random streams: numpy PCG64 seeded by SeedSequence([seed, workload, stream,
...]).  Large tensors are drawn in fixed 4 Mi-element chunks, chunk i from the
i-th spawned child of the stream's SeedSequence, so the bytes do not depend
on how many threads draw them.  Values are drawn in float32 and rounded to
BF16 (round to nearest, ties to even) on the host.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 0
CHUNK = 1 << 22

# workload ids used in the seed sequences
W_SMALL, W_DECODE, W_MOE_UNIFORM, W_MOE_ZIPF, W_LARGE, W_FUZZ = 1, 2, 3, 4, 5, 6
S_WEIGHT, S_ACT, S_ROUTE, S_AUX = 0, 1, 2, 3


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest, ties to even); returns uint16 bits."""
    import torch  # CPU cast only

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, std: float, key) -> np.ndarray:
    """N(0, std^2) float32 array of `shape`, drawn chunk-wise from `key`."""
    total = int(np.prod(shape, dtype=np.int64))
    out = np.empty(total, np.float32)
    nchunks = (total + CHUNK - 1) // CHUNK
    children = np.random.SeedSequence(list(key)).spawn(nchunks)

    def fill(i):
        lo, hi = i * CHUNK, min(total, (i + 1) * CHUNK)
        rng = np.random.default_rng(children[i])
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def normal_bf16(shape, std: float, key) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(shape, std, key))


# ---- routings ---------------------------------------------------------------

@dataclass
class Routing:
    """Tokens routed to experts, rows sorted by (expert, token)."""
    num_experts: int
    tokens: int
    topk: int
    row_token: np.ndarray          # [rows] token index of each routed row
    offsets: np.ndarray            # int32 [E+1] prefix sums of per-expert counts
    counts: np.ndarray = field(init=False)

    def __post_init__(self):
        self.counts = np.diff(self.offsets).astype(np.int64)

    @property
    def rows(self) -> int:
        return int(self.offsets[-1])

    def token_rows(self) -> np.ndarray:
        """int32 [tokens, topk]: the routed rows of each token, in row order."""
        order = np.argsort(self.row_token, kind="stable")
        return order.reshape(self.tokens, self.topk).astype(np.int32)


def _sorted_routing(choices: np.ndarray, num_experts: int) -> Routing:
    tokens, topk = choices.shape
    tok = np.repeat(np.arange(tokens), topk)
    exp = choices.reshape(-1)
    order = np.lexsort((tok, exp))  # primary key expert, then token
    counts = np.bincount(exp, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return Routing(num_experts, tokens, topk, tok[order].astype(np.int64), offsets)


def routing_uniform(tokens: int, topk: int, num_experts: int, excluded, key) -> Routing:
    """Each token picks `topk` distinct experts uniformly among the experts not
    in `excluded` (which therefore stay empty)."""
    rng = np.random.default_rng(np.random.SeedSequence(list(key)))
    allowed = np.array([e for e in range(num_experts) if e not in set(excluded)])
    choices = np.stack([rng.choice(allowed, topk, replace=False) for _ in range(tokens)])
    return _sorted_routing(choices, num_experts)


def routing_zipf(tokens: int, topk: int, num_experts: int, s: float, key,
                 excluded=()) -> Routing:
    """Each token picks `topk` distinct experts, drawn one after another without
    replacement with probability proportional to rank^-s (rank 1..E); ranks map
    to expert ids through a seeded permutation.  Experts in `excluded` get
    probability 0."""
    rng = np.random.default_rng(np.random.SeedSequence(list(key)))
    perm = rng.permutation(num_experts)              # rank r -> expert perm[r]
    w = np.arange(1, num_experts + 1, dtype=np.float64) ** (-s)
    for e in excluded:
        w[np.where(perm == e)[0]] = 0.0
    choices = np.empty((tokens, topk), np.int64)
    for t in range(tokens):
        p = w.copy()
        for j in range(topk):
            r = rng.choice(num_experts, p=p / p.sum())
            choices[t, j] = perm[r]
            p[r] = 0.0
    return _sorted_routing(choices, num_experts)


# ---- the workloads ------------------------------------------------------------

def small_dense():
    """16 x 256 x 512 dense case: weights and activations N(0, 1)."""
    w = normal_bf16((256, 512), 1.0, (SEED, W_SMALL, S_WEIGHT))
    x = normal_bf16((16, 512), 1.0, (SEED, W_SMALL, S_ACT))
    return x, w


def decode_weight(n: int = 4096, k: int = 7168):
    """N(0, 0.02) weight with floor(0.001 * n * k) outliers (x20) at positions
    drawn uniformly without replacement, applied before the BF16 rounding."""
    w = normal_f32((n, k), 0.02, (SEED, W_DECODE, S_WEIGHT))
    count = (n * k) // 1000
    rng = np.random.default_rng(np.random.SeedSequence([SEED, W_DECODE, S_AUX]))
    pos = rng.choice(n * k, size=count, replace=False)
    flat = w.reshape(-1)
    flat[pos] *= np.float32(20.0)
    return f32_to_bf16_bits(w)


def decode_act(m: int, k: int = 7168):
    return normal_bf16((m, k), 1.0, (SEED, W_DECODE, S_ACT, m))


# MoE at ~16 tokens / expert: 128 tokens, top-8, uniform over 60 of 64 experts.
MOE_UNIFORM_EXCLUDED = (7, 23, 39, 55)


def moe_uniform_routing(tokens: int = 128, topk: int = 8, num_experts: int = 64) -> Routing:
    return routing_uniform(tokens, topk, num_experts, MOE_UNIFORM_EXCLUDED,
                           (SEED, W_MOE_UNIFORM, S_ROUTE))


def moe_uniform_inputs(n: int = 4096, k: int = 6144, num_experts: int = 64,
                       tokens: int = 128, topk: int = 8, weights: bool = True):
    """Returns (routing, x [rows, k], w [E, n, k] or None)."""
    r = moe_uniform_routing(tokens, topk, num_experts)
    x_tok = normal_bf16((tokens, k), 1.0, (SEED, W_MOE_UNIFORM, S_ACT))
    x = x_tok[r.row_token]
    w = normal_bf16((num_experts, n, k), 0.02, (SEED, W_MOE_UNIFORM, S_WEIGHT)) if weights else None
    return r, x, w


def moe_zipf_routing(tokens: int = 512, topk: int = 8, num_experts: int = 64, s: float = 1.2,
                     excluded=()) -> Routing:
    return routing_zipf(tokens, topk, num_experts, s, (SEED, W_MOE_ZIPF, S_ROUTE),
                        excluded=excluded)


def moe_zipf_up_inputs(n: int = 4096, k: int = 6144, num_experts: int = 64, tokens: int = 512,
                       topk: int = 8, excluded=(), weights: bool = True):
    r = moe_zipf_routing(tokens, topk, num_experts, excluded=excluded)
    x_tok = normal_bf16((tokens, k), 1.0, (SEED, W_MOE_ZIPF, S_ACT, 0))
    x = x_tok[r.row_token]
    w = normal_bf16((num_experts, n, k), 0.02, (SEED, W_MOE_ZIPF, S_WEIGHT, 0)) if weights else None
    return r, x, w


def moe_zipf_down_inputs(n: int = 6144, k: int = 2048, num_experts: int = 64, tokens: int = 512,
                         topk: int = 8, excluded=(), weights: bool = True):
    """Down projection: the input rows are drawn independently of the up
    projection's output (same routing)."""
    r = moe_zipf_routing(tokens, topk, num_experts, excluded=excluded)
    h = normal_bf16((r.rows, k), 1.0, (SEED, W_MOE_ZIPF, S_ACT, 1))
    w = normal_bf16((num_experts, n, k), 0.02, (SEED, W_MOE_ZIPF, S_WEIGHT, 1)) if weights else None
    return r, h, w


def large_dense(m: int = 8192, n: int = 8192, k: int = 8192):
    w = normal_bf16((n, k), 0.02, (SEED, W_LARGE, S_WEIGHT))
    x = normal_bf16((m, k), 1.0, (SEED, W_LARGE, S_ACT))
    return x, w


def fuzz_weight(n: int, k: int, case: str, key_extra: int = 0):
    """Weights that stress the encoder: subnormal BF16s, zero blocks, signed
    zeros, a single huge outlier, values on rounding ties."""
    key = (SEED, W_FUZZ, S_WEIGHT, key_extra)
    rng = np.random.default_rng(np.random.SeedSequence(list(key)))
    if case == "normal":
        return normal_bf16((n, k), 1.0, key)
    if case == "subnormal":
        # BF16 subnormals and tiny normals only (exponent field 0..3)
        bits = rng.integers(0, 1 << 9, size=(n, k), dtype=np.uint32)
        sign = rng.integers(0, 2, size=(n, k), dtype=np.uint32) << 15
        return (bits | sign).astype(np.uint16)
    if case == "zeros":
        w = normal_bf16((n, k), 1.0, key)
        blocks = w.reshape(n, k // 16, 16)
        mask = rng.random((n, k // 16)) < 0.3
        blocks[mask] = 0
        negz = rng.random((n, k // 16)) < 0.1
        blocks[negz & mask, 0] = 0x8000
        return blocks.reshape(n, k)
    if case == "outlier":
        w = normal_f32((n, k), 0.01, key)
        w[rng.integers(0, n), rng.integers(0, k)] = np.float32(3.0e4)
        return f32_to_bf16_bits(w)
    if case == "ties":
        # every block holds +-6 * 2^j and values that land on E2M1 midpoints
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, 1.0, 3.0, 4.0,
                         0.5, 1.5, 2.0, 6.0], np.float32)
        j = rng.integers(-20, 20, size=(n, k // 16, 1)).astype(np.float32)
        sign = np.where(rng.random((n, k // 16, 16)) < 0.5, -1.0, 1.0).astype(np.float32)
        w = (mids[None, None, :] * np.exp2(j) * sign).reshape(n, k)
        return f32_to_bf16_bits(w)
    if case == "wide":
        # per-row magnitudes spread over ~60 binades
        e = rng.integers(-60, 60, size=(n, 1)).astype(np.float32)
        return f32_to_bf16_bits(normal_f32((n, k), 1.0, key) * np.exp2(e))
    raise ValueError(case)
