"""Host model of the grouped GEMM's work-unit numbering and of the split-K
workspace bound, run on the CPU (no kernel is launched).

The persistent grouped scheduler ("The FP4 Frontier", Finding 5: one grouped
launch over all experts) turns the device offsets into units (expert, row
tile, K split, column tile).  Each unit's output tile indexes the split-K
arrival counters and the FP32 partial tiles, and those two accesses are not
bounds-checked by a buffer resource: the counter is an atomic at
`counters[tile]` and the partials resource is based at
`partials + tile * splits * BM * BN`.  This model restates, in Python, the
unit numbering of gemm.hip's `build_schedule` and `decode_unit`:
- experts ranked by rows (descending, ties by id) when there are at most 256;
- the per-expert unit prefix;
- the binary search of a unit's expert;
- the tile number `prefix / splits + nt * mtiles + mt`.

It then asserts, for many expert-count patterns, row tiles, column tiles and
split counts, including the shape of the GPU fault recorded in the design
notes (4 experts with 70 / 0 / 5 / 33 rows, N = 513, K = 2048, BM = 32, splits
2, 5 and 12), that:
  * every (tile, split) pair occurs exactly once, and each unit's rows lie in
    its expert's segment;
  * every tile is below the planner's bound
    `(ceil(rows / BM) + min(E, rows)) * n_tiles`, which is below the counter
    capacity whenever K is split;
  * the workspace the library reports (`nvfp4_grouped_gemm_workspace_size`
    with the same forced row tile and split count) holds the counters plus
    the partial tiles of the largest tile index.
"""
import math

import numpy as np
import pytest

import block_scaled_fp4_nibble_amd as nv
from gpu_helpers import EnvOverride

SORT_MAX = 256  # gemm.hip: experts ranked by rows up to this count


def schedule(counts, bm, n_tiles, splits):
    E = len(counts)
    order = sorted(range(E), key=lambda e: (-counts[e], e)) if E <= SORT_MAX else list(range(E))
    prefix, base = [], 0
    for e in order:
        prefix.append(base)
        base += -(-counts[e] // bm) * n_tiles * splits
    return order, prefix, base


def decode(unit, order, prefix, seg, counts, bm, splits):
    # last schedule position whose prefix is <= unit (empty experts have
    # equal bounds; the search lands on the non-empty one after them)
    lo, hi = 0, len(order)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if prefix[mid] <= unit:
            lo = mid
        else:
            hi = mid
    e = order[lo]
    mtiles = -(-counts[e] // bm)
    local = unit - prefix[lo]
    mt, rest = local % mtiles, local // mtiles
    ks, nt = rest % splits, rest // splits
    tile = prefix[lo] // splits + nt * mtiles + mt
    row0 = seg[e] + mt * bm
    return dict(e=e, ks=ks, nt=nt, tile=tile, row0=row0, row_end=min(row0 + bm, seg[e + 1]))


def check(counts, bm, n_tiles, splits):
    counts = list(counts)
    E, rows = len(counts), sum(counts)
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    order, prefix, total = schedule(counts, bm, n_tiles, splits)
    seen = set()
    max_tile = -1
    for u in range(total):
        d = decode(u, order, prefix, seg, counts, bm, splits)
        key = (d["tile"], d["ks"])
        assert key not in seen, (counts, bm, n_tiles, splits, u)
        seen.add(key)
        assert seg[d["e"]] <= d["row0"] < d["row_end"] <= seg[d["e"] + 1]
        assert 0 <= d["nt"] < n_tiles
        max_tile = max(max_tile, d["tile"])
    bound = (-(-rows // bm) + min(E, rows)) * n_tiles
    assert max_tile < bound
    # every tile number below the largest one is used: the numbering is dense
    assert len({t for t, _ in seen}) == max_tile + 1
    return max_tile, bound


RNG = np.random.default_rng(np.random.SeedSequence([555, 1]))
PATTERNS = [
    [70, 0, 5, 33],                      # the recorded fault's experts
    [0, 0, 0, 9],                        # leading empty experts
    [40, 0, 0, 0],                       # trailing empty experts
    [1] * 64,                            # one row each
    [16, 17, 15, 32, 33, 64, 65, 0],     # row-tile boundaries
    list(RNG.integers(0, 120, size=64)),  # random ~uniform
    list(RNG.zipf(1.3, size=64) % 500),  # skewed
    list(RNG.integers(0, 5, size=300)),  # more experts than the sorted schedule takes
]


@pytest.mark.parametrize("counts", PATTERNS, ids=["p%d" % i for i in range(len(PATTERNS))])
@pytest.mark.parametrize("bm", [16, 32, 64])
@pytest.mark.parametrize("n_tiles", [1, 3, 16])
@pytest.mark.parametrize("splits", [1, 2, 5, 12])
def test_unit_numbering(counts, bm, n_tiles, splits):
    if sum(counts) == 0:
        pytest.skip("no rows")
    check(counts, bm, n_tiles, splits)


@pytest.mark.parametrize("splits", [2, 5, 12])
def test_recorded_fault_shape_workspace(splits):
    """4 experts (70 / 0 / 5 / 33 rows), N = 513, K = 2048, BM = 32: the
    library's workspace covers the counters and every tile's partials."""
    lib = nv.load_library()
    counts, n, k, bm = [70, 0, 5, 33], 513, 2048, 32
    rows, E = sum(counts), len(counts)
    with EnvOverride(NVFP4_BM=bm, NVFP4_SPLITK=splits):
        name = lib.nvfp4_kernel_name(rows, E, n, k, 1, 0).decode()
        ws = lib.nvfp4_grouped_gemm_workspace_size(rows, E, n, k)
    assert name.startswith("nvfp4::gemm_kp_kernel<32,"), name
    bn = int(name.split(",")[3].strip().rstrip(">"))
    # the planner's own rounding of the split: K per split a multiple of 64
    ksplit = -(-k // splits)
    ksplit = -(-ksplit // 64) * 64
    s = -(-k // ksplit)
    n_tiles = -(-n // bn)
    max_tile, bound = check(counts, bm, n_tiles, s)
    counter_bytes = nv.nvfp4_workspace_counter_bytes()
    assert bound <= counter_bytes // 4  # counters[tile] in range
    need = counter_bytes + (max_tile + 1) * s * bm * bn * 4
    assert ws >= need, (ws, need)
    assert ws == counter_bytes + bound * s * bm * bn * 4


def test_model_detects_a_wrong_tile_formula():
    """The model has teeth: numbering tiles without the per-expert prefix
    (nt * mtiles + mt only) collides across experts."""
    counts, bm, n_tiles, splits = [70, 0, 5, 33], 32, 3, 2
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    order, prefix, total = schedule(counts, bm, n_tiles, splits)
    seen, collided = set(), False
    for u in range(total):
        d = decode(u, order, prefix, seg, counts, bm, splits)
        mtiles = -(-counts[d["e"]] // bm)
        wrong = (d["nt"] * mtiles + (d["row0"] - seg[d["e"]]) // bm, d["ks"])
        collided |= wrong in seen
        seen.add(wrong)
    assert collided
