"""Host model of the split-K decode kernel's token-row staging (gemv.hip:
decode_sk_kernel), run on the CPU.

Each wave stages the token rows of its 128-deep K groups in an LDS region of
its own with direct buffer -> LDS loads (1 KB per instruction: lane l writes
its 16 bytes at M0 + 16 l) and reads them back as MFMA A fragments.  Which
16-byte chunk of a row a lane loads is chosen so that the chunk lands where
the reads look for it: with a swizzle on both sides, a mismatch would
silently multiply the wrong activations, and a destination past a slot would
write into the wave's other group or another wave's rows.  The model
restates the kernel's index formulas (a group's rows are 256 bytes, chunk c
of row r at 16-byte position c ^ (r % 16); the region holds both of the
wave's groups up to 32 rows and one above) and checks, for every row-fragment
count the kernel is instantiated with:

  * every load's destination lies inside its group slot, and each slot
    position is written exactly once;
  * MFMA step t of lane group q finds, for its row, the chunk
    K = 32 q + 8 t .. + 7 of the group (the K its weight fragment supplies);
  * a 16-lane pass of the reads touches 16 distinct 16-byte positions of a
    256-byte window (no bank conflict);
  * the waves' regions fit the 128 KB set aside for them, and each wave's
    sums (published at the start of its region) fit it.
"""
import pytest

WAVES = 8
GROUPS_PER_WAVE = 2
REGION_BYTES = 128 * 1024


def resident_groups(nf):
    # both of a wave's groups when 8 waves x 2 groups fit, else one
    return 2 if WAVES * GROUPS_PER_WAVE * nf * 4096 <= REGION_BYTES else 1


def group_loads(bm):
    """(destination within the group slot, row, chunk) of every lane of
    every load of one group."""
    out = []
    for t in range(bm * 256 // 1024):
        for lane in range(64):
            r = 4 * t + (lane >> 4)
            q = lane & 15
            out.append((t * 1024 + lane * 16, r, q ^ (r & 15)))
    return out


def fragment_read(row, g, t):
    """Byte offset within the group slot that lane group g reads for `row`
    in MFMA step t."""
    c = 4 * g + t
    return (row * 16 + (c ^ (row & 15))) * 16


@pytest.mark.parametrize("nf", [1, 2, 3, 4])
def test_token_row_staging(nf):
    bm = 16 * nf
    gb = bm * 256
    res = resident_groups(nf)
    assert res == (2 if nf <= 2 else 1)
    assert WAVES * res * gb <= REGION_BYTES
    # each wave's sums: NF x 4 column tiles x 64 lanes of 16 bytes
    assert nf * 4 * 64 * 16 <= res * gb
    slot = {}
    for dst, r, c in group_loads(bm):
        assert 0 <= dst and dst + 16 <= gb, "destination past the group slot"
        assert dst not in slot, "position written twice"
        slot[dst] = (r, c)
    assert len(slot) == gb // 16
    for t in range(4):
        for f in range(nf):
            for lane in range(64):
                g, c16 = lane >> 4, lane & 15
                row = 16 * f + c16
                r, c = slot[fragment_read(row, g, t)]
                assert r == row
                assert 8 * c == 32 * g + 8 * t
            for g in range(4):
                pos = {(fragment_read(16 * f + c16, g, t) // 16) % 16 for c16 in range(16)}
                assert len(pos) == 16


def test_model_catches_a_swizzle_mismatch():
    """A read swizzle that differs from the load's (row % 8 instead of
    row % 16) is caught by the chunk check."""
    bm = 64
    slot = {dst: (r, c) for dst, r, c in group_loads(bm)}
    bad = 0
    for row in range(bm):
        for g in range(4):
            c = 4 * g
            r, got = slot[(row * 16 + (c ^ (row & 7))) * 16]
            bad += (r, got) != (row, c)
    assert bad > 0
