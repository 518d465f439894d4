"""Index maps of the eight-wave kernels' LDS ring, checked on the CPU.

These restate, in Python, the integer maps that ``kernels_w8.hip`` uses for the
256 x 256 tile with both operands K-contiguous (the pair ring): which LDS bytes of a
B slab each wave's loads write, and which bytes each wave's fragment reads touch.
The property under test is the one that makes refilling a B slot in the same phase
as its last reads safe: a wave of group 1 overwrites only bytes that it has read
itself (its own reads are complete when it issues the loads) or that group 0 read in
the previous phase (complete before the barrier in between).
"""
import pytest

GROUP, LOADS = 4, 4
BK, BN, NBL, WTN = 32, 256, 4, 64     # 256 x 256 tile: 32-deep slabs, 4 B blocks of 16 a wave


def kswz(bk, r):
    return 2 * ((r >> 3) & 1) if bk == 32 else (r >> 1) & 7 if bk == 64 else r & 15


def kc_off(bk, r, c):
    return r * 2 * bk + 16 * (c ^ kswz(bk, r))


def block_of(own, wave, j):
    return GROUP * wave + j if own else GROUP * j + wave


def loaded_bytes(wave, own):
    """LDS bytes (within one operand slab) written by the wave's LOADS loads."""
    out = set()
    for j in range(LOADS):
        for lane in range(64):
            slot = block_of(own, wave, j) * 64 + lane
            out.update(range(16 * slot, 16 * slot + 16))
    return out


def loaded_rows(wave, own):
    """(row, chunk) of the global chunk each lane loads, K-contiguous operand."""
    cpr = BK // 8
    out = {}
    for j in range(LOADS):
        for lane in range(64):
            slot = block_of(own, wave, j) * 64 + lane
            r = slot // cpr
            c = (slot % cpr) ^ kswz(BK, r)
            out[16 * slot] = (r, c)
    return out


def read_bytes(wn):
    """LDS bytes of the B slab read by a wave whose block of C is column block wn (one
    16-byte read per 16-column block and lane: row 16 j + l % 16, k chunk l / 16)."""
    out = set()
    for lane in range(64):
        base = kc_off(BK, lane & 15, lane >> 4) + 2 * BK * WTN * wn
        for j in range(NBL):
            a = base + 32 * BK * j
            out.update(range(a, a + 16))
    return out


@pytest.mark.parametrize("own", [False, True])
def test_loads_fill_the_slab_once(own):
    seen = []
    for w in range(GROUP):
        seen.extend(sorted(loaded_bytes(w, own)))
    assert sorted(seen) == list(range(BN * BK * 2))


def test_own_loads_write_only_the_rows_the_wave_reads():
    for w in range(GROUP):
        assert loaded_bytes(w, True) == read_bytes(w)


def test_interleaved_loads_would_write_other_waves_rows():
    # the map the refill used before: every wave wrote into the other waves' rows
    for w in range(GROUP):
        assert loaded_bytes(w, False) - read_bytes(w)


def test_each_lane_loads_the_chunk_its_slot_holds():
    # The swizzle is applied on the global side: the LDS slot at byte b holds chunk c of
    # row r exactly where the fragment reads look for (r, c).
    where = {}
    for r in range(BN):
        for c in range(BK // 8):
            where[(r, c)] = kc_off(BK, r, c)
    for w in range(GROUP):
        for byte, rc in loaded_rows(w, True).items():
            assert where[rc] == byte
