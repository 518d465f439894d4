"""Index maps of the eight-wave kernels (``kernels_w8.hip``), checked on the CPU.

The kernels feed ``v_mfma_f32_16x16x32`` from LDS: lane l needs row l % 16 and k
8 (l / 16) .. +7 of a 16-row block of each operand.  These tests restate in Python the
integer maps the kernels use (the LDS layouts with their XOR swizzles, the slab loads,
the fragment reads, including the semantics of the LDS transpose read, and the
epilogue's staging) and check that:

* every chunk a load brings lands where the fragment reads look for it;
* every lane's fragment holds exactly the elements the matrix instruction expects;
* the accesses that the LDS serves together touch distinct banks (256 bytes of the 64
  four-byte banks).  The groupings were measured on the MI355X with the LDS conflict
  counter (one lane pair per dispatch at the same banks, the other lanes
  broadcasting): a 16-byte read goes in four passes, each the four-lane quads of one
  half-wave whose quad index has the same parity (lanes 0-3, 12-15, 20-23, 24-27 for
  lane 0); an 8-byte read (plain or transpose) in two passes of 32 consecutive lanes;
  an 8-byte write in four passes of 16 consecutive lanes, whose banks repeat every 128
  bytes (measured with only the two lanes of the pair active, the method checked
  against the known 16-byte grouping);
* the epilogue's staging writes every element of a wave's block of C once, and the
  store loop reads it back at the right row and column.
"""
import pytest

TILES = {  # BM, BN, BK, FM, FN (a wave's block is 32 FM x 32 FN)
    256: (256, 256, 32, 4, 2),
    128: (128, 128, 64, 2, 2),
    64: (64, 64, 128, 1, 1),
}


def kswz(bk, r):
    return 2 * ((r >> 3) & 1) if bk == 32 else (r >> 1) & 7 if bk == 64 else r & 15


def swz16(r):
    return r & 15


def swz8(r):
    return (r >> 1) & 7


def kc_off(bk, r, c):
    return r * 2 * bk + 16 * (c ^ kswz(bk, r))


def mswz(R, k):
    return (4 * (k & 3) if R >= 128 else 4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1))


def mn_off(R, k, c):
    return k * 2 * R + 16 * (c ^ mswz(R, k))


def kc_lane(bk, lane):
    return kc_off(bk, lane & 15, lane >> 4)


def mn_lane(R, lane, b):
    g, t = lane >> 4, lane & 15
    q, u = t >> 2, t & 3
    return mn_off(R, 8 * g + q, 2 * b + (u >> 1)) + 8 * (u & 1)


# ---- a fake LDS slab: byte address -> (m-or-n, k) element --------------------------------

def kc_slab(R, BK):
    """K-contiguous layout: rows of R (m or n), BK values each (2 bytes)."""
    lds = {}
    for r in range(R):
        for c in range(BK // 8):
            for e in range(8):
                lds[kc_off(BK, r, c) + 2 * e] = (r, 8 * c + e)
    return lds


def mn_slab(R, BK):
    """M/N-contiguous layout: k-rows of R values."""
    lds = {}
    for k in range(BK):
        for c in range(R // 8):
            for e in range(8):
                lds[mn_off(R, k, c) + 2 * e] = (8 * c + e, k)
    return lds


def read_b128(lds, addr):
    return [lds[addr + 2 * e] for e in range(8)]


def read_tr16(lds, addrs):
    """ds_read_b64_tr_b16 on one 16-lane group: addrs[i] is lane i's 8-byte address.
    Lane t receives element t & 3 of the rows addressed by lanes 4 q + (t >> 2)."""
    out = []
    for t in range(16):
        out.append([lds[addrs[4 * q + (t >> 2)] + 2 * (t & 3)] for q in range(4)])
    return out


@pytest.mark.parametrize("tile", sorted(TILES))
def test_loads_place_chunks_where_the_reads_look(tile):
    BM, BN, BK, FM, FN = TILES[tile]
    # the loaders: LDS slot s (16 bytes) of a slab holds global chunk (s % CPx) ^ swizzle
    for R in (BM, BN):
        cpr = BK // 8
        for slot in range(R * BK * 2 // 16):
            r, p = divmod(slot, cpr)
            c = p ^ kswz(BK, r)
            assert 0 <= c < cpr and kc_off(BK, r, c) == 16 * slot
        cpk = R // 8
        for slot in range(R * BK * 2 // 16):
            k, p = divmod(slot, cpk)
            c = p ^ mswz(R, k)
            assert 0 <= c < cpk and mn_off(R, k, c) == 16 * slot


@pytest.mark.parametrize("tile", sorted(TILES))
def test_k_contiguous_fragments(tile):
    BM, BN, BK, FM, FN = TILES[tile]
    steps = BK // 32
    for R, WT, MBk in ((BM, 32 * FM, 2 * FM), (BN, 32 * FN, 2 * FN)):
        lds = kc_slab(R, BK)
        for w in range(R // WT):
            for lane in range(64):
                base = kc_lane(BK, lane) + 2 * BK * WT * w
                for s in range(steps):
                    for b in range(MBk):
                        got = read_b128(lds, (base ^ (64 * s)) + 32 * BK * b)
                        row, k0 = WT * w + 16 * b + (lane & 15), 32 * s + 8 * (lane >> 4)
                        assert got == [(row, k0 + e) for e in range(8)]


def test_pair_ring_fragments():
    # 256 x 256 with both operands K-contiguous: A's LDS rows hold a pair of 32-deep
    # slabs (64 k, 128 bytes); slab t reads half t % 2 of each row (an XOR of 64 bytes).
    lds = kc_slab(256, 64)
    WTM = 128
    for wm in range(2):
        for lane in range(64):
            base = kc_lane(64, lane) + 2 * 64 * WTM * wm
            for h in range(2):
                for f in range(8):
                    got = read_b128(lds, (base ^ (64 * h)) + 32 * 64 * f)
                    row, k0 = WTM * wm + 16 * f + (lane & 15), 32 * h + 8 * (lane >> 4)
                    assert got == [(row, k0 + e) for e in range(8)]


@pytest.mark.parametrize("tile", sorted(TILES))
def test_transposed_fragments(tile):
    BM, BN, BK, FM, FN = TILES[tile]
    steps = BK // 32
    for R, WT, MBk in ((BM, 32 * FM, 2 * FM), (BN, 32 * FN, 2 * FN)):
        lds = mn_slab(R, BK)
        for w in range(R // WT):
            for b in range(MBk):
                blk = MBk * w + b
                for s in range(steps):
                    for e in range(2):
                        for g in range(4):
                            addrs = [mn_lane(R, 16 * g + i, blk) + 32 * s * 2 * R + 4 * 2 * R * e for i in range(16)]
                            got = read_tr16(lds, addrs)
                            for t in range(16):
                                k0 = 32 * s + 8 * g + 4 * e
                                assert got[t] == [(16 * blk + t, k0 + q) for q in range(4)]


def _banks(addr, nbytes):
    return {((addr + o) // 4) % 64 for o in range(0, nbytes, 4)}


def _conflict_free(addresses, nbytes):
    seen = set()
    for a in addresses:
        b = _banks(a, nbytes)
        if seen & b:
            return False
        seen |= b
    return True


def pass16(lane):
    """The pass of a 16-byte LDS access that serves a lane: its half-wave and the parity
    of its quad index."""
    return 2 * ((lane >> 5) & 1) + (((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1)


def _passes16(addrs):
    return [[addrs[l] for l in range(64) if pass16(l) == p] for p in range(4)]


def test_pass_grouping_as_measured():
    assert sorted(l for l in range(64) if pass16(l) == pass16(0)) == [0, 1, 2, 3, 12, 13, 14, 15,
                                                                        20, 21, 22, 23, 24, 25, 26, 27]


@pytest.mark.parametrize("tile", sorted(TILES))
def test_fragment_reads_are_conflict_free(tile):
    BM, BN, BK, FM, FN = TILES[tile]
    steps = BK // 32
    for R, WT, MBk in ((BM, 32 * FM, 2 * FM), (BN, 32 * FN, 2 * FN)):
        for w in range(R // WT):
            for s in range(steps):
                for b in range(MBk):
                    addrs = [(kc_lane(BK, l) + 2 * BK * WT * w ^ (64 * s)) + 32 * BK * b for l in range(64)]
                    for grp in _passes16(addrs):
                        assert _conflict_free(grp, 16), (R, w, s, b)
                    for e in range(2):
                        addrs = [mn_lane(R, l, MBk * w + b) + 32 * s * 2 * R + 8 * R * e for l in range(64)]
                        for half in range(2):       # 32 lanes of an 8-byte read together
                            assert _conflict_free(addrs[32 * half:32 * half + 32], 8), (R, w, s, b, e, half)


def test_old_swizzle_would_conflict_at_256():
    # Without the k-row bit-3 term, the two 16-lane groups of a transpose read served
    # together (k-rows 8 apart) would hit the same banks.
    def old(R, k):
        return 4 * (k & 3) if R >= 128 else 4 * ((k >> 1) & 1)
    R = 256
    addrs = []
    for l in range(32):
        g, t = l >> 4, l & 15
        q, u = t >> 2, t & 3
        k = 8 * g + q
        addrs.append(k * 2 * R + 16 * ((u >> 1) ^ old(R, k)) + 8 * (u & 1))
    assert not _conflict_free(addrs, 8)


def piece(i, j, lane):
    """(row, first column) in the wave's block of accumulator [i][j] of a lane."""
    return 16 * i + (lane & 15), 16 * j + 4 * (lane >> 4)


# The blocks a wave finishes: all of them, or (128 x 128, where the two groups split K)
# half each, the first or the second.
def _parts(tile):
    _, _, _, FM, FN = TILES[tile]
    MB = 2 * FM
    return [(0, MB)] + ([(0, MB // 2), (MB // 2, MB // 2)] if tile == 128 else [])


@pytest.mark.parametrize("tile", [256, 128])
def test_fp32_staging_round_trip(tile):
    _, _, _, FM, FN = TILES[tile]
    NBL = 2 * FN
    for I0, NI in _parts(tile):
        for pas in range((NI + 3) // 4):
            nb = min(4, NI - 4 * pas)
            region = {}
            for lane in range(64):
                for i4 in range(nb):
                    for j in range(NBL):
                        r, col = piece(i4, j, lane)
                        c = col >> 2
                        addr = r * 256 + 16 * (c ^ swz16(r))
                        assert addr not in region
                        row, col0 = piece(I0 + 4 * pas + i4, j, lane)
                        region[addr] = [(row, col0 + e) for e in range(4)]
            assert len(region) == 64 * 4 * nb
            for lane in range(64):
                for k in range(4 * nb):
                    r, c = 4 * k + (lane >> 4), lane & 15
                    got = region[r * 256 + 16 * (c ^ swz16(r))]
                    assert got == [(16 * I0 + 64 * pas + r, 4 * c + e) for e in range(4)]


def stage16_slot(i2, j, lane):
    """16-byte unit of a lane's pieces of blocks 2 i2 and 2 i2 + 1 in column block j."""
    t, g = lane & 15, lane >> 4
    return (i2 * 4 + j) * 64 + 16 * g + (t ^ (4 * j + 2 * (g >> 1) + (g & 1)))


def stage16_read(k, lane):
    """Store instruction k of the 16-bit read-back: (row, first column, the two 8-byte
    piece addresses) of a lane."""
    i2, rho, c = k >> 2, lane >> 3, lane & 7
    sh, tt = rho & 1, 4 * (k & 3) + (rho >> 1)
    j = c >> 1
    u, f = (i2 * 4 + j) * 64 + 16 * (2 * (c & 1)), 4 * j + 2 * (c & 1)
    return 32 * i2 + 16 * sh + tt, 8 * c, (16 * (u + (tt ^ f)) + 8 * sh, 16 * (u + 16 + (tt ^ (f + 1))) + 8 * sh)


@pytest.mark.parametrize("tile", [256, 128])
def test_16bit_staging_round_trip(tile):
    for I0, NI in _parts(tile):
        region = {}
        for lane in range(64):
            for i2 in range(NI // 2):
                for j in range(4):
                    base = 16 * stage16_slot(i2, j, lane)
                    for s in range(2):
                        r, col = piece(2 * i2 + s, j, lane)
                        for e in range(4):
                            a = base + 8 * s + 2 * e
                            assert a not in region
                            region[a] = (r, col + e)
        assert len(region) == 16 * NI * 64
        rows = set()
        for k in range(2 * NI):
            for lane in range(64):
                row, col, (a0, a1) = stage16_read(k, lane)
                got = [region[a0 + 2 * e] for e in range(4)] + [region[a1 + 2 * e] for e in range(4)]
                assert got == [(row, col + e) for e in range(8)]
                rows.add(row)
        assert rows == set(range(16 * NI))
        # every store instruction writes whole 128-byte rows: 8 rows of 8 chunks
        for k in range(2 * NI):
            got = sorted((stage16_read(k, l)[0], stage16_read(k, l)[1]) for l in range(64))
            assert len({r for r, _ in got}) == 8 and all(c in range(0, 64, 8) for _, c in got)


def _banks128(addr, nbytes):
    return {((addr + o) // 4) % 32 for o in range(0, nbytes, 4)}


def _write8_conflict_free(addresses):
    """An 8-byte write pass: 16 consecutive lanes within 128 bytes of banks."""
    seen = set()
    for a in addresses:
        b = _banks128(a, 8)
        if seen & b:
            return False
        seen |= b
    return True


@pytest.mark.parametrize("tile", [256, 128])
def test_staging_writes_are_conflict_free(tile):
    _, _, _, FM, FN = TILES[tile]
    MB, NBL = 2 * FM, 2 * FN
    for i in range(MB):
        for j in range(NBL):
            a32 = []
            for lane in range(64):
                r, col = piece(i % 4, j, lane)
                a32.append(r * 256 + 16 * ((col >> 2) ^ swz16(r)))
            for grp in _passes16(a32):
                assert _conflict_free(grp, 16)
    for i2 in range(MB // 2):
        for j in range(NBL):
            a16 = [16 * stage16_slot(i2, j, l) for l in range(64)]
            for grp in _passes16(a16):
                assert _conflict_free(grp, 16), (i2, j)
    # the read-backs: 4 rows at 16 chunks (fp32); 8-byte piece pairs (16-bit)
    for k in range(16):
        rb = [(4 * k + (l >> 4)) * 256 + 16 * ((l & 15) ^ swz16(4 * k + (l >> 4))) for l in range(64)]
        assert all(_conflict_free(g, 16) for g in _passes16(rb))
    for k in range(MB * 2):
        for e in range(2):
            rb = [stage16_read(k, l)[2][e] for l in range(64)]
            for half in range(2):
                assert _conflict_free(rb[32 * half:32 * half + 32], 8), (k, e, half)


def test_8byte_staging_writes_would_conflict():
    # The earlier 16-bit staging: 128-byte rows, chunk c of row r at 16 (c ^ ((r / 2) % 8)),
    # each lane writing its 8-byte piece of one block.  Conflict-free in 32-lane passes
    # over 256 bytes, but the measured 8-byte write passes (16 lanes, 128 bytes of
    # banks) put rows t and t ^ 1 on the same banks: one extra cycle a pass, the
    # 262 144 conflict cycles the counter showed at 4096^3 (four per write instruction).
    for i in range(8):
        for j in range(4):
            addrs = []
            for lane in range(64):
                r, col = piece(i, j, lane)
                addrs.append(r * 128 + 16 * ((col >> 3) ^ swz8(r)) + 2 * (col & 7))
            assert all(_conflict_free(addrs[32 * h:32 * h + 32], 8) for h in range(2))
            assert not any(_write8_conflict_free(addrs[16 * q:16 * q + 16]) for q in range(4))


def test_direct_store_pieces_cover_the_block():
    # the 64 x 64 tile stores its 32 x 32 blocks straight from the accumulators
    seen = set()
    for lane in range(64):
        for i in range(2):
            for j in range(2):
                r, c = piece(i, j, lane)
                for e in range(4):
                    assert (r, c + e) not in seen
                    seen.add((r, c + e))
    assert seen == {(r, c) for r in range(32) for c in range(32)}


def test_plain_row_swizzle_would_conflict():
    # 16 rows at 4 chunks with the plain (r >> 2) & 3 swizzle of 32-deep slabs: two-way
    # conflicts in the measured passes (the counter showed them), none in 16
    # consecutive lanes (the model that first chose it).
    addrs = [(l & 15) * 64 + 16 * ((l >> 4) ^ ((l & 15) >> 2 & 3)) for l in range(64)]
    assert all(_conflict_free(addrs[16 * g:16 * g + 16], 16) for g in range(4))
    assert not all(_conflict_free(g, 16) for g in _passes16(addrs))


def test_lean_epilogue_offsets_match_the_general_maps():
    """The lean epilogues (wave blocks inside C, no fused epilogue) split each staging
    address into per-lane offsets computed once and immediate parts; they must land on
    exactly the addresses of the general maps above."""
    for lane in range(64):
        t, g = lane & 15, lane >> 4
        # fp32: writes of block (i4, j), read-back k
        for j in range(4):
            for i4 in range(4):
                r, c = 16 * i4 + t, 4 * j + g
                assert t * 256 + 16 * ((g ^ t) & 3) + 64 * (j ^ (t >> 2)) + 4096 * i4 == r * 256 + 16 * (c ^ swz16(r))
        u = lane & 15
        for k in range(16):
            r = 4 * k + g
            lean = g * 256 + 16 * ((u ^ g) & 3) + 64 * (((u ^ g) >> 2) ^ (k & 3)) + 1024 * k
            assert lean == r * 256 + 16 * (u ^ swz16(r))
        # 16-bit: writes of pair i2 in column block j, read-back k (row and both pieces)
        for i2 in range(4):
            for j in range(4):
                woff = 16 * (64 * j + 16 * g + (t ^ (4 * j + 2 * (g >> 1) + (g & 1))))
                assert woff + 16 * 64 * 4 * i2 == 16 * stage16_slot(i2, j, lane)
        rho, c = lane >> 3, lane & 7
        sh, r2, jj, cb = rho & 1, rho >> 1, c >> 1, c & 1
        rb = 16 * (64 * jj + 32 * cb + (r2 ^ (2 * cb))) + 8 * sh
        rb2 = 16 * (64 * jj + 32 * cb + 16 + (r2 ^ (2 * cb + 1))) + 8 * sh
        for k in range(16):
            qo, kb = 64 * ((k & 3) ^ jj), 4096 * (k >> 2)
            row, col, (a0, a1) = stage16_read(k, lane)
            assert (rb + qo + kb, rb2 + qo + kb) == (a0, a1)
            assert (32 * (k >> 2) + 4 * (k & 3) + 16 * sh + r2, 8 * c) == (row, col)


def test_lean_prior_epilogue_offsets_match_prior_at():
    """The prior C of the 256 x 256 fused epilogue sits in the ring's slots past K:
    quarter q of the tile (rows 64 q ..) in the slot of slab KT + q, its halves of 32
    rows OP_BYTES apart, rows of 512 bytes with chunk c at c ^ pswz(row).  The lean form
    splits each address into uniform, per-lane and immediate parts."""
    SLOTS, SLOT, OP = 5, 32768, 16384

    def pswz(r):
        return ((r >> 1) & 7) | ((r & 1) << 3)

    def slot_addr(s):
        return (s % SLOTS) * SLOT

    def prior_at(KT, R, c):
        r = R & 31
        return slot_addr(KT + R // 64) + ((R >> 5) & 1) * OP + r * 512 + 16 * (c ^ pswz(r))

    for KT in (1, 2, 3, 7, 128):
        for wm in range(2):
            for wn in range(4):
                sA, sB = slot_addr(KT + 2 * wm), slot_addr(KT + 2 * wm + 1)
                for lane in range(64):
                    t, g = lane & 15, lane >> 4
                    lo = [t * 512 + 16 * ((8 * wn + 2 * j + (g >> 1)) ^ pswz(t)) + 8 * (g & 1) for j in range(4)]
                    for i in range(8):
                        for j in range(4):
                            R, Cc = 128 * wm + 16 * i + t, 64 * wn + 16 * j + 4 * g
                            lean = (sA if i < 4 else sB) + ((i >> 1) & 1) * OP + (i & 1) * 16 * 512 + lo[j]
                            assert lean == prior_at(KT, R, Cc >> 3) + 8 * ((Cc >> 2) & 1)
                    r3, cc = lane >> 3, lane & 7
                    so = [r3 * 512 + 16 * ((8 * wn + cc) ^ (4 * q + (r3 >> 1) + 8 * (r3 & 1))) for q in range(2)]
                    for k in range(16):
                        lean = (sA if k < 8 else sB) + ((k >> 2) & 1) * OP + 8 * (k & 3) * 512 + so[k & 1]
                        assert lean == prior_at(KT, 128 * wm + 8 * k + r3, 8 * wn + cc)
