"""CPU model of the LDS bank mapping of the e4m3 / MXFP4 forward's operand
reads (64 banks of 4 bytes; an 8-byte read serves 32 lanes per pass, a
16-byte read 16 lanes): the chunk permutations of the K and V tiles leave
every pass free of bank conflicts.  The index formulas restate those of
exact_attention_50_amd/csrc/fa_fwd8.hip (slot_key, swz8, swzv, swz4 and the
operand offsets); a change there must be mirrored here."""


def slot_key(g, j):
    return 32 * (j // 16) + 8 * ((j % 16) // 4) + 4 * g + (j % 4)


def swz8(r):
    return (r >> 1) & 7


def swzv(r):
    return (r & 2) | ((r >> 1) & 4)


def swz4(r):
    return (r >> 2) & 3


def worst_conflict(addrs, nbytes, lanes_per_pass):
    worst = 1
    for p0 in range(0, len(addrs), lanes_per_pass):
        cnt = {}
        for a in addrs[p0:p0 + lanes_per_pass]:
            for w in range(nbytes // 4):
                bank = (a // 4 + w) % 64
                cnt[bank] = cnt.get(bank, 0) + 1
        worst = max(worst, max(cnt.values()))
    return worst


def v_read_addrs(sw, ks, q, db):
    """Byte offsets of the 64 lanes of one transposed V read (8 bytes each)."""
    out = []
    for lane in range(64):
        g, par, m8, half = lane >> 5, lane & 1, (lane & 15) >> 1, (lane >> 4) & 1
        row = slot_key(g, 8 * q + m8)
        s = sw(row)
        out.append(ks * 64 * 128 + row * 128 + 8 * par + 16 * (half ^ (s & 1)) + ((32 * db) ^ (32 * (s >> 1))))
    return out


def test_v_reads_address_their_logical_chunks():
    for ks in range(2):
        for q in range(4):
            for db in range(4):
                for lane, a in enumerate(v_read_addrs(swzv, ks, q, db)):
                    g, par, m8, half = lane >> 5, lane & 1, (lane & 15) >> 1, (lane >> 4) & 1
                    row = slot_key(g, 8 * q + m8)
                    assert a // 128 == ks * 64 + row
                    assert ((a % 128) // 16) ^ swzv(row) == 2 * db + half and (a % 16) // 8 == par


def test_v_reads_conflict_free_with_their_permutation():
    for ks in range(2):
        for q in range(4):
            for db in range(4):
                assert worst_conflict(v_read_addrs(swzv, ks, q, db), 8, 32) == 1


def test_k_permutation_on_v_reads_conflicts():
    """The K tiles' permutation applied to V tiles (the earlier layout): a
    2-way conflict on the transposed reads, which the counters showed."""
    assert max(worst_conflict(v_read_addrs(swz8, 0, q, db), 8, 32) for q in range(4) for db in range(4)) == 2


def test_k_reads_conflict_free():
    # e4m3 K: rows r32 = 0..31 of a 32-key block, 16-byte chunk c at c ^ swz8(r)
    for kb in range(4):
        for c in range(8):
            addrs = [(32 * kb + r) * 128 + 16 * (c ^ swz8(r)) for r in range(32)]
            assert worst_conflict(addrs, 16, 16) == 1
    # MXFP4 K: 64-byte rows, chunk c (0..3) at c ^ swz4(r)
    for kb in range(4):
        for c in range(4):
            addrs = [(32 * kb + r) * 64 + 16 * (c ^ swz4(r)) for r in range(32)]
            assert worst_conflict(addrs, 16, 16) == 1


# ---- e4m3 tiles at d = 64: 64-byte rows (4 rows per 256-byte bank line)
def swz64(r):
    return (r >> 2) & 3


def swzv64(r):
    return (r >> 2) & 2


def v64_read_addrs(sw, ks, q, db):
    out = []
    for lane in range(64):
        g, par, m8, half = lane >> 5, lane & 1, (lane & 15) >> 1, (lane >> 4) & 1
        row = slot_key(g, 8 * q + m8)
        s = sw(row)
        out.append(ks * 64 * 64 + row * 64 + 8 * par + 16 * (half ^ (s & 1)) + ((32 * db) ^ (32 * (s >> 1))))
    return out


def test_d64_v_reads_address_their_logical_chunks_and_are_conflict_free():
    for ks in range(2):
        for q in range(4):
            for db in range(2):
                addrs = v64_read_addrs(swzv64, ks, q, db)
                for lane, a in enumerate(addrs):
                    g, par, m8, half = lane >> 5, lane & 1, (lane & 15) >> 1, (lane >> 4) & 1
                    row = slot_key(g, 8 * q + m8)
                    assert a // 64 == ks * 64 + row
                    assert ((a % 64) // 16) ^ swzv64(row) == 2 * db + half and (a % 16) // 8 == par
                assert worst_conflict(addrs, 8, 32) == 1


def test_d64_k_reads_conflict_free():
    # lane (r32, g) reads chunks 2 g, 2 g + 1 of row r32 of a 32-key block
    for kb in range(4):
        for c in range(4):
            addrs = [(32 * kb + r) * 64 + 16 * (c ^ swz64(r)) for r in range(32)]
            assert worst_conflict(addrs, 16, 16) == 1
