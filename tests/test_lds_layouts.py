"""LDS tile layouts of the HIP kernels (CPU only): every read pattern the
kernels issue hits distinct banks, and the reader finds the element the
writer put there.

The per-lane address formulas below restate the kernels' (named at each
case); the bank model is gfx950's LDS: 64 banks of 4 bytes.  A 16-byte
read (ds_read_b128) is served 8 lanes at a time and an 8-byte transposed
read (ds_read_b64_tr_b16) 16 lanes at a time; a pattern is conflict-free
when no two distinct 4-byte words of one such lane group share a bank (the
check also holds for 16- and 32-lane groups respectively, which covers a
hardware that serves twice as many lanes per pass).
"""
import collections

import pytest

BANKS = 64


def worst_conflict(addrs, nbytes, group):
    """Largest number of distinct words one bank serves within a lane group."""
    w = 1
    for g0 in range(0, len(addrs), group):
        banks = collections.defaultdict(set)
        for a in addrs[g0:g0 + group]:
            for b in range(0, nbytes, 4):
                banks[((a + b) // 4) % BANKS].add((a + b) // 4)
        w = max(w, max(len(v) for v in banks.values()))
    return w


def krow(mt, m):
    """Key held by row m of score tile mt (the forward's read order)."""
    return ((m >> 2) & 1) * 32 + mt * 16 + (m >> 3) * 4 + (m & 3)


def qperm(m):
    """Query held by slot m of a key-kernel query tile."""
    return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3)


SLOT_OF_KEY = {krow(mt, m): mt * 32 + m for mt in range(2) for m in range(32)}


def tr_lane(lane, row0, d0_tile):
    """ds_read_b64_tr_b16 addressing: within each 16 lanes, lane r reads row
    row0 + r // 4 (relative) and channels 4 (r % 4) .. + 3 of the 16-channel
    group of its 16-lane block; it receives channel (block base + r) of 4 rows."""
    r32 = lane & 31
    r = r32 & 15
    return row0 + (r >> 2), d0_tile + (r32 >> 4) * 16 + 4 * (r & 3)


@pytest.mark.parametrize("D", [64, 128])
def test_forward_fp16_stage(D):
    """attention.hip F16Pipe: chunk-column-major (16-byte chunk c of slot s at
    c*1088 + s*16), K slots in krow order read by qk_f16p, V slots in key order
    read transposed by pv_f16p."""
    CS = 1088
    for mt in range(2):
        for kk in range(D // 16):
            addrs = [(kk * 2 + (l >> 5)) * CS + (mt * 32 + (l & 31)) * 16 for l in range(64)]
            assert worst_conflict(addrs, 16, 8) == 1 and worst_conflict(addrs, 16, 16) == 1
    for stp in range(4):
        for h2 in range(2):
            for dt in range(D // 32):
                addrs = []
                for l in range(64):
                    key, ch = tr_lane(l, (l >> 5) * 32 + 8 * stp + 4 * h2, dt * 32)
                    addrs.append((ch // 8) * CS + key * 16 + (ch % 8) * 2)
                assert worst_conflict(addrs, 8, 16) == 1 and worst_conflict(addrs, 8, 32) == 1


@pytest.mark.parametrize("D", [64, 128])
def test_backward_row_stage(D):
    """backward.hip RowStage: K and V tiles in krow order (1088-byte columns);
    S^T and dP^T read rows, K^T / V^T are read transposed through kslot_of."""
    CS = 1088

    def kslot_of(k):  # the kernel's closed form
        return ((k >> 4) & 1) * 32 + ((k >> 2) & 3) * 8 + ((k >> 5) & 1) * 4 + (k & 3)

    assert all(kslot_of(k) == SLOT_OF_KEY[k] for k in range(64))
    # direct loads: lane l of the wave load for column c writes slot l, row krow(l // 32, l % 32)
    written = {(c, l): krow(l >> 5, l & 31) for c in range(D // 8) for l in range(64)}
    for mt in range(2):
        for kk in range(D // 16):
            addrs = []
            for l in range(64):
                c, s = kk * 2 + (l >> 5), mt * 32 + (l & 31)
                assert written[(c, s)] == krow(mt, l & 31)  # the S^T operand's key
                addrs.append(c * CS + s * 16)
            assert worst_conflict(addrs, 16, 8) == 1 and worst_conflict(addrs, 16, 16) == 1
    for st in range(4):
        for h2 in range(2):
            for dt in range(D // 32):
                addrs = []
                for l in range(64):
                    key, ch = tr_lane(l, (l >> 5) * 32 + 8 * st + 4 * h2, dt * 32)
                    c, s = ch // 8, kslot_of(key)
                    assert written[(c, s)] == key
                    addrs.append(c * CS + s * 16 + (ch % 8) * 2)
                assert worst_conflict(addrs, 8, 16) == 1 and worst_conflict(addrs, 8, 32) == 1


@pytest.mark.parametrize("D", [64, 128])
def test_backward_key_stage(D):
    """backward.hip KeyStage: 32-row tiles, 512-byte columns, query qperm(m)
    of chunk c at slot (m + 4c) % 32; one 64-lane direct load fills columns
    2p and 2p + 1; S/dP read rows, dV/dK read transposed."""
    inv = {qperm(m): m for m in range(32)}
    written = {}
    for p in range(D // 16):
        for l in range(64):
            c, s = 2 * p + (l >> 5), l & 31
            assert p * 1024 + l * 16 == c * 512 + s * 16  # one contiguous wave load
            written[(c, s)] = qperm((s - 4 * c) & 31)  # key_issue's source row
    assert len(written) == (D // 8) * 32
    for kk in range(D // 16):
        addrs = []
        for l in range(64):
            c, m = 2 * kk + (l >> 5), l & 31
            s = (m + 4 * c) & 31
            assert written[(c, s)] == qperm(m)
            addrs.append(c * 512 + s * 16)
        assert worst_conflict(addrs, 16, 8) == 1 and worst_conflict(addrs, 16, 16) == 1
    for st in range(2):
        for h2 in range(2):
            for dt in range(D // 32):
                addrs = []
                for l in range(64):
                    q, ch = tr_lane(l, (l >> 5) * 16 + 8 * st + 4 * h2, dt * 32)
                    c = ch // 8
                    s = (inv[q] + 4 * c) & 31
                    assert written[(c, s)] == q
                    addrs.append(c * 512 + s * 16 + (ch % 8) * 2)
                assert worst_conflict(addrs, 8, 16) == 1 and worst_conflict(addrs, 8, 32) == 1


@pytest.mark.parametrize("D", [64, 128])
def test_forward_mx_stage(D):
    """attention.hip MxStage: K code rows of D/2 bytes and V^T rows of 32 bytes
    with XOR-swizzled 16-byte chunks (kswz, vswz), read 16 bytes per lane by
    load_k_mx / load_v_mx; the swizzle is a permutation of each row's chunks."""
    cpr = D // 32

    def kswz(r, c):
        return c ^ (((r >> 1) ^ (r >> 3)) & 3) if cpr == 4 else c ^ (((r >> 2) ^ (r >> 3)) & 1)

    def vswz(d, h):
        return h ^ (((d >> 2) ^ (d >> 3)) & 1)

    for r in range(64):
        assert sorted(kswz(r, c) for c in range(cpr)) == list(range(cpr))
    for mt in range(2):
        for kk in range(D // 64):
            addrs = [(mt * 32 + (l & 31)) * (D // 2) + kswz(mt * 32 + (l & 31), kk * 2 + (l >> 5)) * 16
                     for l in range(64)]
            assert worst_conflict(addrs, 16, 8) == 1 and worst_conflict(addrs, 16, 16) == 1
    for dt in range(D // 32):
        addrs = [(dt * 32 + (l & 31)) * 32 + vswz(dt * 32 + (l & 31), l >> 5) * 16 for l in range(64)]
        assert worst_conflict(addrs, 16, 8) == 1 and worst_conflict(addrs, 16, 16) == 1


@pytest.mark.parametrize("D", [64, 128])
def test_backward_prep_v_tile(D):
    """backward.hip bwd_prep_kernel, V role: thread t of 256 decodes channels
    2dp, 2dp+1 (dp = t % (D/2)) of keys kq*KPG .. kq*KPG+KPG-1 (kq = t // (D/2),
    KPG = 64 / (256 // (D/2))) and writes each key's channel pair as one word at
    half (key*RS + 2dp) of the tile (RS = D + 8 halves per row); the tile then
    leaves as 16-byte row chunks, thread c reading row c // (D/8), halves
    8 (c % (D/8)) ..  Every element is written once and read once, each wave's
    word writes hit every bank at most once, and the chunk reads are free of
    conflicts within each 8-lane pass."""
    NP, RS = D // 2, D + 8
    KPG = 64 // (256 // NP)
    written = collections.Counter()
    for w in range(4):
        addrs_by_e = collections.defaultdict(list)
        for lane in range(64):
            t = w * 64 + lane
            dp, kq = t % NP, t // NP
            for e in range(KPG):
                key = kq * KPG + e
                half = key * RS + 2 * dp
                written[(key, 2 * dp)] += 1
                written[(key, 2 * dp + 1)] += 1
                addrs_by_e[e].append(half * 2)
        for e, addrs in addrs_by_e.items():  # one ds_write_b32 per element index
            assert worst_conflict(addrs, 4, 64) == 1
    assert set(written) == {(k, d) for k in range(64) for d in range(D)}
    assert all(v == 1 for v in written.values())
    read = collections.Counter()
    for it in range((64 * D // 8) // 256):
        addrs = []
        for t in range(256):
            c = t + it * 256
            r, c8 = c // (D // 8), (c % (D // 8)) * 8
            addrs.append((r * RS + c8) * 2)
            for u in range(8):
                read[(r, c8 + u)] += 1
        for w in range(4):
            assert worst_conflict(addrs[w * 64:(w + 1) * 64], 16, 8) == 1
    assert read == written
