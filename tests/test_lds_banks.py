"""LDS bank mapping of the attention kernels' tile accesses (host only).

The kernels keep 64-row K / V / Q / dO tiles in LDS, each row's 16-byte
pieces permuted by the library's swizzle (queried through the C ABI, so
these checks follow the shipped layout). The model: 64 banks of 4 bytes,
one 256-byte sweep per LDS cycle, so a 16-byte-per-lane access is served 16
lanes at a time and an 8-byte-per-lane access 32 lanes at a time; a cycle
conflicts when two lanes touch the same bank at different addresses. (On
the box the bank-conflict counter of the forward fell from 5.1e7 to 1.2e6
cycles per launch at the 480p layer when the transposed V reads became
conflict-free in this model.)
"""

import numpy as np
import pytest

import block_sparse_attention_avg_amd as bsa

BANKS, WORD = 64, 4


@pytest.fixture(scope="module")
def swz():
    lib = bsa.load()
    return lambda d, r: lib.bsa_lds_swizzle(d, r)


def _conflicts(addrs, nbytes, group):
    """Worst number of distinct addresses sharing one bank within a group of
    `group` lanes, over all groups (1 = conflict-free)."""
    worst = 1
    for g0 in range(0, len(addrs), group):
        banks = {}
        for a in addrs[g0:g0 + group]:
            for w in range(nbytes // WORD):
                b = ((a + WORD * w) // WORD) % BANKS
                banks.setdefault(b, set()).add(a + WORD * w)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


def test_swizzle_is_a_permutation(swz):
    for d in (64, 128):
        vals = [swz(d, r) for r in range(16)]
        if d == 128:
            assert sorted(vals) == list(range(16))
        # rows r and r + 8 differ by one constant (the transposed reads rely on it)
        assert len({swz(d, r) ^ swz(d, r + 8) for r in range(8)}) == 1
    assert swz(32, 0) == -1


def test_row_operand_reads_are_conflict_free(swz):
    # k_read / row_read: lane (l32, half) reads row 32 kb + l32, data piece
    # 2 cc + half, 16 bytes (d = 128: 256-byte rows)
    d, rowb = 128, 256
    for kb in range(2):
        for cc in range(8):
            addrs = []
            for lane in range(64):
                half, l32 = lane >> 5, lane & 31
                row = 32 * kb + l32
                addrs.append(row * rowb + (((2 * cc + half) ^ swz(d, l32 & 15)) << 4))
            assert _conflicts(addrs, 16, 16) == 1, (kb, cc)


def test_transposed_reads_are_conflict_free(swz):
    # v_read / tr_read (ds_read_b64_tr_b16): lane (g16, sj, sq) of half h
    # addresses row 8 t + 4 h + sj (+ 32 kb + 16 hh), data piece
    # 4 dg + 2 g16 + (sq >> 1), byte 8 (sq & 1)
    d, rowb = 128, 256
    for base in (0, 16, 32, 48):
        for dg in range(4):
            for t in range(2):
                addrs = []
                for lane in range(64):
                    half, g16, sj, sq = lane >> 5, (lane >> 4) & 1, (lane & 15) >> 2, lane & 3
                    row = 8 * t + 4 * half + sj
                    piece = 4 * dg + 2 * g16 + (sq >> 1)
                    addrs.append((base + row) * rowb + ((piece ^ swz(d, row & 15)) << 4) + 8 * (sq & 1))
                assert _conflicts(addrs, 8, 32) == 1, (base, dg, t)


def test_tile_loads_and_output_reads_are_conflict_free(swz):
    d, rowb, ppr = 128, 256, 16
    # direct-to-LDS loads write 16 bytes per lane at consecutive addresses
    assert _conflicts([16 * lane for lane in range(64)], 16, 16) == 1
    # the epilogue reads one output row (its 16 pieces) per 16 lanes
    for r in range(4):
        addrs = []
        for tid in range(64):
            u = tid + 64 * r
            row, p = u // ppr, u % ppr
            addrs.append(row * rowb + ((p ^ swz(d, row & 15)) << 4))
        assert _conflicts(addrs, 16, 16) == 1


def test_epilogue_staging_writes_at_most_two_way(swz):
    # accumulators to rows: lane (l32, half) of wave w writes 8 bytes of row
    # 32 w + l32 at data piece 4 dg + j4; rows 16 apart share a swizzle, so
    # these once-per-tile writes meet 2-way conflicts
    d, rowb = 128, 256
    for dg in range(4):
        for j4 in range(4):
            addrs = []
            for lane in range(64):
                half, l32 = lane >> 5, lane & 31
                addrs.append(l32 * rowb + (((4 * dg + j4) ^ swz(d, l32 & 15)) << 4) + 8 * half)
            assert _conflicts(addrs, 8, 32) <= 2
