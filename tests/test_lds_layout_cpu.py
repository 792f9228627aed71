"""Host check of the LDS layout of the gradient kernel's Q, dO and K tiles.

Those tiles are read both row-wise (ds_read_b128: lane l reads row l mod 32, 16-byte
chunk 2*kk + l/32) and transposed (ds_read_b64_tr_b16: within a 16-lane group G, lane L
reads row 16*sg + 8*hh + 4*(lane/32) + L/4 at columns 32*db + 16*(G mod 2) + 4*(L mod 4)),
and their 16-byte chunks are XOR-swizzled by key(row) = s(row mod 4) ^ ((row/4) mod 4),
s = (0, 10, 4, 14). This test restates that address arithmetic (TileReads in
fa_bwd_mfma.hip) and checks that neither read has a bank conflict, whether the LDS serves
128 or 256 bytes per clock, and that the kernel's XOR form of each offset (a per-lane base
XOR a compile-time constant) equals the plain one.
"""

import pytest


def dual_key(row):
    return ((row & 1) * 10 + (row & 2) * 2) ^ ((row >> 2) & 3)


def row_offsets(W, kk):
    ch = W // 8
    return [(l & 31) * W * 2 + (((2 * kk + (l >> 5)) ^ (dual_key(l & 31) & (ch - 1))) * 16) for l in range(64)]


def tr_offsets(W, sg, db, hh):
    ch = W // 8
    out = []
    for lane in range(64):
        g, G, L = lane >> 5, lane >> 4, lane & 15
        row = 16 * sg + 8 * hh + 4 * g + (L >> 2)
        col = 32 * db + 16 * (G & 1) + 4 * (L & 3)
        out.append(row * W * 2 + (((col >> 3) ^ (dual_key(row) & (ch - 1))) * 16) + (col & 7) * 2)
    return out


def max_ways(offsets, size, lanes_per_clock, bytes_per_clock):
    worst = 1
    for g0 in range(0, 64, lanes_per_clock):
        banks = {}
        for o in offsets[g0:g0 + lanes_per_clock]:
            for b in range(o // 4, (o + size) // 4):
                k = b % (bytes_per_clock // 4)
                banks[k] = banks.get(k, 0) + 1
        worst = max(worst, max(banks.values()))
    return worst


@pytest.mark.parametrize("W", [64, 128])
@pytest.mark.parametrize("bytes_per_clock", [128, 256])
def test_row_and_transposed_reads_are_conflict_free(W, bytes_per_clock):
    for kk in range(W // 16):
        assert max_ways(row_offsets(W, kk), 16, bytes_per_clock // 16, bytes_per_clock) == 1
    for sg in range(4):
        for db in range(W // 32):
            for hh in range(2):
                assert max_ways(tr_offsets(W, sg, db, hh), 8, bytes_per_clock // 8, bytes_per_clock) == 1


@pytest.mark.parametrize("W", [64, 128])
def test_xor_form_of_the_offsets(W):
    ch = W // 8
    for lane in range(64):
        g, l32, G, L = lane >> 5, lane & 31, lane >> 4, lane & 15
        rbase = (l32 * W * 2) | (((g ^ dual_key(l32)) & (ch - 1)) * 16)
        for kk in range(W // 16):
            assert row_offsets(W, kk)[lane] == rbase ^ (32 * kk)
        c1 = 16 * (G & 1) + 4 * (L & 3)
        for hh in range(2):
            row = 8 * hh + 4 * g + (L >> 2)
            tb = (row * W * 2) | ((((c1 >> 3) ^ dual_key(row)) & (ch - 1)) * 16) | ((c1 & 7) * 2)
            for db in range(W // 32):
                assert tr_offsets(W, 0, db, hh)[lane] == tb ^ (64 * db)
