"""CPU: the work plan of fa_fwd (fa_plan_describe, no GPU needed).

Every (batch*head, query tile) must see each of its key tiles in exactly one unit,
the unit table must fit its packed fields and the kernel's limits, and the plan
must keep the properties the kernels rely on (query tiles from the last one, the
same cut for every b*h, at most 16 ranges per tile, one dispatch wave of units).
"""

import math
import os

import pytest

from exact_attention_35_amd import capi

pytestmark = pytest.mark.skipif(not os.path.exists(capi.library_path()),
                                reason="libfa.so not built (run __graft_entry__.build())")


def ntiles(N, qt, causal, bm=128, bn=64, Nq=None):
    coff = 0 if Nq is None else N - Nq
    kv = max(0, min(N, (qt + 1) * bm + coff)) if causal else N
    return (kv + bn - 1) // bn


SHAPES = [  # (B, H, N, d, dv, causal)
    (1, 1, 8192, 128, 128, True), (1, 1, 8192, 128, 128, False), (1, 1, 1000, 128, 128, True),
    (1, 2, 1100, 128, 128, True), (1, 2, 1500, 128, 128, True), (1, 1, 16384, 128, 128, True),
    (1, 1, 32640, 128, 128, True), (1, 1, 32640, 64, 64, False), (2, 16, 600, 64, 128, False),
    (1, 64, 200, 64, 64, True), (1, 65, 200, 64, 64, True), (1, 1, 1, 64, 64, True),
    (1, 1, 129, 128, 64, True), (3, 5, 1000, 128, 64, False), (1, 8, 3000, 128, 128, True),
    (4, 32, 4096, 128, 128, True), (1, 8, 32768, 128, 128, True), (2, 16, 2048, 64, 128, False),
    (1, 4, 8192, 128, 128, True), (1, 3, 8192, 64, 64, False),
    (8, 32, 100, 128, 128, True), (2, 100, 40, 64, 64, False), (1, 300, 128, 128, 64, True),
    (1, 1, 32768, 128, 128, False), (1, 1, 32768, 64, 64, True),
]


def check_plan(info, table, B, H, Nq, Nk, dv, causal, cus):
    """Every (b*h, query tile) sees each of its key tiles in exactly one unit; the
    packed fields fit; the table keeps the order and limits the kernels rely on."""
    BH = B * H
    n_qt = math.ceil(Nq / 128)
    assert (info.n_qtiles, info.qtile_rows, info.key_tile) == (n_qt, 128, 64)
    if not info.split:
        assert info.units == BH * n_qt and info.merge_blocks == 0 and info.workspace_bytes == 0
        return 0
    # split only where the query tiles give the CUs fewer than two workgroups each,
    # within the table's limits (b*h < 64, or < 2^14 with a single query tile)
    assert BH * n_qt < 2 * cus and (BH <= 64 or n_qt == 1) and n_qt <= 256
    assert len(table) == info.units <= min(512, 2 * cus)
    G = 1 << info.unit_tile_shift
    assert 0 <= info.unit_tile_shift <= 15
    ranges, order = {}, []
    for w in table:
        qt, g0, gn, bh = w & 0xFF, (w >> 8) & 0x1FF, (w >> 17) & 0x1FF, w >> 26
        if n_qt == 1:  # the query-tile bits hold b*h's low 8 bits
            qt, bh = 0, (w & 0xFF) | (w >> 26) << 8
        assert qt < n_qt and bh < BH
        nt = ntiles(Nk, qt, causal, Nq=Nq)
        t0, t1 = g0 * G, min(g0 * G + gn * G, nt)  # the kernel's decode: clipped to the tile
        assert gn >= 1 or nt == 0
        assert t0 < t1 or nt == 0
        ranges.setdefault((qt, bh), []).append((t0, t1 - t0))
        order.append(qt)
    assert order == sorted(order, reverse=True)  # query tiles from the last one
    n_split = 0
    for qt in range(n_qt):
        cuts = [ranges[(qt, bh)] for bh in range(BH)]
        assert all(c == cuts[0] for c in cuts)  # the same cut for every b*h
        assert 1 <= len(cuts[0]) <= 16
        t = 0
        for t0, n in cuts[0]:
            assert t0 == t
            t += n
        assert t == ntiles(Nk, qt, causal, Nq=Nq)
        n_split += len(cuts[0]) > 1
    assert n_split > 0
    groups = 128 * dv // (1024 * 2)  # row groups of a query tile
    used = groups if n_qt > 1 else min(groups, -(-Nq // (128 // groups)))  # groups holding rows
    assert info.merge_blocks == n_split * BH * used
    assert info.workspace_bytes >= info.units * (8 + 2 * 128 * 4 + 128 * dv * 2)
    return n_split


@pytest.mark.parametrize("cus", [256, 80])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s}" for s in SHAPES])
def test_plan_covers_every_key_tile_once(shape, cus):
    B, H, N, d, dv, causal = shape
    info, table = capi.fa_plan_describe(B, H, N, d, dv, capi.FA_BF16, causal, cus)
    check_plan(info, table, B, H, N, N, dv, causal, cus)


RECT = [  # (B, H, N_q, N_k, causal): query tiles whose key ranges need more than 9 bits
    (1, 1, 1, 32769, True), (1, 1, 1, 40000, True), (1, 1, 1, 65536, False),
    (1, 8, 1, 65536, True), (1, 32, 1, 131072, True), (1, 1, 1, 600000, True),
    (1, 1, 128, 600000, False), (2, 2, 300, 70000, True), (1, 1, 1, 4097, True),
    (8, 32, 1, 8192, True), (1, 1, 2000, 100, True),
]


@pytest.mark.parametrize("cus", [256, 200, 80])
@pytest.mark.parametrize("shape", RECT, ids=[f"{s}" for s in RECT])
def test_rectangular_plan_fields_fit(shape, cus):
    B, H, Nq, Nk, causal = shape
    info, table = capi.fa_plan_describe_qk(B, H, Nq, Nk, 128, 128, capi.FA_BF16, causal, cus)
    n_split = check_plan(info, table, B, H, Nq, Nk, 128, causal, cus)
    longest = max(ntiles(Nk, qt, causal, Nq=Nq) for qt in range(math.ceil(Nq / 128)))
    if info.split:
        # the granule is the smallest one whose fields hold the longest tile's key tiles
        G = 1 << info.unit_tile_shift
        assert -(-longest // G) <= 511
        assert info.unit_tile_shift == 0 or -(-longest // (G // 2)) > 511
    if Nq == 1 and Nk >= 32769 and B * H < cus:
        assert info.split and n_split == 1  # long decoding rows are still split over keys


def test_headline_plan_fills_the_chip():
    # the single causal head of N = 8192 is cut into about two units per CU
    info, table = capi.fa_plan_describe(1, 1, 8192, 128, 128, capi.FA_BF16, True, 256)
    assert info.split and 400 <= info.units <= 512
    # the first workgroups of the CUs get more key tiles than the second ones
    first = [(w >> 17) & 0x1FF for w in table[:256]]
    second = [(w >> 17) & 0x1FF for w in table[256:]]
    assert sum(first) / len(first) > sum(second) / len(second)


def test_fp32_and_invalid_plans():
    info, table = capi.fa_plan_describe(1, 1, 256, 64, 64, capi.FA_F32, False, 256)
    assert (info.split, info.n_qtiles, info.units, info.qtile_rows) == (0, 0, 0, 64) and table == []
    # other widths take the general kernel: no matrix-core plan; fp16 at 64/128 has one
    info, table = capi.fa_plan_describe(1, 1, 256, 96, 64, capi.FA_BF16, False, 256)
    assert (info.split, info.units, info.qtile_rows) == (0, 0, 64) and table == []
    info, _ = capi.fa_plan_describe(1, 1, 256, 64, 64, capi.FA_F16, False, 256)
    assert info.qtile_rows == 128 and info.units >= 2
    with pytest.raises(capi.FaError):
        capi.fa_plan_describe(1, 1, 256, 257, 64, capi.FA_BF16, False, 256)
    with pytest.raises(capi.FaError):
        capi.fa_plan_describe(1, 1, 256, 64, 64, capi.FA_BF16, False, 0)
