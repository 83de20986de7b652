"""Pins of the rearrangement oracle: the pages' printed worked example
(tests/golden/page_example.json), the invariants the pages state for a
coordination matrix, and König's theorem on random relations."""
import json
import os
import random

import pytest

from oracle import remap as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_example.json")))


def _printed_relation():
    out = []
    for i in range(4):
        row = GOLD["relation"][f"new t{i}"]
        out.append([(int(t[1:]), int(c[1:])) for t, c in row])
    return out


def test_relation_builder_reproduces_printed_example():
    src, dst = R.page_example_layouts()
    rel = R.per_lane(R.relation(src, dst), 4, 4)
    assert rel == _printed_relation()


def test_coordination_matrix_row0_and_f0():
    H = R.coordination_matrix(_printed_relation())
    assert [list(c) for c in H[0]] == GOLD["fig4_row_thread0"]
    f, g, h = R.encode_fgh(H)
    f0 = [((i & 2) >> 1) + ((i & 1) << 1) for i in range(4)]   # the printed encoding of f0
    assert f[0] == f0
    ok, why = R.validate(H, _printed_relation())
    assert ok, why


def test_naive_schedule_is_rejected():
    """Taking destination slot r in round r (the unscheduled order) asks t0 for
    two different elements in the first round: not a valid coordination matrix."""
    rel = _printed_relation()
    naive = [[(p, q, r) for r, (p, q) in enumerate(row)] for row in rel]
    ok, why = R.validate(naive, rel)
    assert not ok and "round 0" in why


def test_register_group_offset():
    """A second register group (elements 4..7 of the same threads) lands at the
    same positions plus 4: the relation of the doubled example is block diagonal."""
    src, dst = [], []
    for t in range(4):
        for g in range(2):
            src += [(g, 0, 2 * t), (g, 0, 2 * t + 1), (g, 8, 2 * t), (g, 8, 2 * t + 1)]
    for i in range(4):
        for g in range(2):
            dst += [(g, 0, i), (g, 8, i), (g, 0, i + 4), (g, 8, i + 4)]
    rel = R.per_lane(R.relation(src, dst), 4, 8)
    base = _printed_relation()
    for i in range(4):
        assert rel[i][:4] == base[i]
        assert rel[i][4:] == [(p, q + 4) for p, q in base[i]]


SHAPES = ["f16_16x16x32", "bf16_16x16x32", "f16_32x32x16", "f16_16x16x16", "f64_16x16x4"]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("orient", ["T", "N"])
def test_cascade_relations_schedule_and_replay(shape, orient):
    src, dst, meta = R.cascade_layouts(shape, orient)
    rel = R.per_lane(R.relation(src, dst), 64, meta["elems"])
    H = R.coordination_matrix(rel)
    assert len(H[0]) == meta["elems"]
    ok, why = R.validate(H, rel)
    assert ok, why


def test_16x16x32_T_closed_form():
    """Orientation T, 16x16x32: destination lane l = m + 16g wants columns
    8g..8g+7 of row m.  Those live in accumulator tile g // 2 (16 columns each),
    in lane group 2(g % 2) + e // 2 (4 columns per lane group), packed pair
    e % 2 -- a move between 16-lane rows that keeps 16-bit pairs together."""
    src, dst, meta = R.cascade_layouts("f16_16x16x32", "T")
    rel = R.pack_pairs(R.per_lane(R.relation(src, dst), 64, 8))
    for l in range(64):
        m, g = l % 16, l // 16
        for e in range(4):
            tile, h, half = g // 2, 2 * (g % 2) + e // 2, e % 2
            assert rel[l][e] == (m + 16 * h, 2 * tile + half)


def test_16x16x16_T_is_identity():
    """With the legacy 16x16x16 shape the accumulator of the transposed first
    GEMM already is the second GEMM's operand: the rules are equal and the
    operators fuse directly."""
    src, dst, meta = R.cascade_layouts("f16_16x16x16", "T")
    assert R.relation(src, dst) == list(range(len(src)))


def test_f64_T_is_identity():
    """fp64: the accumulator of the transposed first GEMM holds row m, column
    g + 4v in register v of lane group g -- exactly the operand's K-step v,
    lane group g, k = 4v + g.  The rules are equal: fuse directly."""
    src, dst, meta = R.cascade_layouts("f64_16x16x4", "T")
    assert R.relation(src, dst) == list(range(len(src)))


def test_f64_N_moves_every_element_between_lane_groups():
    src, dst, meta = R.cascade_layouts("f64_16x16x4", "N")
    rel = R.per_lane(R.relation(src, dst), 64, 4)
    for l in range(64):
        m, g = l % 16, l // 16
        for s in range(4):     # wants column 4s + g of row m = (m % 4) + 4 (m // 4)
            assert rel[l][s] == ((4 * s + g) + 16 * (m % 4), m // 4)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("m", [2, 4, 8])
def test_random_relations_always_schedule(seed, m):
    """Any bijection between 64 lanes x m elements schedules in exactly m
    conflict-free rounds (the transfer multigraph is m-regular bipartite)."""
    rnd = random.Random(seed * 31 + m)
    cells = [(k, e) for k in range(64) for e in range(m)]
    rnd.shuffle(cells)
    rel = [cells[i * m:(i + 1) * m] for i in range(64)]
    H = R.coordination_matrix(rel)
    ok, why = R.validate(H, rel)
    assert ok, why


def test_non_bijection_rejected():
    with pytest.raises(ValueError):
        R.relation([(0, 0), (0, 1)], [(0, 0), (0, 0)])
    with pytest.raises(ValueError):
        R.relation([(0, 0), (0, 1)], [(0, 0), (1, 1)])
