"""The remap compiler (b2b_remap_compile) on the host: for every layout pair
of the catalogue its relation equals the oracle's and its rounds pass the
oracle's checks (one give and one take per lane per round, distinct senders,
replay equals the relation); random relations of every element count and a
mixed-shape pair (a 16x16x32 result feeding a 32x32x16 operand) schedule as
well; inconsistent layouts are refused."""
import numpy as np
import pytest

import chip_fusion_amd as cf
from oracle import remap as R


def _labels(coords, width):
    return np.array([m * width + n for m, n in coords], np.int32)


def _H(p, q, r):
    """receiver-major coordination matrix H[i][j] = (p, q, r) from round-major tables"""
    E = p.shape[0]
    return [[(int(p[j, i]), int(q[j, i]), int(r[j, i])) for j in range(E)] for i in range(64)]


@pytest.mark.parametrize("shape", ["f16_16x16x32", "f16_32x32x16", "f16_16x16x16", "f64_16x16x4"])
@pytest.mark.parametrize("orient", ["T", "N"])
def test_catalogue_pairs_match_oracle(shape, orient):
    src, dst, meta = R.cascade_layouts(shape, orient)
    width = meta["width"]
    rel, p, q, r = cf.remap_compile(_labels(src, width), _labels(dst, width))
    want = R.relation(src, dst)
    assert list(rel) == want
    ok, why = R.validate(_H(p, q, r), R.per_lane(want, 64, meta["elems"]))
    assert ok, why


@pytest.mark.parametrize("E", [1, 2, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("seed", [0, 1])
def test_random_relations(E, seed):
    rng = np.random.default_rng(1000 * E + seed)
    src = rng.permutation(64 * E).astype(np.int32) * 7 + 3      # arbitrary labels
    dst = rng.permutation(src)
    rel, p, q, r = cf.remap_compile(src, dst)
    assert np.array_equal(src[rel], dst)
    ok, why = R.validate(_H(p, q, r), R.per_lane(list(rel), 64, E))
    assert ok, why


def mixed_shape_layouts():
    """A 16x16x32 first GEMM (transposed) feeding a 32x32x16 second GEMM:
    source = two 16-row units of 16x16x32 results (rows m 0-15, 16-31; each
    two 16-column tiles, 8 values per lane), destination = two K-steps of the
    32x32x16 operand (lane l: row l%32, k = 8(l/32) + u).  Labels m*32 + n1."""
    s16 = R.SHAPES["f16_16x16x32"]
    s32 = R.SHAPES["f16_32x32x16"]
    E = 16
    src = [None] * (64 * E)
    for half in range(2):               # rows 16*half .. +15
        for t in range(2):              # 16-column tiles of the intermediate
            for l in range(64):
                for v in range(s16.c_elems):
                    i, j = s16.c(l, v)   # result of C0^T: i = n1 within the tile, j = m
                    src[l * E + half * 8 + t * 4 + v] = (16 * half + j, 16 * t + i)
    dst = [None] * (64 * E)
    for c in range(2):                  # K-steps of 16
        for l in range(64):
            for u in range(s32.a_elems):
                k, m = s32.b(l, u)
                dst[l * E + c * 8 + u] = (m, 16 * c + k)
    return src, dst


def test_mixed_shape_pair():
    src, dst = mixed_shape_layouts()
    rel, p, q, r = cf.remap_compile(_labels(src, 32), _labels(dst, 32))
    want = R.relation(src, dst)
    assert list(rel) == want
    ok, why = R.validate(_H(p, q, r), R.per_lane(want, 64, 16))
    assert ok, why


def test_refuses_inconsistent_layouts():
    src = np.arange(128, dtype=np.int32)
    with pytest.raises(cf.B2BError):
        cf.remap_compile(src, np.r_[src[:-1], 0].astype(np.int32))        # a label twice
    with pytest.raises(cf.B2BError):
        cf.remap_compile(src, src + 1)                                    # different labels
    with pytest.raises(cf.B2BError):
        cf.remap_compile(np.arange(64 * 17, dtype=np.int32), np.arange(64 * 17, dtype=np.int32))   # E > 16
