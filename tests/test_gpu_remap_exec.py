"""Compiled coordination rounds executed on the GPU (b2b_remap_execute, one
ds_bpermute per round): index payloads come out exactly where the relation
puts them, for random relations of every element count, the catalogue's
cascade pairs and a mixed-shape pair (16x16x32 result -> 32x32x16 operand)."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
from oracle import remap as R
from test_remap_compile import _labels, mixed_shape_layouts

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _check(src, dst, what):
    rel, p, q, r = cf.remap_compile(src, dst)
    n = src.size
    payload = torch.tensor(np.arange(n, dtype=np.int32) * 3 + 11, device="cuda")
    out = cf.remap_execute(p, q, r, payload)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = (np.arange(n, dtype=np.int64) * 3 + 11)[rel]
    assert np.array_equal(got, want), f"{what}: {int((got != want).sum())} elements misplaced"


@pytest.mark.parametrize("E", [1, 2, 4, 7, 8, 16])
def test_random_relations_on_device(E):
    _flush(f"remap exec random E={E}")
    rng = np.random.default_rng(77 + E)
    src = rng.permutation(64 * E).astype(np.int32)
    _check(src, rng.permutation(src), f"random E={E}")


@pytest.mark.parametrize("shape,orient", [("f16_16x16x32", "T"), ("f16_16x16x32", "N"),
                                          ("f16_32x32x16", "T"), ("f64_16x16x4", "N")])
def test_catalogue_pairs_on_device(shape, orient):
    _flush(f"remap exec {shape} {orient}")
    src, dst, meta = R.cascade_layouts(shape, orient)
    _check(_labels(src, meta["width"]), _labels(dst, meta["width"]), f"{shape} {orient}")


def test_mixed_shape_pair_on_device():
    _flush("remap exec mixed 16x16x32 -> 32x32x16")
    src, dst = mixed_shape_layouts()
    _check(_labels(src, 32), _labels(dst, 32), "mixed shapes")
