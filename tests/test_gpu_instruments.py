"""The measurement instruments (include/b2b_bench.h) move and compute what
they claim: the copy and the mixed stream write exactly the bytes their
definitions give and nothing past them; the matrix-core loop runs the rounds
and chains its FLOP count assumes."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _bytes(n, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()


# pieces of 16 bytes: below one grid stride, a ragged tail, several strides
@pytest.mark.parametrize("n16,wgs", [(4, 1), (1000, 3), (70000, 64)])
def test_copy_writes_src(n16, wgs):
    _flush(f"bench copy {n16} pieces, {wgs} workgroups")
    n = 16 * n16
    src = _bytes(n, n16)
    guard = _bytes(n + 4096, n16 + 1)
    keep = guard[n:].clone()
    cf.bench_copy(src, guard[:n], wgs)
    torch.cuda.synchronize()
    assert torch.equal(guard[:n], src)
    assert torch.equal(guard[n:], keep)


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("n16,wgs", [(4, 1), (1000, 3), (70000, 64)])
def test_stream_folds_r_streams(R, n16, wgs):
    _flush(f"bench stream R={R} {n16} pieces, {wgs} workgroups")
    n = 16 * n16
    src = _bytes(R * n, 7 * R + n16)
    guard = _bytes(n + 4096, n16 + 2)
    keep = guard[n:].clone()
    cf.bench_stream(src, guard[:n], wgs)
    torch.cuda.synchronize()
    parts = src.cpu().numpy().reshape(R, n)
    want = np.bitwise_xor.reduce(parts, axis=0)
    assert np.array_equal(guard[:n].cpu().numpy(), want)
    assert torch.equal(guard[n:], keep)


@pytest.mark.parametrize("dtype,per_round", [("f16", 8.0), ("bf16", 8.0), ("f64", 32.0)])
def test_mfma_loop_rounds_and_chains(dtype, per_round):
    """Operands 1/16 (16-bit: 32-term dot products of 1/256 = 1/8 per
    instruction and element; 16 chains x 4 elements per lane) and 1/2 (fp64:
    4 terms of 1/4 = 1; 8 chains x 4 elements): every thread's sum is exactly
    per_round x iters, and the FLOP count is workgroups x 4 waves x iters x
    chains x the instruction's 2 M N K."""
    _flush(f"bench mfma {dtype}")
    wgs, iters = 8, 64
    sink = torch.full((wgs * 256,), -1.0, dtype=torch.float64, device="cuda")
    flop = cf.bench_mfma(dtype, wgs, iters, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == per_round * iters)
    chains, mnk = (16, 16 * 16 * 32) if dtype != "f64" else (8, 16 * 16 * 4)
    assert flop == wgs * 4 * iters * chains * 2 * mnk
