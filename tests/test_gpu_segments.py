"""Workgroups whose tile range crosses a batch boundary.

Each workgroup walks a contiguous range of row tiles; where that range holds
tiles of two batches, the kernel stages the second batch's weights partway
through (a second weight segment, the path after the first segment's copies,
which go out at the kernel's entry).  For every kernel family a (batch, M) is
chosen from the plan's own tile height and grid so that some workgroup's range
straddles a batch boundary; the rows of those workgroups' tiles and a random
sample of the others are checked against the oracle (the fp8 cascade against
its unfused form, bit for bit), and no element of D is left unwritten."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close, nan_output

pytestmark = pytest.mark.gpu

FAMILIES = [
    # name, type (or a type per GEMM and D), widths, plan options
    ("fixed fp16, two GEMMs", "f16", (128, 128, 128), {}),
    ("fixed fp16, three GEMMs", "f16", (128, 128, 128, 64), {}),
    ("fixed fp64", "f64", (64, 64, 64), {}),
    ("column split bf16", "bf16", (256, 256, 256), {}),
    ("32x32x16 fp16, two GEMMs", "f16", (128, 128, 128), {"mfma32": True}),
    ("32x32x16 fp16, three GEMMs", "f16", (128, 128, 128, 64), {"mfma32": True}),
    ("32x32x16 bf16 256 wide", "bf16", (256, 128, 256), {}),
    ("32x32x16 five GEMMs", "f16", (128, 128, 128, 128, 128, 64), {}),
    ("type per stage, read at run time", ("f16", "bf16", "f16", "bf16", "f16", "f16"),
     (128, 128, 128, 128, 128, 64), {}),
    ("fp64 run-time widths", "f64", (48, 48, 48), {}),
    ("fp64 run-time widths, four GEMMs", "f64", (64, 64, 64, 64, 64), {}),
    ("fp64 run-time widths up to 96", "f64", (96, 80, 96), {}),
    ("32x32x16 fp16 up to 192", "f16", (192, 160, 192), {}),
    ("32x32x16 bf16 chain up to 192", "bf16", (192, 64, 192, 64, 192), {}),
    ("tf32, two GEMMs", "tf32", (128, 128, 128), {}),
    ("tf32, three GEMMs", "tf32", (128, 128, 128, 64), {}),
    ("fp8 second GEMM", ("f16", "fp8", "f16"), (128, 128, 128), {}),
    ("fp8 second GEMM, 256 wide", ("bf16", "fp8", "bf16"), (256, 128, 256), {}),
]


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _plan(kind, batch, M, widths, opts, unfused=False):
    if isinstance(kind, tuple):
        return cf.Chain(list(kind), batch, M, list(widths), unfused=unfused)
    return cf.Chain(kind, batch, M, list(widths), unfused=unfused, **opts)


def _info(p):
    return dict(kv.split("=", 1) for kv in p.info().split())


def ranges(total, grid):
    """The workgroups' tile ranges, as the kernels partition them."""
    g = min(grid, total)
    per, extra = divmod(total, g)
    out = []
    for lid in range(g):
        t0 = lid * per + min(lid, extra)
        out.append((t0, t0 + per + (1 if lid < extra else 0)))
    return out


def straddling_shape(rows_wg, grid):
    """(batch, M, straddling ranges): the fewest tiles (more than the grid,
    so that some workgroups take two) for which a workgroup's range holds
    tiles of two batches; M leaves the last tile of each batch ragged."""
    for total in range(grid + 1, 3 * grid):
        for batch in range(2, 12):
            if total % batch:
                continue
            tb = total // batch
            if tb < 2:
                continue
            st = [(t0, t1) for t0, t1 in ranges(total, grid) if t1 > t0 and t0 // tb != (t1 - 1) // tb]
            if st:
                return batch, tb * rows_wg - rows_wg // 3, tb, st
    raise AssertionError("no straddling shape")


def test_ranges_helper_matches_the_partition():
    """The helper covers every tile once, in order (host-side sanity)."""
    for total, grid in [(300, 256), (513, 512), (7, 256), (1024, 256)]:
        r = ranges(total, grid)
        assert r[0][0] == 0 and r[-1][1] == total
        assert all(a[1] == b[0] for a, b in zip(r, r[1:]))


@pytest.mark.parametrize("fam", range(len(FAMILIES)))
def test_second_weight_segment(fam):
    name, kind, widths, opts = FAMILIES[fam]
    # the plan sizes its grid at its first launch: one small launch first
    types = list(kind) if isinstance(kind, tuple) else [kind] * len(widths)
    probe = _plan(kind, 1, 1000, widths, opts)
    tdt = {"tf32": torch.float32, "fp8": torch.uint8}
    zeros = lambda shape, t: torch.zeros(shape, dtype=tdt.get(t, cf.TORCH_DTYPES.get(cf.DTYPES.get(t))),
                                         device="cuda")
    probe.run(zeros((1, 1000, widths[0]), types[0]),
              *[zeros((1, widths[s], widths[s + 1]), types[s]) for s in range(len(widths) - 1)],
              D=zeros((1, 1000, widths[-1]), types[-1]))
    torch.cuda.synchronize()
    pi = _info(probe)
    probe.close()
    rows_wg, grid = int(pi["rows_per_wg"]), int(pi["grid"])
    assert grid > 0, pi
    batch, M, tb, st = straddling_shape(rows_wg, grid)
    _flush(f"segments {name}: batch={batch} M={M} ({tb} tiles of {rows_wg} rows a batch, grid {grid}, "
           f"{len(st)} straddling workgroups)")
    seed = 0x5E6A0000 + 97 * fam
    A = synth.tensor(seed, 0, (batch, M, widths[0]), types[0], "normal")
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), types[s], "normal",
                       1.0 / math.sqrt(widths[s])) for s in range(len(widths) - 1)]
    p = _plan(kind, batch, M, widths, opts)

    def run(plan):
        if types[0] == "tf32":
            Ad = torch.from_numpy(A).cuda()
            Bd = [torch.from_numpy(b).cuda() for b in Bs]
            D = torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float32, device="cuda")
        else:
            Ad = cf.to_device(A, types[0])
            Bd = [cf.to_device(b, types[s]) for s, b in enumerate(Bs)]
            D = nan_output(types[-1], batch, M, widths[-1])
        plan.run(Ad, *Bd, D=D)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(D).all()), f"{name}: D has unwritten elements"
        return cf.to_host(D)

    got = run(p)
    info = _info(p)
    p.close()
    assert (int(info["rows_per_wg"]), int(info["grid"])) == (rows_wg, grid), info
    if "fp8" in types:
        # the unfused form rounds the intermediate to the same E4M3 codes and
        # multiplies in the same slot order: identical D
        pu = _plan(kind, batch, M, widths, opts, unfused=True)
        ref = run(pu)
        pu.close()
        assert np.array_equal(got, ref), f"{name}: fused and unfused D differ"
        return
    # rows of the straddling workgroups' tiles, and a random sample of the rest
    sel = set()
    for t0, t1 in st:
        for t in range(t0, t1):
            b, r0 = divmod(t, tb)
            r0 *= rows_wg
            sel.update(b * M + r for r in range(r0, min(r0 + rows_wg, M)))
    rng = np.random.default_rng(seed)
    sel.update(rng.integers(0, batch * M, 256).tolist())
    rows = np.array(sorted(sel), np.int64)
    g = got.reshape(batch * M, widths[-1])[rows]
    if types[0] == "tf32":
        ref = oracle.cascade("tf32", A, Bs, rows=rows).astype(np.float64)
        gv = g.astype(np.float64)
        assert np.linalg.norm(gv - ref) / np.linalg.norm(ref) <= 1e-3, name
    else:
        ref = oracle.cascade(types if len(set(types)) > 1 else types[0], A, Bs, rows=rows)
        assert_close(types[-1], g, ref, f"{name} batch={batch} M={M}")
