"""Rearrangement oracle (TEST INFRASTRUCTURE ONLY; the product never imports it).

Page 1 ("数据处理方法、装置、设备及介质", detailed description) fuses two cascaded
GEMMs whose register layouts ("data-processing rules") differ.  The first
operator's result sits in a multi-thread register set in one layout, the second
operator wants its input in another; the method

  1. splits both register sets into groups and derives, element by element, the
     correspondence between them (the rearrangement relation; Figs. 2a/2b/3 and
     the worked tf32 example with threads t0..t3 and elements c0..c3);
  2. builds a coordination matrix H: in exchange round j, thread i takes element
     q of thread p and files it as its element r, each thread giving exactly one
     element and taking one per round, so that the p of one column never repeat
     (Fig. 4);
  3. encodes H as per-round functions f, g, h of the thread index (p, q, r),
     written with add / subtract / bit operations.

This module states those steps plainly on explicit index maps.  A layout is a
list ``coord[lane * E + e]`` giving the logical matrix coordinate held by element
``e`` of lane ``lane``.  The register layouts of the gfx950 matrix instructions
are written out here from AMD's published CDNA matrix-instruction layouts, on
their own, independently of the product library; a one-instruction GPU probe
with integer operands (tests/test_gpu_layouts.py) and the GPU parity tests pin
them to the hardware.
"""
from collections import defaultdict

LANES = 64


# ----------------------------------------------------------------------------
# Matrix-instruction fragment layouts on gfx950 (wave of 64 lanes).
# For each shape: operand A (rows x k), operand B (k x cols), accumulator C.
# Each function returns, for (lane, element), the coordinate in the tile.
# ----------------------------------------------------------------------------
class Shape:
    def __init__(self, name, m, n, k, a_elems, c_elems, a_fn, b_fn, c_fn, width_bits):
        self.name, self.m, self.n, self.k = name, m, n, k
        self.a_elems, self.c_elems = a_elems, c_elems
        self.a, self.b, self.c = a_fn, b_fn, c_fn
        self.width_bits = width_bits   # operand element width


def _s16x16x32(name):
    return Shape(name, 16, 16, 32, 8, 4,
                 lambda l, u: (l % 16, 8 * (l // 16) + u),
                 lambda l, u: (8 * (l // 16) + u, l % 16),
                 lambda l, v: (4 * (l // 16) + v, l % 16), 16)


def _s32x32x16(name):
    return Shape(name, 32, 32, 16, 8, 16,
                 lambda l, u: (l % 32, 8 * (l // 32) + u),
                 lambda l, u: (8 * (l // 32) + u, l % 32),
                 lambda l, v: (8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32), 16)


SHAPES = {
    "f16_16x16x32": _s16x16x32("f16_16x16x32"),
    "bf16_16x16x32": _s16x16x32("bf16_16x16x32"),
    "f16_32x32x16": _s32x32x16("f16_32x32x16"),
    "bf16_32x32x16": _s32x32x16("bf16_32x32x16"),
    "f16_16x16x16": Shape("f16_16x16x16", 16, 16, 16, 4, 4,
                          lambda l, u: (l % 16, 4 * (l // 16) + u),
                          lambda l, u: (4 * (l // 16) + u, l % 16),
                          lambda l, v: (4 * (l // 16) + v, l % 16), 16),
    # fp64: the accumulator interleaves rows -- register v of lane group g
    # holds row g + 4v (not 4g + v as in the float32 shapes)
    "f64_16x16x4": Shape("f64_16x16x4", 16, 16, 4, 1, 4,
                         lambda l, u: (l % 16, l // 16),
                         lambda l, u: (l // 16, l % 16),
                         lambda l, v: (l // 16 + 4 * v, l % 16), 64),
}


def _lcm(a, b):
    from math import gcd
    return a * b // gcd(a, b)


def cascade_layouts(shape_name, orientation):
    """Source and destination layouts of one remap unit of the cascade.

    The unit covers one M-tile (shape.m rows of the intermediate, which the
    second GEMM consumes as its K dimension) and the smallest run of the
    intermediate's columns that is a whole number of first-GEMM output tiles
    and of second-GEMM K-steps.

    Orientation "T" computes the first GEMM transposed (C0^T = B0^T . A^T) so an
    accumulator lane holds a row of C0; orientation "N" computes C0 = A . B0 so
    a lane holds a column.  Either way the second GEMM takes C0 as the operand
    holding (row m, k = column of C0) -- in the product it is the B operand of
    D^T = B1^T . C0^T, whose layout equals the A operand's.

    Returns (src, dst, meta): src[lane*Es + e] and dst[lane*Ed + e] are (m, n1)
    coordinates; the source element index is tile*C + reg, the destination
    element index is kstep*A + slot.
    """
    sh = SHAPES[shape_name]
    assert sh.m == sh.n
    T = sh.n                      # first-GEMM output tile width along n1
    KW = sh.k                     # second-GEMM K-step
    W = _lcm(T, KW)
    tiles, ksteps = W // T, W // KW
    Es, Ed = tiles * sh.c_elems, ksteps * sh.a_elems
    assert Es == Ed
    src = [None] * (LANES * Es)
    for t in range(tiles):
        for l in range(LANES):
            for v in range(sh.c_elems):
                i, j = sh.c(l, v)
                if orientation == "T":      # C0^T tile: row index is n1, column index is m
                    m, n1 = j, T * t + i
                elif orientation == "N":
                    m, n1 = i, T * t + j
                else:
                    raise ValueError(orientation)
                src[l * Es + t * sh.c_elems + v] = (m, n1)
    dst = [None] * (LANES * Ed)
    for c in range(ksteps):
        for l in range(LANES):
            for u in range(sh.a_elems):
                k, m = sh.b(l, u)          # B operand of D^T = B1^T . C0^T
                dst[l * Ed + c * sh.a_elems + u] = (m, KW * c + k)
    meta = {"tiles": tiles, "ksteps": ksteps, "elems": Es, "width": W,
            "c_elems": sh.c_elems, "a_elems": sh.a_elems}
    return src, dst, meta


def relation(src, dst):
    """rel[d] = s with src[s] == dst[d]; both must hold every coordinate once."""
    where = {}
    for s, c in enumerate(src):
        if c in where:
            raise ValueError(f"source layout holds {c} twice")
        where[c] = s
    if len(dst) != len(src):
        raise ValueError("layouts differ in size")
    rel = []
    seen = set()
    for c in dst:
        if c not in where:
            raise ValueError(f"destination wants {c}, which no source element holds")
        if c in seen:
            raise ValueError(f"destination holds {c} twice")
        seen.add(c)
        rel.append(where[c])
    return rel


def per_lane(rel, lanes, elems):
    """rel as [receiver][r] -> (sender p, element q)."""
    return [[divmod(rel[i * elems + r], elems) for r in range(elems)] for i in range(lanes)]


def pack_pairs(rel_lanes):
    """Relation on 32-bit containers of two adjacent 16-bit elements.

    Valid only when every destination pair (2a, 2a+1) comes from one source
    pair (2b, 2b+1) of one sender, in order; raises otherwise.
    """
    out = []
    for row in rel_lanes:
        prow = []
        for a in range(len(row) // 2):
            (p0, q0), (p1, q1) = row[2 * a], row[2 * a + 1]
            if p0 != p1 or q0 % 2 or q1 != q0 + 1:
                raise ValueError("relation does not keep 16-bit pairs together")
            prow.append((p0, q0 // 2))
        out.append(prow)
    return out


# ----------------------------------------------------------------------------
# Coordination matrix (Fig. 4): in round j receiver i takes element q of sender
# p and files it as its element r.  Per round every sender appears once.  The
# figure shows only row 0; rounds are chosen here as the lexicographically
# first perfect matching (receivers ascending, each taking its lowest
# destination slot r still open), which reproduces the printed row and the
# printed f0.  Existence in every round: the remaining transfers form a
# regular bipartite multigraph (each receiver still needs as many elements as
# each sender still holds), which always has a perfect matching.
# ----------------------------------------------------------------------------
def _augment_filtered(i, adj, match_sender, seen, banned):
    for p in adj[i]:
        if p in banned or p in seen:
            continue
        seen.add(p)
        cur = match_sender.get(p)
        if cur is None or (cur != -1 and _augment_filtered(cur, adj, match_sender, seen, banned)):
            match_sender[p] = i
            return True
    return False


def coordination_matrix(rel_lanes):
    """H[i][j] = (p, q, r) for every receiver i and round j."""
    n = len(rel_lanes)
    m = len(rel_lanes[0])
    remaining = [sorted(((p, q, r) for r, (p, q) in enumerate(row)), key=lambda t: t[2])
                 for row in rel_lanes]
    H = [[None] * m for _ in range(n)]
    for j in range(m):
        adj = {i: sorted({p for (p, _, _) in remaining[i]}) for i in range(n)}
        fixed = set()
        for i in range(n):
            for opt in remaining[i]:
                p = opt[0]
                if p in fixed:
                    continue
                trial = fixed | {p}
                ms = {}
                ok = True
                for i2 in range(i + 1, n):
                    if not _augment_filtered(i2, adj, ms, set(), trial):
                        ok = False
                        break
                if ok:
                    H[i][j] = opt
                    fixed = trial
                    remaining[i].remove(opt)
                    break
            else:
                raise RuntimeError("no perfect matching; the relation is not a bijection")
    return H


def sender_table(H):
    """s[j][k]: the element sender k offers in round j (the q asked of it)."""
    n, m = len(H), len(H[0])
    s = [[None] * n for _ in range(m)]
    for i in range(n):
        for j in range(m):
            p, q, _ = H[i][j]
            if s[j][p] is not None:
                raise ValueError(f"round {j}: sender {p} asked twice")
            s[j][p] = q
    return s


def validate(H, rel_lanes):
    """Checks the invariants the pages state for a coordination matrix."""
    n, m = len(H), len(H[0])
    for j in range(m):
        ps = [H[i][j][0] for i in range(n)]
        if len(set(ps)) != n:
            return False, f"round {j}: a sender is asked twice"
    for i in range(n):
        if sorted(H[i][j][2] for j in range(m)) != list(range(m)):
            return False, f"receiver {i}: destination slots not filled exactly once"
    src = [[(k, e) for e in range(m)] for k in range(n)]
    out = replay(H, src)
    for i in range(n):
        for r in range(m):
            if out[i][r] != tuple(rel_lanes[i][r]):
                return False, f"replay mismatch at receiver {i} slot {r}"
    return True, "ok"


def replay(H, data):
    """Runs the exchange rounds on data[k][e]; returns the rearranged data."""
    n, m = len(H), len(H[0])
    s = sender_table(H)
    out = [[None] * m for _ in range(n)]
    for j in range(m):
        offered = [data[k][s[j][k]] for k in range(n)]   # each sender gives one element
        for i in range(n):
            p, _, r = H[i][j]
            out[i][r] = offered[p]                          # each receiver takes one
    return out


def encode_fgh(H):
    """Splits H into per-round tables f_j(i) = p, g_j(i) = q, h_j(i) = r."""
    n, m = len(H), len(H[0])
    f = [[H[i][j][0] for i in range(n)] for j in range(m)]
    g = [[H[i][j][1] for i in range(n)] for j in range(m)]
    h = [[H[i][j][2] for i in range(n)] for j in range(m)]
    return f, g, h


# ----------------------------------------------------------------------------
# The worked example of the pages (tf32 cascade on "a certain GPGPU", groups of
# four threads with four elements each).  Read as: accumulator thread t holds
# the result row pair (r, r+8) at columns 2t, 2t+1 as c0 = (r, 2t),
# c1 = (r, 2t+1), c2 = (r+8, 2t), c3 = (r+8, 2t+1); the second operator's
# thread i wants (r, i), (r+8, i), (r, i+4), (r+8, i+4).  Building the relation
# from these two layouts must give the printed newt0..newt3.
# ----------------------------------------------------------------------------
def page_example_layouts():
    src, dst = [], []
    for t in range(4):
        src += [(0, 2 * t), (0, 2 * t + 1), (8, 2 * t), (8, 2 * t + 1)]
    for i in range(4):
        dst += [(0, i), (8, i), (0, i + 4), (8, i + 4)]
    return src, dst
