// Layout catalogue, relation builder and coordination scheduler (host).
#include "plan.hpp"

#include <algorithm>
#include <map>
#include <utility>

namespace b2b {

namespace {
// Published gfx950 (CDNA4) matrix-instruction shapes used by the cascade.
const MfmaShape kShapes[SH_COUNT] = {
    {16, 16, 32, 8, 4, 16},   // v_mfma_f32_16x16x32_f16
    {16, 16, 32, 8, 4, 16},   // v_mfma_f32_16x16x32_bf16
    {32, 32, 16, 8, 16, 16},  // v_mfma_f32_32x32x16_f16
    {32, 32, 16, 8, 16, 16},  // v_mfma_f32_32x32x16_bf16
    {16, 16, 16, 4, 4, 16},   // v_mfma_f32_16x16x16_f16
    {16, 16, 4, 1, 4, 64},    // v_mfma_f64_16x16x4_f64
};
}  // namespace

const MfmaShape& shape_info(Shape s) { return kShapes[s]; }

// A operand: lane owns one row (lane mod m); lanes are split into groups
// along k, each holding a contiguous run of a_elems k values.
void a_coord(Shape s, int lane, int e, int* row, int* k) {
    B2B_CHECK(s >= 0 && s < SH_COUNT && lane >= 0 && lane < kLanes);
    const MfmaShape& sh = kShapes[s];
    B2B_CHECK(e >= 0 && e < sh.a_elems);
    *row = lane % sh.m;
    *k = (lane / sh.m) * sh.a_elems + e;
    B2B_CHECK(*k < sh.k);
}

// B operand: the mirror image, lane owns one column.
void b_coord(Shape s, int lane, int e, int* k, int* col) {
    B2B_CHECK(s >= 0 && s < SH_COUNT && lane >= 0 && lane < kLanes);
    const MfmaShape& sh = kShapes[s];
    B2B_CHECK(e >= 0 && e < sh.a_elems);
    *col = lane % sh.n;
    *k = (lane / sh.n) * sh.a_elems + e;
    B2B_CHECK(*k < sh.k);
}

// Accumulator: lane owns one column.  float32 accumulators: rows come in
// blocks of 4 per lane group, the 32x32 shape repeating the 4-row block every
// 8 rows.  fp64 16x16x4: rows are interleaved, register e of lane group g
// holding row g + 4e (measured on gfx950 with a one-instruction probe).
void c_coord(Shape s, int lane, int e, int* row, int* col) {
    B2B_CHECK(s >= 0 && s < SH_COUNT && lane >= 0 && lane < kLanes);
    const MfmaShape& sh = kShapes[s];
    B2B_CHECK(e >= 0 && e < sh.c_elems);
    *col = lane % sh.n;
    int group = lane / sh.n;            // 4 groups of 16 lanes, or 2 of 32
    int groups = kLanes / sh.n;
    if (s == SH_F64_16x16x4) {
        *row = group + groups * e;
    } else {
        *row = (e / 4) * (4 * groups) + group * 4 + (e % 4);
    }
    B2B_CHECK(*row < sh.m);
}

static int gcd_i(int a, int b) { while (b) { int t = a % b; a = b; b = t; } return a; }

bool build_relation(Shape s, bool orient_n, Relation* out) {
    if (s < 0 || s >= SH_COUNT) return false;
    const MfmaShape& sh = kShapes[s];
    const int T = sh.n, KW = sh.k;
    const int W = T / gcd_i(T, KW) * KW;         // columns of C0 in one unit
    const int tiles = W / T, ksteps = W / KW;
    const int E = tiles * sh.c_elems;
    if (E != ksteps * sh.a_elems) return false;
    // where does each (m, n1) of the unit live in the accumulator registers?
    std::map<std::pair<int, int>, int> where;
    for (int t = 0; t < tiles; ++t)
        for (int l = 0; l < kLanes; ++l)
            for (int v = 0; v < sh.c_elems; ++v) {
                int i, j;
                c_coord(s, l, v, &i, &j);
                // transposed first GEMM: the tile is C0^T, rows are n1, columns m
                int m = orient_n ? i : j;
                int n1 = T * t + (orient_n ? j : i);
                if (!where.emplace(std::make_pair(m, n1), l * E + t * sh.c_elems + v).second)
                    return false;
            }
    out->elems = E;
    out->tiles = tiles;
    out->ksteps = ksteps;
    out->src_of.assign(kLanes * E, -1);
    std::vector<char> used(kLanes * E, 0);
    // the next GEMM consumes C0 as the operand that owns (row m, k = n1)
    for (int c = 0; c < ksteps; ++c)
        for (int l = 0; l < kLanes; ++l)
            for (int u = 0; u < sh.a_elems; ++u) {
                int k, m;
                b_coord(s, l, u, &k, &m);
                auto it = where.find(std::make_pair(m, KW * c + k));
                if (it == where.end() || used[it->second]) return false;
                used[it->second] = 1;
                B2B_CHECK(l * E + c * sh.a_elems + u < (int)out->src_of.size());
                out->src_of[l * E + c * sh.a_elems + u] = it->second;
            }
    // every source element feeds exactly one destination
    B2B_CHECK(std::find(used.begin(), used.end(), 0) == used.end());
    return true;
}

bool build_relation_from_labels(int elems, const int32_t* src, const int32_t* dst, Relation* out) {
    if (elems < 1 || !src || !dst) return false;
    const int n = kLanes * elems;
    std::map<int32_t, int> where;
    for (int i = 0; i < n; ++i)
        if (!where.emplace(src[i], i).second) return false;   // a label twice in the source
    out->elems = elems;
    out->tiles = 0;
    out->ksteps = 0;
    out->src_of.assign(n, -1);
    std::vector<char> used(n, 0);
    for (int d = 0; d < n; ++d) {
        auto it = where.find(dst[d]);
        if (it == where.end() || used[it->second]) return false;   // missing or taken twice
        used[it->second] = 1;
        out->src_of[d] = it->second;
    }
    return true;
}

bool pack_relation(const Relation& r, Relation* packed) {
    if (r.elems % 2) return false;
    const int E = r.elems, P = E / 2;
    packed->elems = P;
    packed->tiles = r.tiles;
    packed->ksteps = r.ksteps;
    packed->src_of.assign(kLanes * P, -1);
    for (int l = 0; l < kLanes; ++l)
        for (int a = 0; a < P; ++a) {
            int s0 = r.src_of[l * E + 2 * a], s1 = r.src_of[l * E + 2 * a + 1];
            if (s0 % 2 != 0 || s1 != s0 + 1) return false;   // pair split or reversed
            int lane = s0 / E, e = s0 % E;
            packed->src_of[l * P + a] = lane * P + e / 2;
        }
    return true;
}

namespace {
// Kuhn's augmenting path over receivers [from, n) with senders in `taken`
// unavailable; match[p] = receiver holding sender p or -1.
bool augment(int i, const std::vector<std::vector<int>>& adj, const std::vector<char>& taken,
             std::vector<int>& match, std::vector<char>& seen) {
    for (int p : adj[i]) {
        if (taken[p] || seen[p]) continue;
        seen[p] = 1;
        if (match[p] < 0 || augment(match[p], adj, taken, match, seen)) {
            match[p] = i;
            return true;
        }
    }
    return false;
}

bool rest_matchable(int from, const std::vector<std::vector<int>>& adj,
                    const std::vector<char>& taken) {
    const int n = (int)adj.size();
    std::vector<int> match(n, -1);
    std::vector<char> seen(n);
    for (int i = from; i < n; ++i) {
        std::fill(seen.begin(), seen.end(), 0);
        if (!augment(i, adj, taken, match, seen)) return false;
    }
    return true;
}
}  // namespace

bool build_schedule(const Relation& rel, Schedule* out) {
    const int n = kLanes, m = rel.elems;
    // open[i] lists (slot r) still to fill for receiver i, ascending
    std::vector<std::vector<int>> open(n);
    for (int i = 0; i < n; ++i)
        for (int r = 0; r < m; ++r) open[i].push_back(r);
    out->rounds = m;
    out->p.assign(m * n, -1);
    out->q.assign(m * n, -1);
    out->r.assign(m * n, -1);
    out->give.assign(m * n, -1);
    for (int j = 0; j < m; ++j) {
        std::vector<std::vector<int>> adj(n);
        for (int i = 0; i < n; ++i) {
            for (int r : open[i]) adj[i].push_back(rel.src_of[i * m + r] / m);
            std::sort(adj[i].begin(), adj[i].end());
            adj[i].erase(std::unique(adj[i].begin(), adj[i].end()), adj[i].end());
        }
        std::vector<char> taken(n, 0);
        for (int i = 0; i < n; ++i) {
            bool placed = false;
            for (size_t x = 0; x < open[i].size() && !placed; ++x) {
                int r = open[i][x];
                int src = rel.src_of[i * m + r];
                int p = src / m, q = src % m;
                if (taken[p]) continue;
                taken[p] = 1;
                if (!rest_matchable(i + 1, adj, taken)) { taken[p] = 0; continue; }
                out->p[j * n + i] = p;
                out->q[j * n + i] = q;
                out->r[j * n + i] = r;
                out->give[j * n + p] = q;
                open[i].erase(open[i].begin() + x);
                placed = true;
            }
            if (!placed) return false;
        }
    }
    return check_schedule(rel, *out);
}

bool check_schedule(const Relation& rel, const Schedule& s) {
    const int n = kLanes, m = rel.elems;
    if (s.rounds != m) return false;
    std::vector<int> got(n * m, -1);
    for (int j = 0; j < m; ++j) {
        std::vector<char> asked(n, 0);
        for (int i = 0; i < n; ++i) {
            int p = s.p[j * n + i];
            if (p < 0 || p >= n || asked[p]) return false;       // a sender asked twice
            asked[p] = 1;
            if (s.give[j * n + p] != s.q[j * n + i]) return false;
            int r = s.r[j * n + i];
            if (r < 0 || r >= m || got[i * m + r] >= 0) return false;
            got[i * m + r] = p * m + s.give[j * n + p];
        }
    }
    for (int d = 0; d < n * m; ++d)
        if (got[d] != rel.src_of[d]) return false;
    return true;
}

}  // namespace b2b
