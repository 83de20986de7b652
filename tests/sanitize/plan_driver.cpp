// Drives the host planner (layout catalogue, relation builder, exchange
// scheduler, checker) over every shape and orientation and over random
// relations, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.
// Exit status 0 when every relation schedules and replays to itself.
#include <string>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <vector>

#include "plan.hpp"

int main(int argc, char** argv) {
    if (argc > 1 && std::string(argv[1]) == "--out-of-range") {
        // a planted mistake: an operand element past the shape's run; a
        // B2B_DEBUG build aborts naming the check
        int row, k;
        b2b::a_coord(b2b::SH_F16_16x16x32, 0, 99, &row, &k);
        std::printf("no check fired\n");
        return 0;
    }
    int failures = 0;
    for (int s = 0; s < b2b::SH_COUNT; ++s)
        for (int orn = 0; orn < 2; ++orn) {
            b2b::Relation rel, packed;
            if (!b2b::build_relation((b2b::Shape)s, orn != 0, &rel)) continue;
            for (int pk = 0; pk < 2; ++pk) {
                const b2b::Relation* use = &rel;
                if (pk) {
                    if (!b2b::pack_relation(rel, &packed)) continue;
                    use = &packed;
                }
                b2b::Schedule sch;
                if (!b2b::build_schedule(*use, &sch) || !b2b::check_schedule(*use, sch)) {
                    std::fprintf(stderr, "shape %d orient %d packed %d: no valid schedule\n", s, orn, pk);
                    ++failures;
                }
            }
        }
    // random bijections between two label layouts, 1..16 elements a lane
    std::mt19937 gen(12345);
    for (int trial = 0; trial < 200; ++trial) {
        const int e = 1 + trial % 16, n = 64 * e;
        std::vector<int32_t> src(n), dst(n);
        std::iota(src.begin(), src.end(), 1000);
        dst = src;
        std::shuffle(dst.begin(), dst.end(), gen);
        b2b::Relation rel;
        b2b::Schedule sch;
        if (!b2b::build_relation_from_labels(e, src.data(), dst.data(), &rel) || !b2b::build_schedule(rel, &sch) ||
            !b2b::check_schedule(rel, sch)) {
            std::fprintf(stderr, "random relation %d (E = %d) failed\n", trial, e);
            ++failures;
        }
    }
    // malformed label sets are refused
    std::vector<int32_t> a(64, 7), b(64, 7);
    b2b::Relation bad;
    if (b2b::build_relation_from_labels(1, a.data(), b.data(), &bad)) {
        std::fprintf(stderr, "repeated labels accepted\n");
        ++failures;
    }
    std::printf("plan driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
