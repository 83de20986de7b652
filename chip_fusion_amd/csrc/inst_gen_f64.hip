// fp64 instances with run-time widths (16x16x4 instruction).
#include "registry.hpp"
using namespace b2bk;
// (stages, max width, A tiles ahead, result tiles per group)
B2B_GEN64_INSTANCE(1, 64, 1, 4);
B2B_GEN64_INSTANCE(1, 128, 0, 2);
B2B_GEN64_INSTANCE(2, 64, 1, 4);
B2B_GEN64_INSTANCE(2, 128, 0, 2);
// two GEMMs up to 96 wide hold one A tile ahead (3-6 % faster than the
// 128-wide instance on 96x96x96 and 96x48x80)
B2B_GEN64_INSTANCE(2, 96, 1, 2);
B2B_GEN64_INSTANCE(3, 64, 1, 4);
B2B_GEN64_INSTANCE(3, 128, 0, 2);
B2B_GEN64_INSTANCE(4, 64, 1, 4);
B2B_GEN64_INSTANCE(5, 64, 1, 4);
