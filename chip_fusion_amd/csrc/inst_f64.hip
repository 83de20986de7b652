// Kernel instances: fp64, K = N1 = N2 = 64.
#include "registry.hpp"
using namespace b2bk;
B2B_INSTANCE(DT_F64, 2, 64, 64, 64, 0, MODE_RELABEL, false, 1, 8, KM_PAIR64);
B2B_INSTANCE(DT_F64, 2, 64, 64, 64, 0, MODE_PERMLANE, false, 1, 8, KM_PAIR64);
B2B_INSTANCE(DT_F64, 2, 64, 64, 64, 0, MODE_BPERM, false, 1, 8, KM_PAIR64);
B2B_INSTANCE(DT_F64, 2, 64, 64, 64, 0, MODE_LDS, false, 1, 8, KM_PAIR64);
B2B_INSTANCE(DT_F64, 2, 64, 64, 64, 0, MODE_BPERM, true, 1, 8, KM_PAIR64);
B2B_INSTANCE(DT_F64, 2, 64, 64, 64, 0, MODE_LDS, true, 1, 8, KM_PAIR64, 1);
