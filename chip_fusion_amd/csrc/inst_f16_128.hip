// Kernel instances: fp16, K = N1 = N2 = 128.
#include "registry.hpp"
using namespace b2bk;
B2B_INSTANCE(DT_F16, 2, 128, 128, 128, 0, MODE_RELABEL, false, 1, 8, KM_NAT, 1);
B2B_INSTANCE(DT_F16, 2, 128, 128, 128, 0, MODE_PERMLANE, false, 2, 8, KM_NAT, 1);
B2B_INSTANCE(DT_F16, 2, 128, 128, 128, 0, MODE_BPERM, false, 2, 8, KM_NAT, 1);
B2B_INSTANCE(DT_F16, 2, 128, 128, 128, 0, MODE_LDS, false, 2, 8, KM_NAT, 1);
B2B_INSTANCE(DT_F16, 2, 128, 128, 128, 0, MODE_BPERM, true, 2, 8, KM_NAT, 1);
B2B_INSTANCE(DT_F16, 2, 128, 128, 128, 0, MODE_LDS, true, 2, 8, KM_NAT, 1);
