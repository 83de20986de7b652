// Kernel instances: fp16, K = N1 = N2 = 64.
#include "registry.hpp"
using namespace b2bk;
// (dtype, stages, K, N1, N2, N3, remap, orientation N, 16-row sub-tiles per wave, waves, A K-map)
B2B_INSTANCE(DT_F16, 2, 64, 64, 64, 0, MODE_RELABEL, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 2, 64, 64, 64, 0, MODE_PERMLANE, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 2, 64, 64, 64, 0, MODE_BPERM, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 2, 64, 64, 64, 0, MODE_LDS, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 2, 64, 64, 64, 0, MODE_BPERM, true, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 2, 64, 64, 64, 0, MODE_LDS, true, 2, 8, KM_NAT);
