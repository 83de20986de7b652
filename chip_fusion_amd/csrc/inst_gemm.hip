// Single-GEMM instances for the unfused comparison path (each writes its
// rounded result to memory; the next GEMM reads it back).
#include "registry.hpp"
using namespace b2bk;
B2B_INSTANCE(DT_F16, 1, 64, 64, 0, 0, 0, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 1, 128, 128, 0, 0, 0, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_F16, 1, 128, 64, 0, 0, 0, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_BF16, 1, 64, 64, 0, 0, 0, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_BF16, 1, 128, 128, 0, 0, 0, false, 2, 8, KM_NAT);
B2B_INSTANCE(DT_BF16, 1, 256, 256, 0, 0, 0, false, 1, 4, KM_NAT);
B2B_INSTANCE(DT_F64, 1, 64, 64, 0, 0, 0, false, 1, 8, KM_PAIR64);
B2B_INSTANCE(DT_F64, 1, 64, 64, 0, 0, 0, false, 1, 8, KM_NAT);
