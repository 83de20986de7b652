// Column-split instances: cascades whose two weight matrices exceed LDS.
#include "registry.hpp"
using namespace b2bk;
// (dtype, K, N1, N2)
B2B_CS_INSTANCE(DT_BF16, 256, 256, 256, 6);
B2B_CS_INSTANCE(DT_F16, 256, 256, 256, 6);
