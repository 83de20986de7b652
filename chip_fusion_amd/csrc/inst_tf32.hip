// tf32 instances: bf16 passes on the 32x32x16 instruction, run-time widths
// (multiples of 32 up to 128), one to three GEMMs; three passes, or four for
// exact tf32 products.
#include "registry.hpp"
// (stages, max width, passes[, waves per workgroup])
B2B_TF32_INSTANCE(1, 128, 3);
B2B_TF32_INSTANCE(2, 128, 3);
B2B_TF32_INSTANCE(3, 128, 3);
B2B_TF32_INSTANCE(1, 128, 4);
B2B_TF32_INSTANCE(2, 128, 4);
B2B_TF32_INSTANCE(3, 128, 4);
