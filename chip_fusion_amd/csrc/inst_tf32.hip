// tf32 instances: bf16 passes on the 32x32x16 instruction, run-time widths
// (multiples of 32 up to 128), one to three GEMMs; three passes, or four for
// exact tf32 products.  The widths 128, 128, 128 (two GEMMs) and 128, 128,
// 128, 64 (three) also have instances with the widths compiled in.
#include "registry.hpp"
// (stages, max width, passes[, waves per workgroup[, fixed widths]])
B2B_TF32_INSTANCE(1, 128, 3);
B2B_TF32_INSTANCE(2, 128, 3);
B2B_TF32_INSTANCE(3, 128, 3);
B2B_TF32_INSTANCE(1, 128, 4);
B2B_TF32_INSTANCE(2, 128, 4);
B2B_TF32_INSTANCE(3, 128, 4);
B2B_TF32_INSTANCE(2, 128, 3, 8, 128, 128, 128);
B2B_TF32_INSTANCE(3, 128, 3, 8, 128, 128, 128, 64);
B2B_TF32_INSTANCE(2, 128, 4, 8, 128, 128, 128);
B2B_TF32_INSTANCE(3, 128, 4, 8, 128, 128, 128, 64);
