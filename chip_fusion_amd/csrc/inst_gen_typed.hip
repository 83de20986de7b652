// Run-time-width instances on the 32x32x16 instruction with a 16-bit type per
// stage (bit s of the mask: GEMM s computes in bf16, else fp16; bit NST: D).
// Single GEMMs that change type (the unfused path) and two-GEMM cascades.
#include "registry.hpp"
// (stages, max width, A tiles ahead, type mask[, waves])
B2B_GEN_TYPED(1, 128, 1, 1);
B2B_GEN_TYPED(1, 128, 1, 2);
B2B_GEN_TYPED(1, 256, 0, 1);
B2B_GEN_TYPED(1, 256, 0, 2);
B2B_GEN_TYPED(1, 192, 1, 1);
B2B_GEN_TYPED(1, 192, 1, 2);
B2B_GEN_TYPED(2, 128, 1, 1);
B2B_GEN_TYPED(2, 128, 1, 2);
B2B_GEN_TYPED(2, 128, 1, 3);
B2B_GEN_TYPED(2, 128, 1, 4);
B2B_GEN_TYPED(2, 128, 1, 5);
B2B_GEN_TYPED(2, 128, 1, 6);
B2B_GEN_TYPED(2, 256, 0, 1);
B2B_GEN_TYPED(2, 256, 0, 2);
B2B_GEN_TYPED(2, 256, 0, 3);
B2B_GEN_TYPED(2, 256, 0, 4);
B2B_GEN_TYPED(2, 256, 0, 5);
B2B_GEN_TYPED(2, 256, 0, 6);
B2B_GEN_TYPED(2, 192, 1, 1);
B2B_GEN_TYPED(2, 192, 1, 2);
B2B_GEN_TYPED(2, 192, 1, 3);
B2B_GEN_TYPED(2, 192, 1, 4);
B2B_GEN_TYPED(2, 192, 1, 5);
B2B_GEN_TYPED(2, 192, 1, 6);
// four waves (128-row tiles): two workgroups a CU when the weights take at most 64 KB
B2B_GEN_TYPED(2, 128, 1, 1, 4);
B2B_GEN_TYPED(2, 128, 1, 2, 4);
B2B_GEN_TYPED(2, 128, 1, 3, 4);
B2B_GEN_TYPED(2, 128, 1, 4, 4);
B2B_GEN_TYPED(2, 128, 1, 5, 4);
B2B_GEN_TYPED(2, 128, 1, 6, 4);
