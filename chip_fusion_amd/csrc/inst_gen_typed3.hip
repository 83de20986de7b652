// Three-GEMM cascades with a 16-bit type per stage (bit s of the mask: GEMM s
// computes in bf16, else fp16; bit 3: D), relabelled, widths up to 128.
#include "registry.hpp"
// (stages, max width, A tiles ahead, type mask)
B2B_GEN_TYPED(3, 128, 1, 1);
B2B_GEN_TYPED(3, 128, 1, 2);
B2B_GEN_TYPED(3, 128, 1, 3);
B2B_GEN_TYPED(3, 128, 1, 4);
B2B_GEN_TYPED(3, 128, 1, 5);
B2B_GEN_TYPED(3, 128, 1, 6);
B2B_GEN_TYPED(3, 128, 1, 7);
B2B_GEN_TYPED(3, 128, 1, 8);
B2B_GEN_TYPED(3, 128, 1, 9);
B2B_GEN_TYPED(3, 128, 1, 10);
B2B_GEN_TYPED(3, 128, 1, 11);
B2B_GEN_TYPED(3, 128, 1, 12);
B2B_GEN_TYPED(3, 128, 1, 13);
B2B_GEN_TYPED(3, 128, 1, 14);
