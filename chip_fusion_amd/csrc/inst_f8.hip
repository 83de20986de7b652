// Two-GEMM cascades with an fp8 (E4M3) second GEMM: (first GEMM's type, D's
// type, max width, A tiles ahead).  K a multiple of 32, N1 of 64, N2 of 32.
#include "registry.hpp"
using namespace b2bk;
B2B_F8_INSTANCE(DT_F16, DT_F16, 128, 1);
B2B_F8_INSTANCE(DT_F16, DT_F16, 256, 0);
B2B_F8_INSTANCE(DT_BF16, DT_BF16, 128, 1);
B2B_F8_INSTANCE(DT_BF16, DT_BF16, 256, 0);
B2B_F8_INSTANCE(DT_F16, DT_BF16, 128, 1);
B2B_F8_INSTANCE(DT_F16, DT_BF16, 256, 0);
B2B_F8_INSTANCE(DT_BF16, DT_F16, 128, 1);
B2B_F8_INSTANCE(DT_BF16, DT_F16, 256, 0);
// four waves (128-row tiles): two workgroups a CU when the weights and staging fit 80 KB
B2B_F8_INSTANCE(DT_F16, DT_F16, 128, 1, 4);
B2B_F8_INSTANCE(DT_BF16, DT_BF16, 128, 1, 4);
B2B_F8_INSTANCE(DT_F16, DT_BF16, 128, 1, 4);
B2B_F8_INSTANCE(DT_BF16, DT_F16, 128, 1, 4);
// the unfused comparison: a 16-bit GEMM whose result is written as fp8, then an
// fp8 GEMM (D's type, max width)
B2B_GEN_INSTANCE(DT_F16, 1, 128, MODE_RELABEL, 1, -1, 8, true);
B2B_GEN_INSTANCE(DT_F16, 1, 256, MODE_RELABEL, 0, -1, 8, true);
B2B_GEN_INSTANCE(DT_BF16, 1, 128, MODE_RELABEL, 1, -1, 8, true);
B2B_GEN_INSTANCE(DT_BF16, 1, 256, MODE_RELABEL, 0, -1, 8, true);
B2B_F8A_INSTANCE(DT_F16, 128);
B2B_F8A_INSTANCE(DT_F16, 256);
B2B_F8A_INSTANCE(DT_BF16, 128);
B2B_F8A_INSTANCE(DT_BF16, 256);
