// Instances for widths that are not multiples of the instruction granule,
// and for leading dimensions and batch strides at any element alignment:
// every width padded on chip, partial rows loaded and stored element by
// element at the edges.  One type throughout, relabelled.
#include "registry.hpp"
using namespace b2bk;
// 16-bit on the 32x32x16 instruction: (dtype, stages, max width, mode, A tiles
// ahead, type mask, waves, fp8 D, tails)
B2B_GEN_INSTANCE(DT_F16, 1, 128, MODE_RELABEL, 1, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_F16, 1, 256, MODE_RELABEL, 0, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_F16, 2, 128, MODE_RELABEL, 1, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_F16, 2, 256, MODE_RELABEL, 0, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_F16, 3, 128, MODE_RELABEL, 1, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_F16, 3, 256, MODE_RELABEL, 0, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_BF16, 1, 128, MODE_RELABEL, 1, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_BF16, 1, 256, MODE_RELABEL, 0, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_BF16, 2, 128, MODE_RELABEL, 1, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_BF16, 2, 256, MODE_RELABEL, 0, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_BF16, 3, 128, MODE_RELABEL, 1, -1, 8, false, true);
B2B_GEN_INSTANCE(DT_BF16, 3, 256, MODE_RELABEL, 0, -1, 8, false, true);
// fp64 on the 16x16x4 instruction: (stages, max width, A tiles ahead, tiles per
// group, tails); two or three GEMMs up to 64 wide (at 128 the edge handling
// leaves too few registers: those instances would spill), one GEMM to 128
B2B_GEN64_INSTANCE(1, 64, 1, 4, true);
B2B_GEN64_INSTANCE(1, 128, 0, 2, true);
B2B_GEN64_INSTANCE(2, 64, 1, 4, true);
B2B_GEN64_INSTANCE(3, 64, 1, 4, true);
