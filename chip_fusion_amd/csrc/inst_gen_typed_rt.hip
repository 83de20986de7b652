// Cascades with a 16-bit type per stage read at run time (one instance for
// every mixture): three to eight GEMMs, relabelled; up to 256 wide for three
// to five GEMMs (with instances bounded at 192 that hold a prefetched A
// tile), 128 for more.  The two- and three-GEMM mixtures up to 128 wide, and
// the two-GEMM ones up to 256, have compiled masks (inst_gen_typed*.hip).
#include "registry.hpp"
using namespace b2bk;
// (first type (any), stages, max width, rearrangement, A tiles ahead, TM_RUNTIME)
B2B_GEN_INSTANCE(DT_F16, 3, 256, MODE_RELABEL, 0, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 3, 192, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 4, 192, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 5, 192, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 4, 128, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 4, 256, MODE_RELABEL, 0, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 5, 128, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 5, 256, MODE_RELABEL, 0, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 6, 128, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 7, 128, MODE_RELABEL, 1, TM_RUNTIME);
B2B_GEN_INSTANCE(DT_F16, 8, 128, MODE_RELABEL, 1, TM_RUNTIME);
