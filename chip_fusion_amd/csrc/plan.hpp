// Host-side planning of the rearrangement between cascaded GEMMs.
//
// Page 1 ("数据处理方法、装置、设备及介质", detailed description) determines,
// per data type and hardware, the register layout of the first operator's
// result and of the second operator's input (the two "data-processing
// rules"), derives the element-by-element relation between them, and turns
// the relation into exchange rounds -- the coordination matrix of Fig. 4, in
// which each thread gives one element and takes one per round and no thread
// is asked twice in a round -- encoded per round as functions of the thread
// index.  This file holds the gfx950 matrix-instruction layouts and those
// three steps.
#pragma once
#include <cstdint>
#include <vector>

// Bounds and invariant checks of the planner, compiled in with -DB2B_DEBUG
// (the CPU sanitizer build turns them on): a failed check names the file,
// the line and the condition on stderr and aborts.  Without B2B_DEBUG they
// compile to nothing.
#ifdef B2B_DEBUG
#include <cstdio>
#include <cstdlib>
#define B2B_CHECK(cond)                                                                  \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            std::fprintf(stderr, "%s:%d: B2B_DEBUG check failed: %s\n", __FILE__, __LINE__, \
                         #cond);                                                         \
            std::abort();                                                                \
        }                                                                                \
    } while (0)
#else
#define B2B_CHECK(cond) ((void)0)
#endif

namespace b2b {

enum Shape : int {
    SH_F16_16x16x32 = 0,
    SH_BF16_16x16x32 = 1,
    SH_F16_32x32x16 = 2,
    SH_BF16_32x32x16 = 3,
    SH_F16_16x16x16 = 4,
    SH_F64_16x16x4 = 5,
    SH_COUNT = 6
};

constexpr int kLanes = 64;

// One matrix instruction: C[m x n] += A[m x k] . B[k x n] on a 64-lane wave.
struct MfmaShape {
    int m, n, k;
    int a_elems;   // operand elements per lane (A and B alike)
    int c_elems;   // accumulator elements per lane
    int bits;      // operand element width
};

const MfmaShape& shape_info(Shape s);
// (lane, element) -> (row, col) of the operand tiles and of the accumulator.
void a_coord(Shape s, int lane, int e, int* row, int* k);
void b_coord(Shape s, int lane, int e, int* k, int* col);
void c_coord(Shape s, int lane, int e, int* row, int* col);

// The relation of one remap unit (see b2b_remap_relation in b2b.h):
// src_of[d] is the source index (lane*E + tile*C + reg) feeding destination
// index d (lane*E + kstep*A + slot).
struct Relation {
    int elems = 0;        // E, elements per lane
    int tiles = 0;        // accumulator tiles in the unit
    int ksteps = 0;       // next-GEMM K-steps in the unit
    std::vector<int> src_of;
};

// orient_n = false: first GEMM computed transposed (lanes hold rows of C0).
bool build_relation(Shape s, bool orient_n, Relation* out);

// The relation between any two layouts of the same 64*elems elements, each
// given as a label per (lane, element) (index lane*elems + e): src_of[d] = the
// source index holding the label of destination index d.  False unless both
// hold the same labels, each once.
bool build_relation_from_labels(int elems, const int32_t* src, const int32_t* dst, Relation* out);

// Pairs of 16-bit elements moved as one 32-bit value; false when the relation
// splits a pair.
bool pack_relation(const Relation& r, Relation* packed);

// Exchange rounds. Index [round*64 + lane].
struct Schedule {
    int rounds = 0;
    std::vector<int> p, q, r;   // receiver view: sender lane, sender element, own slot
    std::vector<int> give;      // sender view: element lane gives in the round
};

// Per round, the lexicographically first perfect matching of receivers
// (ascending) to senders, each receiver taking its lowest open destination
// slot whose sender is free and keeps the rest of the round matchable.
bool build_schedule(const Relation& r, Schedule* out);

// Replays the rounds on labelled data; true if the result is the relation.
bool check_schedule(const Relation& r, const Schedule& s);

}  // namespace b2b
