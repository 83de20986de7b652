// C ABI of the fused cascaded GEMM: planning (create), execution (run).
//
// Page 1 ("数据处理方法、装置、设备及介质", the apparatus of Fig. 5) splits the
// method into an operator-determination module, a relation-determination
// module and a rearrangement module.  Here create() is the first two -- it
// validates the cascade, picks the kernel instance and derives the
// rearrangement relation and its coordination rounds on the host, once --
// and run() is the third: it only enqueues the fused kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "b2b.h"
#include "plan.hpp"
#include "registry.hpp"

namespace b2b {

std::vector<KernelDesc>& registry() {
    static std::vector<KernelDesc> r;
    return r;
}
std::vector<ProbeDesc>& probe_registry() {
    static std::vector<ProbeDesc> r;
    return r;
}
std::vector<MfmaProbeDesc>& mfma_probe_registry() {
    static std::vector<MfmaProbeDesc> r;
    return r;
}

}  // namespace b2b

using b2b::KernelDesc;

constexpr int kMaxSt = b2bk::kMaxStages;

struct b2b_gemm_plan {
    int dtype = 0, nst = 0, mode = 0, orn = 0;
    int tm = -1;                                 // type per stage (bit s: bf16), or -1: dtype throughout
    int passes = 0;                              // tf32: bf16 passes per product (3 or 4)
    int f8 = 0, dtd = 0;                         // second GEMM in fp8 E4M3, D's type
    int tail = 0;                                // fused on a kernel that takes any widths and leading dimensions
    int64_t batch = 0, M = 0, dims[kMaxSt + 1] = {};
    // leading dimensions and batch strides (elements): [0] A, [1 + s] B_s, [nst + 1] D
    int64_t ld[kMaxSt + 2] = {}, bs[kMaxSt + 2] = {};
    uint32_t flags = 0;
    bool unfused = false;
    bool chain = false;                          // made by b2b_chain_create
    const KernelDesc* fused = nullptr;           // fused path
    const KernelDesc* stage_k[kMaxSt] = {};      // unfused path
    void* work[kMaxSt - 1] = {};                 // unfused intermediates
    int64_t work_bytes[kMaxSt - 1] = {};
    uint16_t sched[2][b2bk::kMaxRounds][64];
    std::mutex grid_mu;
    int grid_dev = -1, grid[kMaxSt] = {};
};

namespace {

int elt_size(int dt) { return dt == B2B_DTYPE_F64 ? 8 : (dt == B2B_DTYPE_TF32 ? 4 : 2); }

b2b::Shape shape_of(int dt) {
    return dt == B2B_DTYPE_F64 ? b2b::SH_F64_16x16x4
                               : (dt == B2B_DTYPE_BF16 ? b2b::SH_BF16_16x16x32 : b2b::SH_F16_16x16x32);
}

const KernelDesc* find_kernel(int dt, int nst, const int64_t* dims, int mode, int orn, int km0) {
    for (const KernelDesc& d : b2b::registry()) {
        if (d.rtw || d.dtype != dt || d.nst != nst || d.orn != orn) continue;
        if (nst > 1 && d.mode != mode) continue;
        if (km0 >= 0 && d.km0 != km0) continue;
        bool ok = true;
        for (int i = 0; i <= nst; ++i) ok = ok && d.dims[i] == dims[i];
        if (ok) return &d;
    }
    return nullptr;
}

// Run-time-width kernel for widths dims[0..nst] (32x32x16 for fp16/bf16,
// 16x16x4 for fp64): the smallest width bound that holds them all, or null
// when a granule, a bound or LDS rules the cascade out.
// tail: an instance that takes any widths (each padded on chip to the
// granule: 32 for fp16/bf16, 8 for fp64's K and 16 for its N) and any
// leading dimensions; the bound and LDS then hold for the padded widths.
bool gen_fits(const KernelDesc& d, int dt, int nst, const int64_t* dims, int tm = -1, int passes = 0,
              int out8 = 0, int tail = 0) {
    if (!d.rtw || d.dtype != dt || d.nst != nst || d.tm != tm || d.passes != passes || d.out8 != out8 ||
        d.tail != tail)
        return false;
    // an instance with its widths compiled in takes exactly those
    if (d.dims[0])
        for (int i = 0; i <= nst; ++i)
            if (dims[i] != d.dims[i]) return false;
    const bool f64 = dt == B2B_DTYPE_F64;
    const int64_t gk = f64 ? 8 : 32, gn = f64 ? 16 : 32;
    int64_t w[kMaxSt + 1];
    for (int i = 0; i <= nst; ++i) {
        const int64_t g = i == 0 ? gk : gn;
        if (!tail && dims[i] % g) return false;
        w[i] = (dims[i] + g - 1) / g * g;
        if (w[i] > d.maxd) return false;
    }
    int64_t lds = 0;
    for (int i = 0; i < nst; ++i) lds += w[i] * w[i + 1] * elt_size(dt);
    return lds <= 160 * 1024;
}

// whether widths d[0..nst] are whole granules of the kernels without tails
// (fp16/bf16: multiples of 32; fp64: K of 8, N of 16)
bool whole_granules(int dt, int nst, const int64_t* d) {
    const bool f64 = dt == B2B_DTYPE_F64;
    if (d[0] % (f64 ? 8 : 32)) return false;
    for (int i = 1; i <= nst; ++i)
        if (d[i] % (f64 ? 16 : 32)) return false;
    return true;
}

// Rank among fitting instances of one width bound: four-wave instances
// first where two of their workgroups fit a CU's LDS, then eight-wave ones,
// then four-wave ones alone on a CU.
int wave_rank(const KernelDesc& d, const int64_t* dims, int nst) {
    int32_t d32[kMaxSt + 1] = {};
    for (int i = 0; i <= nst; ++i) d32[i] = (int32_t)dims[i];
    const bool pair = d.waves == 4 && d.dyn_lds && 2 * d.dyn_lds(d32) <= 160 * 1024;
    return d.waves == 4 ? (pair ? 0 : 2) : 1;
}

// One fp8 GEMM (K = dims[0] a multiple of 64, N = dims[1] of 32), D in dtd.
const KernelDesc* find_f8a(int dtd, const int64_t* dims) {
    const KernelDesc* best = nullptr;
    for (const KernelDesc& d : b2b::registry()) {
        if (d.f8 != 2 || d.dtd != dtd || dims[0] % 64 || dims[1] % 32) continue;
        if (dims[0] > d.maxd || dims[1] > d.maxd || dims[0] * dims[1] > 160 * 1024) continue;
        if (!best || d.maxd < best->maxd) best = &d;
    }
    return best;
}

// Whether fp8-second-GEMM instance d computes the cascade dims[0..2] of a
// first GEMM in dt with D in dtd: the granules, d's own width bound (the
// kernel walks at most maxd of K and of each N), and both weights in LDS.
bool f8_fits(const KernelDesc& d, int dt, int dtd, const int64_t* dims) {
    if (d.f8 != 1 || d.dtype != dt || d.dtd != dtd) return false;
    if (dims[0] % 32 || dims[1] % 64 || dims[2] % 32) return false;
    if (dims[0] > d.maxd || dims[1] > d.maxd || dims[2] > d.maxd) return false;
    return dims[0] * dims[1] * 2 + dims[1] * dims[2] <= 160 * 1024;
}

// Two GEMMs, the second in fp8: the fitting instance with the smallest
// width bound, ranked by waves among equal bounds.
const KernelDesc* find_f8(int dt, int dtd, const int64_t* dims) {
    const KernelDesc* best = nullptr;
    for (const KernelDesc& d : b2b::registry()) {
        if (!f8_fits(d, dt, dtd, dims)) continue;
        if (!best || d.maxd < best->maxd ||
            (d.maxd == best->maxd && wave_rank(d, dims, 2) < wave_rank(*best, dims, 2)))
            best = &d;
    }
    return best;
}

// A type per stage read at run time: the instance for nst GEMMs whose width
// bound holds dims (the smallest), whatever the mixture.
const KernelDesc* find_gen_rt(int nst, const int64_t* dims) {
    const KernelDesc* best = nullptr;
    for (const KernelDesc& d : b2b::registry()) {
        if (d.tm != b2bk::TM_RUNTIME || d.nst != nst) continue;
        if (!gen_fits(d, d.dtype, nst, dims, b2bk::TM_RUNTIME)) continue;
        if (!best || d.maxd < best->maxd) best = &d;
    }
    return best;
}

// Among the fitting instances the smallest width bound wins; of two with the
// same bound, one with the widths compiled in (tf32: 5-11 % faster than
// reading them at run time), then the four-wave one where two of its
// workgroups fit a CU's LDS (twice the tiles in flight per CU, measured 3 %
// faster), else the eight-wave one.
const KernelDesc* find_gen(int dt, int nst, const int64_t* dims, int mode, int tm = -1, int passes = 0,
                           int out8 = 0, int tail = 0) {
    const KernelDesc* best = nullptr;
    auto rank = [&](const KernelDesc& d) { return 4 * (d.dims[0] ? 0 : 1) + wave_rank(d, dims, nst); };
    for (const KernelDesc& d : b2b::registry()) {
        if (d.f8 || !gen_fits(d, dt, nst, dims, tm, passes, out8, tail) || (nst > 1 && d.mode != mode)) continue;
        if (!best || d.maxd < best->maxd || (d.maxd == best->maxd && rank(d) < rank(*best))) best = &d;
    }
    return best;
}

// Device allocation of an unfused plan's workspace.  B2B_FAULT_INJECT=alloc
// (or alloc:N) makes the first (or N-th) such allocation of a create call
// fail as if the device were out of memory: a test hook for the error path,
// which must leave no plan and no allocation behind.
hipError_t ws_alloc(void** p, size_t bytes, int* count) {
    ++*count;
    if (const char* fi = std::getenv("B2B_FAULT_INJECT")) {
        if (std::strncmp(fi, "alloc", 5) == 0) {
            const int n = fi[5] == ':' ? std::atoi(fi + 6) : 1;
            if (n == *count) {
                *p = nullptr;
                return hipErrorOutOfMemory;
            }
        }
    }
    return hipMalloc(p, bytes);
}

// Coordination rounds in the packed per-lane form the kernels read.
bool make_sched(int dt, bool orn, uint16_t (&tab)[b2bk::kMaxRounds][64]) {
    std::memset(tab, 0, sizeof tab);
    b2b::Relation rel, use;
    if (!b2b::build_relation(shape_of(dt), orn, &rel)) return false;
    if (dt != B2B_DTYPE_F64 && !orn) {
        if (!b2b::pack_relation(rel, &use)) return false;    // 16-bit pairs move together
    } else {
        use = rel;
    }
    b2b::Schedule s;
    if (!b2b::build_schedule(use, &s) || s.rounds > b2bk::kMaxRounds) return false;
    for (int j = 0; j < s.rounds; ++j)
        for (int l = 0; l < 64; ++l)
            tab[j][l] = (uint16_t)(s.p[j * 64 + l] | (s.give[j * 64 + l] << 6) | (s.r[j * 64 + l] << 9));
    return true;
}

int pick_mode(int dt, uint32_t flags) {
    int m = (int)((flags & B2B_REMAP_MASK) >> 4);
    if (m != 0) return m;
    (void)dt;
    return b2bk::MODE_RELABEL;
}

b2b_status_t grid_for(b2b_gemm_plan* p, int idx, const KernelDesc* k, int* grid) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return B2B_ERROR_HIP;
    std::lock_guard<std::mutex> lock(p->grid_mu);
    if (p->grid_dev != dev) {
        p->grid_dev = dev;
        for (int& g : p->grid) g = 0;
    }
    if (p->grid[idx] == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return B2B_ERROR_HIP;
        size_t shm = 0;
        if (k->dyn_lds) {
            const int64_t* w = idx == 0 && !p->unfused ? p->dims : p->dims + idx;
            int32_t d32[kMaxSt + 1] = {};
            for (int i = 0; i <= k->nst; ++i) d32[i] = (int32_t)w[i];
            shm = (size_t)k->dyn_lds(d32);
        }
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k->fn, k->threads, shm) != hipSuccess)
            return B2B_ERROR_HIP;
        if (per < 1) per = 1;
        p->grid[idx] = cus * per;
    }
    *grid = p->grid[idx];
    return B2B_SUCCESS;
}

b2b_status_t launch_one(b2b_gemm_plan* p, int idx, const KernelDesc* k, const void* A, int64_t lda,
                        int64_t sA, const void* const* B, const int64_t* ldb, const int64_t* sB,
                        void* D, int64_t ldd, int64_t sD, hipStream_t stream) {
    b2bk::KArgs a;
    std::memset(&a, 0, sizeof a);
    // widths of this launch's GEMMs: the whole cascade, or stage idx alone
    const int64_t* w = idx == 0 && !p->unfused ? p->dims : p->dims + idx;
    for (int i = 0; i <= k->nst; ++i) a.dims[i] = (int32_t)w[i];
    a.tmask = p->tm;
    a.A = A;
    a.D = D;
    a.M = p->M;
    a.lda = lda;
    a.ldd = ldd;
    a.sA = sA;
    a.sD = sD;
    for (int s = 0; s < k->nst; ++s) {
        a.B[s] = B[s];
        a.ldb[s] = ldb[s];
        a.sB[s] = sB[s];
    }
    const int64_t tpb = (p->M + k->rows_wg - 1) / k->rows_wg;
    a.tiles_per_batch = (int32_t)tpb;
    a.total_tiles = (int32_t)(tpb * p->batch);
    std::memcpy(a.sched, p->sched, sizeof a.sched);
    int grid = 0;
    b2b_status_t st = grid_for(p, idx, k, &grid);
    if (st != B2B_SUCCESS) return st;
    if (grid > a.total_tiles) grid = a.total_tiles;
    if (grid < 1) grid = 1;
    return k->launch(a, grid, stream) == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
}

}  // namespace

extern "C" {

const char* b2b_status_string(b2b_status_t s) {
    switch (s) {
        case B2B_SUCCESS: return "success";
        case B2B_ERROR_INVALID_VALUE: return "invalid value";
        case B2B_ERROR_NOT_SUPPORTED: return "not supported";
        case B2B_ERROR_HIP: return "HIP runtime error";
        case B2B_ERROR_OUT_OF_MEMORY: return "out of memory";
        case B2B_ERROR_WORKSPACE_LIMIT: return "intermediates exceed the static workspace";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// Validates and plans a cascade of nst GEMMs with widths d[0..nst]; L and S hold
// nst + 2 leading dimensions and batch strides ([0] A, [1 + s] B_s, [nst + 1] D)
// or are null (dense).
// tm >= 0: a 16-bit type per stage (bit s set: GEMM s in bf16; bit nst: D), dt
// the type of bit 0; the cascade then runs on the 32x32x16 kernels.
// f8_dtd >= 0: two GEMMs, the second in fp8 E4M3 (B1 one byte per element),
// D in type f8_dtd.
// plan_fill validates and plans into *p (a fresh plan the caller owns): it
// picks the kernels and, for the unfused path, sizes the workspace
// (p->work_bytes) without allocating anything, on the host or the device.
b2b_status_t plan_fill(b2b_gemm_plan* p, int dt, int64_t batch, int64_t M, int nst, const int64_t* d,
                       const int64_t* Lin, const int64_t* Sin, uint32_t flags, bool chain, int tm, int f8_dtd) {
    if (dt != B2B_DTYPE_F16 && dt != B2B_DTYPE_BF16 && dt != B2B_DTYPE_F64 && dt != B2B_DTYPE_TF32)
        return B2B_ERROR_NOT_SUPPORTED;
    if (nst < 1 || nst > kMaxSt || !d) return B2B_ERROR_INVALID_VALUE;
    if (batch < 1 || M < 1) return B2B_ERROR_INVALID_VALUE;
    for (int i = 0; i <= nst; ++i)
        if (d[i] < 1 || d[i] > (int64_t)1 << 24) return B2B_ERROR_INVALID_VALUE;
    if (batch > (int64_t)1 << 30 || M > (int64_t)1 << 31) return B2B_ERROR_INVALID_VALUE;
    const uint32_t known =
        B2B_FLAG_UNFUSED | B2B_FLAG_ORIENT_N | B2B_FLAG_MFMA_32X32 | B2B_FLAG_TF32_EXACT | B2B_REMAP_MASK;
    if (flags & ~known) return B2B_ERROR_INVALID_VALUE;
    const bool tf32 = dt == B2B_DTYPE_TF32;
    if ((flags & B2B_FLAG_TF32_EXACT) && !tf32) return B2B_ERROR_INVALID_VALUE;
    const int passes = tf32 ? ((flags & B2B_FLAG_TF32_EXACT) ? 4 : 3) : 0;
    const int mode = pick_mode(dt, flags);
    if (mode > b2bk::MODE_RELABEL) return B2B_ERROR_INVALID_VALUE;
    const int orn = (flags & B2B_FLAG_ORIENT_N) ? 1 : 0;
    if (orn && mode != b2bk::MODE_BPERM && mode != b2bk::MODE_LDS) return B2B_ERROR_INVALID_VALUE;
    const bool typed = tm >= 0, f8 = f8_dtd >= 0;
    // typed, tf32 and fp8 cascades are relabelled on the 32x32x16 kernels
    if ((typed || tf32 || f8) && (orn || mode != b2bk::MODE_RELABEL)) return B2B_ERROR_NOT_SUPPORTED;
    if (f8 && nst != 2) return B2B_ERROR_NOT_SUPPORTED;
    const bool s32 = (flags & B2B_FLAG_MFMA_32X32) != 0 || typed || tf32;
    if (s32 && (orn || dt == B2B_DTYPE_F64)) return B2B_ERROR_NOT_SUPPORTED;
    // the 32x32x16 kernels rearrange by relabelling or by lane-half swaps
    const int mode32 = (flags & B2B_REMAP_MASK) == B2B_REMAP_AUTO ? b2bk::MODE_RELABEL : mode;

    int64_t dims[kMaxSt + 1] = {};
    for (int i = 0; i <= nst; ++i) dims[i] = d[i];
    const int n = nst + 2;
    int64_t L[kMaxSt + 2], S[kMaxSt + 2];
    const int es = elt_size(dt);
    bool ld16 = true;
    for (int i = 0; i < n; ++i) {
        // operand i: A (rows M, width K), B_s (rows d[s], width d[s+1]), D (rows M, width d[nst])
        const int64_t rows = (i == 0 || i == n - 1) ? M : dims[i - 1];
        const int64_t width = i == 0 ? dims[0] : (i == n - 1 ? dims[nst] : dims[i]);
        const int eo = (f8 && i == 2) ? 1 : es;    // the fp8 weights: one byte an element
        L[i] = Lin ? Lin[i] : width;
        if (L[i] < width) return B2B_ERROR_INVALID_VALUE;
        S[i] = Sin ? Sin[i] : rows * L[i];
        if (S[i] < 0) return B2B_ERROR_INVALID_VALUE;
        // rows and batches starting on 16-byte boundaries (else only the tail kernels)
        if ((L[i] * eo) % 16 || (S[i] * eo) % 16) ld16 = false;
        // the kernels address a wave's rows of A or D (at most 32) and a whole
        // weight matrix through one buffer resource, with 32-bit signed offsets
        const int64_t span_rows = (i == 0 || i == n - 1) ? std::min<int64_t>(M, 32) : rows;
        if (span_rows * L[i] * eo > (int64_t)INT32_MAX) return B2B_ERROR_INVALID_VALUE;
    }
    if (batch > 1 && (S[0] == 0 || S[n - 1] < M * L[n - 1])) return B2B_ERROR_INVALID_VALUE;
    // Widths off the granule, or rows / batches not on 16-byte boundaries:
    // the tail kernels (one type, fp16 / bf16 / fp64, relabelled).
    const bool tail = !(ld16 && whole_granules(dt, nst, dims));
    const bool tail_ok = (dt == B2B_DTYPE_F16 || dt == B2B_DTYPE_BF16 || dt == B2B_DTYPE_F64) && !typed && !f8 &&
                         !orn && mode == b2bk::MODE_RELABEL;
    if (tail && !tail_ok) return ld16 ? B2B_ERROR_NOT_SUPPORTED : B2B_ERROR_INVALID_VALUE;

    p->dtype = dt;
    p->tm = tm;
    p->passes = passes;
    p->f8 = f8 ? 1 : 0;
    p->dtd = f8 ? f8_dtd : dt;
    p->nst = nst;
    p->mode = mode;
    p->orn = orn;
    p->batch = batch;
    p->M = M;
    p->chain = chain;
    for (int i = 0; i <= nst; ++i) p->dims[i] = dims[i];
    for (int i = 0; i < n; ++i) { p->ld[i] = L[i]; p->bs[i] = S[i]; }
    p->flags = flags;
    p->unfused = (flags & B2B_FLAG_UNFUSED) != 0;
    std::memset(p->sched, 0, sizeof p->sched);

    if (!p->unfused && tail) {
        p->fused = find_gen(dt, nst, dims, b2bk::MODE_RELABEL, -1, 0, 0, 1);
        p->mode = b2bk::MODE_RELABEL;
        p->tail = 1;
        if (!p->fused) return B2B_ERROR_NOT_SUPPORTED;
    } else if (!p->unfused && f8) {
        p->fused = find_f8(dt, f8_dtd, dims);
        p->mode = b2bk::MODE_RELABEL;
        if (!p->fused) return B2B_ERROR_NOT_SUPPORTED;
    } else if (!p->unfused) {
        if (s32 || nst > 3) {
            // the fixed-width kernels cover up to three GEMMs
            if (orn) return B2B_ERROR_NOT_SUPPORTED;
            p->fused = find_gen(dt, nst, dims, mode32, tm, passes);
            // a mixture without a compiled mask: the types read at run time
            if (!p->fused && typed) p->fused = find_gen_rt(nst, dims);
            p->mode = mode32;
        } else if ((flags & B2B_REMAP_MASK) == B2B_REMAP_AUTO) {
            // the cheapest rearrangement compiled for this shape
            static const int order[] = {b2bk::MODE_RELABEL, b2bk::MODE_PERMLANE, b2bk::MODE_LDS,
                                        b2bk::MODE_BPERM};
            for (int m : order) {
                p->fused = find_kernel(dt, nst, dims, m, orn, -1);
                if (p->fused) { p->mode = m; break; }
            }
        } else {
            p->fused = find_kernel(dt, nst, dims, mode, orn, -1);
        }
        // widths no fixed-width kernel covers: the run-time-width kernels
        if (!p->fused && !s32 && !orn) {
            p->fused = find_gen(dt, nst, dims, mode32);
            p->mode = mode32;
        }
        if (!p->fused) return B2B_ERROR_NOT_SUPPORTED;
        if (p->mode == b2bk::MODE_BPERM) {
            if (!make_sched(dt, orn != 0, p->sched[0]) || !make_sched(dt, false, p->sched[1]))
                return B2B_ERROR_NOT_SUPPORTED;
        }
    } else if (f8) {
        // unfused: the first GEMM writes its result as fp8, the second reads it
        const int64_t d0[4] = {dims[0], dims[1], 0, 0}, d1[4] = {dims[1], dims[2], 0, 0};
        p->stage_k[0] = dims[1] % 64 ? nullptr : find_gen(dt, 1, d0, 0, -1, 0, 1);
        p->stage_k[1] = find_f8a(f8_dtd, d1);
        if (!p->stage_k[0] || !p->stage_k[1]) return B2B_ERROR_NOT_SUPPORTED;
        p->work_bytes[0] = batch * M * dims[1];      // one byte an element
    } else {
        if (orn) return B2B_ERROR_INVALID_VALUE;
        for (int s = 0; s < nst; ++s) {
            const int64_t d2[4] = {dims[s], dims[s + 1], 0, 0};
            const int km0 = (s == 0 && dt == B2B_DTYPE_F64) ? b2bk::KM_PAIR64 : b2bk::KM_NAT;
            // stage s alone: its own type in, the next stage's type out
            const int sub = typed ? (tm >> s) & 3 : 0;
            const int sdt = typed ? ((sub & 1) ? B2B_DTYPE_BF16 : B2B_DTYPE_F16) : dt;
            const int stm = (sub == 1 || sub == 2) ? sub : -1;
            // this GEMM's operands: A or the previous intermediate (dense), B_s,
            // and D or its own intermediate (dense)
            const bool last = s + 1 == nst;
            const int64_t lx = s == 0 ? L[0] : dims[s], sx = s == 0 ? S[0] : M * dims[s];
            const int64_t ly = last ? L[n - 1] : dims[s + 1], sy = last ? S[n - 1] : M * dims[s + 1];
            const bool al16 = (lx * es) % 16 == 0 && (sx * es) % 16 == 0 && (L[1 + s] * es) % 16 == 0 &&
                              (S[1 + s] * es) % 16 == 0 && (ly * es) % 16 == 0 && (sy * es) % 16 == 0;
            if (!al16 || !whole_granules(sdt, 1, d2)) {
                if (!tail_ok) return B2B_ERROR_NOT_SUPPORTED;
                p->stage_k[s] = find_gen(sdt, 1, d2, 0, -1, 0, 0, 1);
                if (!p->stage_k[s]) return B2B_ERROR_NOT_SUPPORTED;
                continue;
            }
            p->stage_k[s] = (s32 || stm >= 0) ? nullptr : find_kernel(sdt, 1, d2, 0, 0, km0);
            if (!p->stage_k[s]) p->stage_k[s] = find_gen(sdt, 1, d2, 0, stm, passes);
            if (!p->stage_k[s]) return B2B_ERROR_NOT_SUPPORTED;
        }
        for (int s = 0; s + 1 < nst; ++s) p->work_bytes[s] = batch * M * dims[s + 1] * es;
    }
    // the kernels count tiles (rows_wg rows of one batch) in 32 bits
    auto tiles_fit = [&](const KernelDesc* k) {
        return !k || ((M + k->rows_wg - 1) / k->rows_wg) * batch <= (int64_t)INT32_MAX;
    };
    bool fit = tiles_fit(p->fused);
    for (const KernelDesc* k : p->stage_k) fit = fit && tiles_fit(k);
    return fit ? B2B_SUCCESS : B2B_ERROR_INVALID_VALUE;
}

// A new plan (plan_fill) with its unfused workspace allocated.
b2b_status_t create_impl(b2b_gemm_t* plan, int dt, int64_t batch, int64_t M, int nst, const int64_t* d,
                         const int64_t* Lin, const int64_t* Sin, uint32_t flags, bool chain, int tm = -1,
                         int f8_dtd = -1) {
    if (!plan) return B2B_ERROR_INVALID_VALUE;
    *plan = nullptr;
    b2b_gemm_plan* p = new (std::nothrow) b2b_gemm_plan();
    if (!p) return B2B_ERROR_OUT_OF_MEMORY;
    const b2b_status_t st = plan_fill(p, dt, batch, M, nst, d, Lin, Sin, flags, chain, tm, f8_dtd);
    if (st != B2B_SUCCESS) {
        delete p;
        return st;
    }
    int allocs = 0;   // workspace allocations of this call
    for (int s = 0; s + 1 < kMaxSt; ++s) {
        if (!p->work_bytes[s]) continue;
        if (ws_alloc(&p->work[s], (size_t)p->work_bytes[s], &allocs) != hipSuccess) {
            (void)hipGetLastError();
            p->work[s] = nullptr;
            for (void* w : p->work)
                if (w) (void)hipFree(w);
            delete p;
            return B2B_ERROR_OUT_OF_MEMORY;
        }
    }
    *plan = p;
    // B2B_LOG=1: the chosen plan on stderr (the grid is settled at the first run)
    if (const char* lg = std::getenv("B2B_LOG")) {
        if (lg[0] && std::strcmp(lg, "0") != 0) {
            char buf[512];
            if (b2b_gemm_get_info(p, buf, sizeof buf) == B2B_SUCCESS) std::fprintf(stderr, "[b2b] plan: %s\n", buf);
        }
    }
    return B2B_SUCCESS;
}

// Enqueues the cascade; B holds the plan's nst weight pointers.
b2b_status_t run_impl(b2b_gemm_t p, const void* A, const void* const* B, void* D, hipStream_t stream) {
    if (!A || !D || (uintptr_t)A % 16 || (uintptr_t)D % 16 || A == (const void*)D) return B2B_ERROR_INVALID_VALUE;
    for (int s = 0; s < p->nst; ++s)
        if (!B[s] || (uintptr_t)B[s] % 16 || B[s] == (const void*)D) return B2B_ERROR_INVALID_VALUE;
    hipStream_t st = stream;
    const int nd = p->nst + 1;    // index of D's leading dimension and stride
    if (!p->unfused)
        return launch_one(p, 0, p->fused, A, p->ld[0], p->bs[0], B, p->ld + 1, p->bs + 1, D, p->ld[nd],
                          p->bs[nd], st);
    const void* x = A;
    int64_t ldx = p->ld[0], sx = p->bs[0];
    for (int s = 0; s < p->nst; ++s) {
        const bool last = s + 1 == p->nst;
        void* y = last ? D : p->work[s];
        const int64_t ldy = last ? p->ld[nd] : p->dims[s + 1];
        const int64_t sy = last ? p->bs[nd] : p->M * p->dims[s + 1];
        const void* Bst[1] = {B[s]};
        b2b_status_t r = launch_one(p, s, p->stage_k[s], x, ldx, sx, Bst, p->ld + 1 + s, p->bs + 1 + s, y, ldy,
                                    sy, st);
        if (r != B2B_SUCCESS) return r;
        x = y;
        ldx = ldy;
        sx = sy;
    }
    return B2B_SUCCESS;
}

}  // namespace

extern "C" {

b2b_status_t b2b_gemm_create(b2b_gemm_t* plan, b2b_dtype_t dtype, int64_t batch, int64_t M,
                             int64_t K, int64_t N1, int64_t N2, int64_t N3, const int64_t* ld,
                             const int64_t* batch_stride, uint32_t flags) {
    if (plan) *plan = nullptr;
    if (N3 < 0) return B2B_ERROR_INVALID_VALUE;
    const int nst = N3 > 0 ? 3 : 2;
    const int64_t d[4] = {K, N1, N2, N3};
    // {lda, ldb0, ldb1, ldb2, ldd} -> one entry per operand (ldb2 only with three GEMMs)
    int64_t L[5], S[5];
    if (ld || batch_stride) {
        for (int i = 0, j = 0; i < 5; ++i) {
            if (i == 3 && nst == 2) continue;
            L[j] = ld ? ld[i] : 0;
            S[j] = batch_stride ? batch_stride[i] : 0;
            ++j;
        }
    }
    // missing arrays stay dense: fill the dense values create_impl would use
    if (ld || batch_stride) {
        const int64_t rows[5] = {M, K, N1, N2, M};
        const int64_t width[5] = {K, N1, N2, N3, nst == 3 ? N3 : N2};
        for (int i = 0, j = 0; i < 5; ++i) {
            if (i == 3 && nst == 2) continue;
            if (!ld) L[j] = width[i];
            if (!batch_stride) S[j] = rows[i] * L[j];
            ++j;
        }
    }
    return create_impl(plan, (int)dtype, batch, M, nst, d, (ld || batch_stride) ? L : nullptr,
                       (ld || batch_stride) ? S : nullptr, flags, false);
}

b2b_status_t b2b_chain_create(b2b_gemm_t* plan, b2b_dtype_t dtype, int64_t batch, int64_t M, int32_t nst,
                              const int64_t* widths, const int64_t* ld, const int64_t* batch_stride,
                              uint32_t flags) {
    if (plan) *plan = nullptr;
    if (!widths) return B2B_ERROR_INVALID_VALUE;
    return create_impl(plan, (int)dtype, batch, M, nst, widths, ld, batch_stride, flags, true);
}

b2b_status_t b2b_chain_create_typed(b2b_gemm_t* plan, const b2b_dtype_t* dtypes, int64_t batch, int64_t M,
                                    int32_t nst, const int64_t* widths, const int64_t* ld,
                                    const int64_t* batch_stride, uint32_t flags) {
    if (plan) *plan = nullptr;
    if (!widths || !dtypes || nst < 1 || nst > kMaxSt) return B2B_ERROR_INVALID_VALUE;
    // an fp8 second GEMM between 16-bit types
    bool any_f8 = false;
    for (int s = 0; s <= nst; ++s) any_f8 = any_f8 || dtypes[s] == B2B_DTYPE_FP8_E4M3;
    if (any_f8) {
        auto b16 = [](b2b_dtype_t t) { return t == B2B_DTYPE_F16 || t == B2B_DTYPE_BF16; };
        if (nst != 2 || dtypes[1] != B2B_DTYPE_FP8_E4M3 || !b16(dtypes[0]) || !b16(dtypes[2]))
            return B2B_ERROR_NOT_SUPPORTED;
        return create_impl(plan, (int)dtypes[0], batch, M, nst, widths, ld, batch_stride, flags, true, -1,
                           (int)dtypes[2]);
    }
    bool same = true;
    int tm = 0;
    for (int s = 0; s <= nst; ++s) {
        if (dtypes[s] != B2B_DTYPE_F16 && dtypes[s] != B2B_DTYPE_BF16 && dtypes[s] != B2B_DTYPE_F64 &&
            dtypes[s] != B2B_DTYPE_TF32)
            return B2B_ERROR_NOT_SUPPORTED;
        same = same && dtypes[s] == dtypes[0];
        if (dtypes[s] == B2B_DTYPE_BF16) tm |= 1 << s;
    }
    // one type throughout: exactly the plan of b2b_chain_create
    if (same) return create_impl(plan, (int)dtypes[0], batch, M, nst, widths, ld, batch_stride, flags, true);
    for (int s = 0; s <= nst; ++s)
        if (dtypes[s] == B2B_DTYPE_F64 || dtypes[s] == B2B_DTYPE_TF32) return B2B_ERROR_NOT_SUPPORTED;
    return create_impl(plan, (int)dtypes[0], batch, M, nst, widths, ld, batch_stride, flags, true, tm);
}

b2b_status_t b2b_gemm_run(b2b_gemm_t p, const void* A, const void* B0, const void* B1,
                          const void* B2, void* D, hipStream_t stream) {
    if (!p || p->nst < 2 || p->nst > 3) return B2B_ERROR_INVALID_VALUE;
    if ((p->nst == 3) != (B2 != nullptr)) return B2B_ERROR_INVALID_VALUE;
    const void* Bs[3] = {B0, B1, B2};
    return run_impl(p, A, Bs, D, stream);
}

b2b_status_t b2b_chain_run(b2b_gemm_t p, const void* A, const void* const* B, void* D, hipStream_t stream) {
    if (!p || !B) return B2B_ERROR_INVALID_VALUE;
    return run_impl(p, A, B, D, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The unfused path without allocation (b2b_chain_run_static): the
// intermediates go to `scratch`, a file-scope device array of
// B2B_STATIC_WORKSPACE_BYTES that each GPU holds from the first call on it
// until the process ends.  Host code never uses the array's name as an
// address: its device address is asked for once per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[B2B_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch`
b2b_status_t scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return B2B_ERROR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return B2B_ERROR_NOT_SUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return B2B_ERROR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return B2B_SUCCESS;
}

}  // namespace

extern "C" {

b2b_status_t b2b_chain_run_static(b2b_dtype_t dtype, int64_t batch, int64_t M, int32_t nst, const int64_t* widths,
                                  const int64_t* ld, const int64_t* batch_stride, const void* A,
                                  const void* const* B, void* D, hipStream_t stream) {
    if (!widths || !B) return B2B_ERROR_INVALID_VALUE;
    // the plan lives on the stack: neither device nor host memory is allocated
    b2b_gemm_plan plan;
    b2b_status_t st = plan_fill(&plan, (int)dtype, batch, M, nst, widths, ld, batch_stride, B2B_FLAG_UNFUSED, true,
                                -1, -1);
    if (st != B2B_SUCCESS) return st;
    // intermediate s in half s % 2 (stage s reads half (s - 1) % 2 and writes
    // half s % 2; the stream orders the stages); one intermediate takes the
    // whole array
    int64_t half = 0;
    for (int64_t w : plan.work_bytes) half = std::max(half, (w + 255) / 256 * 256);
    const int64_t need = nst > 2 ? 2 * half : half;
    if (need > (int64_t)B2B_STATIC_WORKSPACE_BYTES) return B2B_ERROR_WORKSPACE_LIMIT;
    void* base = nullptr;
    if (half) {
        st = scratch_address(&base);
        if (st != B2B_SUCCESS) return st;
    }
    for (int s = 0; s + 1 < nst; ++s) plan.work[s] = (char*)base + (s % 2) * half;
    st = run_impl(&plan, A, B, D, stream);
    for (void*& w : plan.work) w = nullptr;   // the array is not the plan's
    return st;
}

b2b_status_t b2b_gemm_destroy(b2b_gemm_t p) {
    if (!p) return B2B_SUCCESS;
    b2b_status_t st = B2B_SUCCESS;
    bool any = false;
    for (void* w : p->work) any = any || w;
    if (any) {
        if (hipDeviceSynchronize() != hipSuccess) st = B2B_ERROR_HIP;
        for (void* w : p->work)
            if (w && hipFree(w) != hipSuccess) st = B2B_ERROR_HIP;
    }
    delete p;
    return st;
}

b2b_status_t b2b_gemm_tune(b2b_gemm_t p, int32_t nsets, const void* const* A, const void* const* B,
                           void* const* D, hipStream_t stream, int32_t reps) {
    if (!p || nsets < 1 || !A || !B || !D || reps < 1 || reps > 10000) return B2B_ERROR_INVALID_VALUE;
    if (p->unfused) return B2B_ERROR_NOT_SUPPORTED;
    const bool any_mode = (p->flags & B2B_REMAP_MASK) == B2B_REMAP_AUTO;
    const bool s32 = (p->flags & B2B_FLAG_MFMA_32X32) != 0;
    // every compiled kernel that computes this cascade under the plan's flags
    std::vector<const KernelDesc*> cands;
    for (const KernelDesc& d : b2b::registry()) {
        const bool rt = p->tm >= 0 && d.tm == b2bk::TM_RUNTIME;   // run-time types serve any mixture
        if ((!rt && (d.dtype != p->dtype || d.tm != p->tm)) || d.nst != p->nst || d.f8 != p->f8) continue;
        if (p->f8) {
            // only instances whose own bounds hold the plan's widths
            if (f8_fits(d, p->dtype, p->dtd, p->dims)) cands.push_back(&d);
            continue;
        }
        if (d.rtw) {
            if (p->orn || !gen_fits(d, d.dtype, p->nst, p->dims, d.tm, p->passes, 0, p->tail)) continue;
        } else {
            if (s32 || d.orn != p->orn || p->tail) continue;
            bool ok = true;
            for (int i = 0; i <= p->nst; ++i) ok = ok && d.dims[i] == p->dims[i];
            if (!ok) continue;
        }
        if (s32 && !d.shape32) continue;
        const int m = p->nst > 1 ? d.mode : p->mode;
        if (!any_mode && p->nst > 1 && m != p->mode) continue;
        cands.push_back(&d);
    }
    if (cands.empty()) return B2B_ERROR_NOT_SUPPORTED;
    hipStream_t st = stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return B2B_ERROR_HIP;
    }
    const KernelDesc* keep = p->fused;
    const int keep_mode = p->mode;
    auto run_set = [&](int i) { return run_impl(p, A[i], B + (size_t)i * p->nst, D[i], stream); };
    // candidates run interleaved over three rounds; in each, one untimed run,
    // then reps runs back to back over the buffer sets in turn (sets larger
    // than the 256 MB Infinity Cache make them cold, as a stream of distinct
    // batches is); the score is the median round
    const int rounds = 3;
    std::vector<float> times(cands.size() * rounds, 0.f);
    std::vector<char> usable(cands.size(), 1);
    b2b_status_t rc = B2B_SUCCESS;
    for (int r = 0; r < rounds && rc == B2B_SUCCESS; ++r)
        for (size_t i = 0; i < cands.size() && rc == B2B_SUCCESS; ++i) {
            if (!usable[i]) continue;
            const KernelDesc* k = cands[i];
            const int mode = p->nst > 1 ? k->mode : keep_mode;
            if (mode == b2bk::MODE_BPERM &&
                (!make_sched(p->dtype, p->orn != 0, p->sched[0]) || !make_sched(p->dtype, false, p->sched[1]))) {
                usable[i] = 0;
                continue;
            }
            p->fused = k;
            p->mode = mode;
            {
                std::lock_guard<std::mutex> lock(p->grid_mu);
                p->grid[0] = 0;   // this kernel's own grid
            }
            rc = run_set(nsets - 1);   // untimed; validates the arguments
            float ms = 0.f;
            if (rc == B2B_SUCCESS) {
                if (hipEventRecord(e0, st) != hipSuccess) rc = B2B_ERROR_HIP;
                for (int q = 0; q < reps && rc == B2B_SUCCESS; ++q) rc = run_set(q % nsets);
                if (rc == B2B_SUCCESS &&
                    (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                     hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
                    rc = B2B_ERROR_HIP;
            }
            times[i * rounds + r] = ms;
        }
    const KernelDesc* best = nullptr;
    int best_mode = 0;
    float best_ms = 0.f, keep_ms = -1.f;
    for (size_t i = 0; i < cands.size() && rc == B2B_SUCCESS; ++i) {
        if (!usable[i]) continue;
        float* t = &times[i * rounds];
        std::sort(t, t + rounds);
        const float ms = t[rounds / 2];
        const int mode = p->nst > 1 ? cands[i]->mode : keep_mode;
        if (cands[i] == keep && mode == keep_mode) keep_ms = ms;
        if (!best || ms < best_ms) {
            best = cands[i];
            best_mode = mode;
            best_ms = ms;
        }
    }
    // the planned kernel stays unless another is clearly (3 %) faster
    if (best && keep_ms >= 0.f && best_ms > 0.97f * keep_ms) {
        best = keep;
        best_mode = keep_mode;
    }
    if (!best) rc = B2B_ERROR_NOT_SUPPORTED;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    p->fused = rc == B2B_SUCCESS ? best : keep;
    p->mode = rc == B2B_SUCCESS ? best_mode : keep_mode;
    if (p->mode == b2bk::MODE_BPERM &&
        (!make_sched(p->dtype, p->orn != 0, p->sched[0]) || !make_sched(p->dtype, false, p->sched[1])))
        return B2B_ERROR_NOT_SUPPORTED;
    {
        std::lock_guard<std::mutex> lock(p->grid_mu);
        p->grid[0] = 0;
    }
    if (rc != B2B_SUCCESS) return rc;
    // leave every D as the kept kernel computes it
    for (int i = 0; i < nsets && rc == B2B_SUCCESS; ++i) rc = run_set(i);
    if (rc == B2B_SUCCESS && hipStreamSynchronize(st) != hipSuccess) rc = B2B_ERROR_HIP;
    return rc;
}

b2b_status_t b2b_gemm_get_info(b2b_gemm_t p, char* buf, size_t len) {
    if (!p || !buf || len == 0) return B2B_ERROR_INVALID_VALUE;
    static const char* dts[] = {"f16", "bf16", "f64", "tf32"};
    static const char* modes[] = {"none", "bpermute", "permlane", "lds", "relabel"};
    const KernelDesc* k = p->unfused ? p->stage_k[0] : p->fused;
    int64_t work = 0;
    for (int64_t w : p->work_bytes) work += w;
    const char* mfma = p->f8                        ? "32x32x16+f8_32x32x64"
                       : p->dtype == B2B_DTYPE_F64  ? "f64_16x16x4"
                       : p->dtype == B2B_DTYPE_TF32 ? (p->passes == 4 ? "bf16x4_32x32x16" : "bf16x3_32x32x16")
                       : k->shape32                 ? "32x32x16"
                                                    : "16x16x32";
    int lds_bytes = k->lds_bytes;
    if (k->dyn_lds) {
        int32_t d32[kMaxSt + 1] = {};
        for (int i = 0; i <= k->nst; ++i) d32[i] = (int32_t)p->dims[i];
        lds_bytes = (int)k->dyn_lds(d32);
    }
    std::string dts_s = dts[p->dtype];
    if (p->f8) dts_s = std::string(dts[p->dtype]) + "/fp8/" + dts[p->dtd];
    if (p->tm >= 0) {
        // a type per stage: GEMM 0's, GEMM 1's, ..., then D's
        dts_s.clear();
        for (int s = 0; s <= p->nst; ++s) dts_s += std::string(s ? "/" : "") + dts[(p->tm >> s) & 1];
    }
    std::string dims = std::to_string(p->dims[0]);
    for (int i = 1; i <= p->nst; ++i) dims += "x" + std::to_string(p->dims[i]);
    std::snprintf(buf, len,
                  "path=%s dtype=%s batch=%lld M=%lld dims=%s mfma=%s orient=%s remap=%s mt=%d "
                  "waves=%d rows_per_wg=%d lds_bytes=%d grid=%d workspace_bytes=%lld launches=%d tail=%d "
                  "widths=%s bound=%d",
                  p->unfused ? "unfused" : "fused", dts_s.c_str(), (long long)p->batch,
                  (long long)p->M, dims.c_str(), mfma,
                  p->orn ? "N" : "T", p->unfused ? "none" : modes[p->mode], k->mt, k->waves,
                  k->rows_wg, lds_bytes, p->grid[0],
                  (long long)work, p->unfused ? p->nst : 1, k->tail,
                  (!k->rtw || k->dims[0]) ? "compiled" : "runtime", k->rtw ? k->maxd : 0);
    return B2B_SUCCESS;
}

b2b_status_t b2b_remap_relation(b2b_shape_t shape, int orient_n, int32_t* rel, int64_t cap,
                                int64_t* n_out, int32_t* elems) {
    if ((int)shape < 0 || (int)shape >= b2b::SH_COUNT) return B2B_ERROR_INVALID_VALUE;
    b2b::Relation r;
    if (!b2b::build_relation((b2b::Shape)shape, orient_n != 0, &r)) return B2B_ERROR_NOT_SUPPORTED;
    const int64_t n = (int64_t)r.src_of.size();
    if (n_out) *n_out = n;
    if (elems) *elems = r.elems;
    if (rel) {
        if (cap < n) return B2B_ERROR_INVALID_VALUE;
        for (int64_t i = 0; i < n; ++i) rel[i] = r.src_of[i];
    }
    return B2B_SUCCESS;
}

b2b_status_t b2b_remap_schedule(b2b_shape_t shape, int orient_n, int packed, int32_t* p, int32_t* q,
                                int32_t* r, int64_t cap, int32_t* rounds) {
    if ((int)shape < 0 || (int)shape >= b2b::SH_COUNT) return B2B_ERROR_INVALID_VALUE;
    b2b::Relation rel, use;
    if (!b2b::build_relation((b2b::Shape)shape, orient_n != 0, &rel)) return B2B_ERROR_NOT_SUPPORTED;
    if (packed) {
        if (!b2b::pack_relation(rel, &use)) return B2B_ERROR_NOT_SUPPORTED;
    } else {
        use = rel;
    }
    b2b::Schedule s;
    if (!b2b::build_schedule(use, &s)) return B2B_ERROR_NOT_SUPPORTED;
    if (rounds) *rounds = s.rounds;
    const int64_t n = (int64_t)s.rounds * 64;
    if (p || q || r) {
        if (cap < n) return B2B_ERROR_INVALID_VALUE;
        for (int64_t i = 0; i < n; ++i) {
            if (p) p[i] = s.p[i];
            if (q) q[i] = s.q[i];
            if (r) r[i] = s.r[i];
        }
    }
    return B2B_SUCCESS;
}

b2b_status_t b2b_remap_compile(int32_t elems, const int32_t* src, const int32_t* dst, int32_t* rel, int32_t* p,
                               int32_t* q, int32_t* r, int32_t* rounds) {
    if (elems < 1 || elems > b2bk::kExecMax || !src || !dst) return B2B_ERROR_INVALID_VALUE;
    b2b::Relation relation;
    if (!b2b::build_relation_from_labels(elems, src, dst, &relation)) return B2B_ERROR_INVALID_VALUE;
    b2b::Schedule s;
    if (!b2b::build_schedule(relation, &s) || !b2b::check_schedule(relation, s)) return B2B_ERROR_NOT_SUPPORTED;
    if (rounds) *rounds = s.rounds;
    const int n = 64 * elems;
    for (int i = 0; i < n; ++i) {
        if (rel) rel[i] = relation.src_of[i];
        if (p) p[i] = s.p[i];
        if (q) q[i] = s.q[i];
        if (r) r[i] = s.r[i];
    }
    return B2B_SUCCESS;
}

b2b_status_t b2b_remap_execute(int32_t elems, int32_t rounds, const int32_t* p, const int32_t* q, const int32_t* r,
                               const uint32_t* in, uint32_t* out, hipStream_t stream) {
    if (elems < 1 || elems > b2bk::kExecMax || rounds != elems || !p || !q || !r || !in || !out)
        return B2B_ERROR_INVALID_VALUE;
    b2bk::ExecArgs a;
    std::memset(&a, 0, sizeof a);
    a.elems = elems;
    a.rounds = rounds;
    // receiver tables -> one code per (round, lane); the sender's element comes
    // from the receiver that asks it.  Each round must ask every lane once and
    // each receiver must fill every slot once.
    std::vector<int> filled(64 * elems, 0);
    for (int j = 0; j < rounds; ++j) {
        int give[64];
        bool asked[64] = {};
        for (int i = 0; i < 64; ++i) {
            const int k = j * 64 + i, pi = p[k], qi = q[k], ri = r[k];
            if (pi < 0 || pi > 63 || qi < 0 || qi >= elems || ri < 0 || ri >= elems || asked[pi])
                return B2B_ERROR_INVALID_VALUE;
            asked[pi] = true;
            give[pi] = qi;
            if (filled[i * elems + ri]++) return B2B_ERROR_INVALID_VALUE;
        }
        for (int i = 0; i < 64; ++i) {
            const int k = j * 64 + i;
            a.code[j][i] = (uint16_t)(p[k] | (give[i] << 6) | (r[k] << 10));
        }
    }
    hipLaunchKernelGGL(b2bk::remap_exec_kernel<>, dim3(1), dim3(64), 0, stream, in, out, a);
    return hipGetLastError() == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
}

b2b_status_t b2b_remap_probe(b2b_shape_t shape, int orient_n, uint32_t mode, const void* in, void* out,
                             hipStream_t stream) {
    int dt;
    if (shape == B2B_SHAPE_F16_16X16X32) dt = B2B_DTYPE_F16;
    else if (shape == B2B_SHAPE_BF16_16X16X32) dt = B2B_DTYPE_BF16;
    else if (shape == B2B_SHAPE_F64_16X16X4) dt = B2B_DTYPE_F64;
    else return B2B_ERROR_NOT_SUPPORTED;
    if (!in || !out) return B2B_ERROR_INVALID_VALUE;
    const int m = (int)((mode & B2B_REMAP_MASK) >> 4);
    if ((mode & ~(uint32_t)B2B_REMAP_MASK) || m < b2bk::MODE_BPERM || m > b2bk::MODE_RELABEL)
        return B2B_ERROR_INVALID_VALUE;
    const int orn = orient_n ? 1 : 0;
    if (orn && m != b2bk::MODE_BPERM && m != b2bk::MODE_LDS) return B2B_ERROR_INVALID_VALUE;
    b2bk::KArgs a;
    std::memset(&a, 0, sizeof a);
    if (m == b2bk::MODE_BPERM && !make_sched(dt, orn != 0, a.sched[0])) return B2B_ERROR_NOT_SUPPORTED;
    for (const b2b::ProbeDesc& d : b2b::probe_registry())
        if (d.dtype == dt && d.mode == m && d.orn == orn)
            return d.launch(in, out, a, stream) == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
    return B2B_ERROR_NOT_SUPPORTED;
}

b2b_status_t b2b_mfma_probe(b2b_shape_t shape, const void* a, const void* b, void* c, hipStream_t stream) {
    int dt, s32 = 0;
    if (shape == B2B_SHAPE_F16_16X16X32) dt = B2B_DTYPE_F16;
    else if (shape == B2B_SHAPE_BF16_16X16X32) dt = B2B_DTYPE_BF16;
    else if (shape == B2B_SHAPE_F16_32X32X16) dt = B2B_DTYPE_F16, s32 = 1;
    else if (shape == B2B_SHAPE_BF16_32X32X16) dt = B2B_DTYPE_BF16, s32 = 1;
    else if (shape == B2B_SHAPE_F64_16X16X4) dt = B2B_DTYPE_F64;
    else if (shape == B2B_SHAPE_FP8_32X32X64) {
        if (!a || !b || !c) return B2B_ERROR_INVALID_VALUE;
        hipLaunchKernelGGL(b2bk::mfma_f8_probe_kernel<>, dim3(1), dim3(64), 0, stream, a, b, c);
        return hipGetLastError() == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
    } else return B2B_ERROR_NOT_SUPPORTED;
    if (!a || !b || !c) return B2B_ERROR_INVALID_VALUE;
    for (const b2b::MfmaProbeDesc& d : b2b::mfma_probe_registry())
        if (d.dtype == dt && d.shape32 == s32)
            return d.launch(a, b, c, stream) == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
    return B2B_ERROR_NOT_SUPPORTED;
}

b2b_status_t b2b_fp8_convert_probe(const float* x, void* y, hipStream_t stream) {
    if (!x || !y) return B2B_ERROR_INVALID_VALUE;
    hipLaunchKernelGGL(b2bk::cvt_f8_probe_kernel<>, dim3(1), dim3(64), 0, stream, x, (int*)y);
    return hipGetLastError() == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
}

}  // extern "C"
