// Table of compiled kernel instances (one per dtype / shape / rearrangement).
#pragma once
#include <hip/hip_runtime.h>

#include <vector>

#include "kernels.hpp"
#include "kernels_cs.hpp"
#include "kernels_gen.hpp"
#include "kernels_gen64.hpp"
#include "kernels_tf32.hpp"
#include "kernels_f8.hpp"

namespace b2b {

struct KernelDesc {
    int dtype, nst, dims[4], mode, orn, km0;
    int mt, waves, threads, rows_wg, lds_bytes;
    int shape32 = 0;  // 1: 32x32x16 instruction
    int rtw = 0;      // 1: widths read at run time, up to maxd (dims are 0), or fixed (dims)
    int maxd = 0;
    int tm = -1;      // type per stage (bit s: bf16 operands of GEMM s, bit nst: D), or -1: all dtype
    int passes = 0;   // tf32: bf16 matrix-instruction passes per product (3 or 4)
    int f8 = 0;       // 1: two GEMMs, the second on the fp8 instruction; 2: one fp8 GEMM (dtd: D's type)
    int dtd = -1;
    int out8 = 0;     // 1: D written as fp8 E4M3 bytes
    int tail = 0;     // 1: any widths, leading dimensions and batch strides (padded on chip)
    const void* fn;   // the __global__ function, for occupancy queries
    // dynamic LDS bytes for the widths d[0..nst] (run-time-width kernels), else 0
    int64_t (*dyn_lds)(const int32_t* d) = nullptr;
    hipError_t (*launch)(const b2bk::KArgs&, int grid, hipStream_t);
};

std::vector<KernelDesc>& registry();

struct Registrar {
    explicit Registrar(const KernelDesc& d) { registry().push_back(d); }
};

template <class C>
KernelDesc describe() {
    KernelDesc d;
    d.dtype = C::DT;
    d.nst = C::NST;
    for (int i = 0; i < 4; ++i) d.dims[i] = i <= C::NST ? C::dim(i) : 0;
    d.mode = C::NST > 1 ? C::MODE : 0;
    d.orn = C::ORN ? 1 : 0;
    d.km0 = C::KM0;
    d.mt = C::MT;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::ROWS_WG;
    d.lds_bytes = C::LDS_BYTES;
    d.fn = (const void*)&b2bk::fused_kernel<C>;
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        hipLaunchKernelGGL(b2bk::fused_kernel<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
        return hipGetLastError();
    };
    return d;
}

// Column-split instances (weights larger than LDS): the rearrangement between
// the GEMMs goes through LDS across the workgroup's waves.
template <class C>
KernelDesc describe_cs() {
    KernelDesc d;
    d.dtype = C::DT;
    d.nst = 2;
    d.dims[0] = C::K;
    d.dims[1] = C::N1;
    d.dims[2] = C::N2;
    d.dims[3] = 0;
    d.mode = b2bk::MODE_LDS;
    d.orn = 0;
    d.km0 = b2bk::KM_NAT;
    d.mt = C::MT;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::R;
    d.lds_bytes = C::LDS_BYTES;
    d.fn = (const void*)&b2bk::cs_kernel<C>;
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        hipLaunchKernelGGL(b2bk::cs_kernel<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
        return hipGetLastError();
    };
    return d;
}

// Instances with run-time widths on the 32x32x16 instruction.
template <class C>
KernelDesc describe_gen() {
    KernelDesc d;
    d.dtype = C::DT;
    d.nst = C::NST;
    for (int& x : d.dims) x = 0;   // never matched by width
    d.mode = C::NST > 1 ? C::MODE : 0;
    d.orn = 0;
    d.km0 = b2bk::KM_NAT;
    d.mt = C::ROWS_WAVE / 16;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::ROWS_WG;
    d.lds_bytes = 0;
    d.shape32 = 1;
    d.rtw = 1;
    d.maxd = C::MAXD;
    d.tm = C::TM;
    d.out8 = C::OUT8 ? 1 : 0;
    d.tail = C::TAIL ? 1 : 0;
    d.fn = (const void*)&b2bk::gen_kernel<C>;
    // LDS for the widths the kernel lays out (padded where it takes tails)
    d.dyn_lds = [](const int32_t* w) -> int64_t {
        int32_t p[b2bk::kMaxStages + 1];
        b2bk::gen_pad(w, C::NST, C::TAIL, p);
        return b2bk::gen_lds_bytes(p, C::NST, C::WAVES);
    };
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        // dynamic LDS up to the whole 160 KB of a CU
        static const hipError_t attr = hipFuncSetAttribute(
            (const void*)&b2bk::gen_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_MAX);
        if (attr != hipSuccess) return attr;
        int32_t p[b2bk::kMaxStages + 1];
        b2bk::gen_pad(a.dims, C::NST, C::TAIL, p);
        const size_t shm = (size_t)b2bk::gen_lds_bytes(p, C::NST, C::WAVES);
        hipLaunchKernelGGL(b2bk::gen_kernel<C>, dim3(grid), dim3(C::THREADS), shm, s, a);
        return hipGetLastError();
    };
    return d;
}

// tf32 instances (bf16 passes on the 32x32x16 instruction), widths read at
// run time or, for the instances that fix them, compiled in (dims: those
// widths, which a plan must match exactly).
template <class C>
KernelDesc describe_tf32() {
    KernelDesc d;
    d.dtype = C::DT;
    d.nst = C::NST;
    for (int i = 0; i < 4; ++i) d.dims[i] = C::FIXED && i <= C::NST ? C::F(i) : 0;
    d.mode = C::NST > 1 ? C::MODE : 0;
    d.orn = 0;
    d.km0 = b2bk::KM_NAT;
    d.mt = C::ROWS_WAVE / 16;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::ROWS_WG;
    d.lds_bytes = 0;
    d.shape32 = 1;
    d.rtw = 1;
    d.maxd = C::MAXD;
    d.passes = C::PASSES;
    d.fn = (const void*)&b2bk::tf32_kernel<C>;
    d.dyn_lds = [](const int32_t* w) -> int64_t { return b2bk::tf32_lds_bytes(w, C::NST); };
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void*)&b2bk::tf32_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_MAX);
        if (attr != hipSuccess) return attr;
        const size_t shm = (size_t)b2bk::tf32_lds_bytes(a.dims, C::NST);
        hipLaunchKernelGGL(b2bk::tf32_kernel<C>, dim3(grid), dim3(C::THREADS), shm, s, a);
        return hipGetLastError();
    };
    return d;
}

// Two-GEMM instances whose second GEMM is fp8, run-time widths.
template <class C>
KernelDesc describe_f8() {
    KernelDesc d;
    d.dtype = C::DT;
    d.nst = 2;
    for (int& x : d.dims) x = 0;   // never matched by width
    d.mode = C::MODE;
    d.orn = 0;
    d.km0 = b2bk::KM_NAT;
    d.mt = C::ROWS_WAVE / 16;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::ROWS_WG;
    d.lds_bytes = 0;
    d.shape32 = 1;
    d.rtw = 1;
    d.maxd = C::MAXD;
    d.f8 = 1;
    d.dtd = C::DTD;
    d.fn = (const void*)&b2bk::f8_kernel<C>;
    d.dyn_lds = [](const int32_t* w) -> int64_t { return b2bk::f8_lds_bytes(w, C::WAVES); };
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void*)&b2bk::f8_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_MAX);
        if (attr != hipSuccess) return attr;
        const size_t shm = (size_t)b2bk::f8_lds_bytes(a.dims, C::WAVES);
        hipLaunchKernelGGL(b2bk::f8_kernel<C>, dim3(grid), dim3(C::THREADS), shm, s, a);
        return hipGetLastError();
    };
    return d;
}

// One fp8 GEMM (the second kernel of an unfused fp8 cascade), run-time widths.
template <class C>
KernelDesc describe_f8a() {
    KernelDesc d;
    d.dtype = -1;
    d.nst = 1;
    for (int& x : d.dims) x = 0;   // never matched by width
    d.mode = 0;
    d.orn = 0;
    d.km0 = b2bk::KM_NAT;
    d.mt = C::ROWS_WAVE / 16;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::ROWS_WG;
    d.lds_bytes = 0;
    d.shape32 = 1;
    d.rtw = 1;
    d.maxd = C::MAXD;
    d.f8 = 2;
    d.dtd = C::DTD;
    d.fn = (const void*)&b2bk::f8a_kernel<C>;
    d.dyn_lds = [](const int32_t* w) -> int64_t { return b2bk::f8a_lds_bytes(w); };
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void*)&b2bk::f8a_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_MAX);
        if (attr != hipSuccess) return attr;
        const size_t shm = (size_t)b2bk::f8a_lds_bytes(a.dims);
        hipLaunchKernelGGL(b2bk::f8a_kernel<C>, dim3(grid), dim3(C::THREADS), shm, s, a);
        return hipGetLastError();
    };
    return d;
}

// fp64 instances with run-time widths.
template <class C>
KernelDesc describe_gen64() {
    KernelDesc d;
    d.dtype = C::DT;
    d.nst = C::NST;
    for (int& x : d.dims) x = 0;   // never matched by width
    d.mode = C::NST > 1 ? C::MODE : 0;
    d.orn = 0;
    d.km0 = b2bk::KM_PAIR64;
    d.mt = 1;
    d.waves = C::WAVES;
    d.threads = C::THREADS;
    d.rows_wg = C::ROWS_WG;
    d.lds_bytes = 0;
    d.rtw = 1;
    d.maxd = C::MAXD;
    d.tail = C::TAIL ? 1 : 0;
    d.fn = (const void*)&b2bk::gen64_kernel<C>;
    d.dyn_lds = [](const int32_t* w) -> int64_t {
        int32_t p[b2bk::kMaxStages + 1];
        b2bk::gen64_pad(w, C::NST, C::TAIL, p);
        return b2bk::gen64_lds_bytes(p, C::NST);
    };
    d.launch = [](const b2bk::KArgs& a, int grid, hipStream_t s) -> hipError_t {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void*)&b2bk::gen64_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_MAX);
        if (attr != hipSuccess) return attr;
        int32_t p[b2bk::kMaxStages + 1];
        b2bk::gen64_pad(a.dims, C::NST, C::TAIL, p);
        const size_t shm = (size_t)b2bk::gen64_lds_bytes(p, C::NST);
        hipLaunchKernelGGL(b2bk::gen64_kernel<C>, dim3(grid), dim3(C::THREADS), shm, s, a);
        return hipGetLastError();
    };
    return d;
}

// Probe instances of the rearrangement executors.
struct ProbeDesc {
    int dtype, mode, orn;
    hipError_t (*launch)(const void*, void*, const b2bk::KArgs&, hipStream_t);
};
std::vector<ProbeDesc>& probe_registry();
struct ProbeRegistrar {
    explicit ProbeRegistrar(const ProbeDesc& d) { probe_registry().push_back(d); }
};
struct MfmaProbeDesc {
    int dtype, shape32;
    hipError_t (*launch)(const void*, const void*, void*, hipStream_t);
};
std::vector<MfmaProbeDesc>& mfma_probe_registry();
struct MfmaProbeRegistrar {
    explicit MfmaProbeRegistrar(const MfmaProbeDesc& d) { mfma_probe_registry().push_back(d); }
};
template <int DT>
MfmaProbeDesc describe_mfma_probe() {
    MfmaProbeDesc d;
    d.dtype = DT;
    d.shape32 = 0;
    d.launch = [](const void* a, const void* b, void* c, hipStream_t s) -> hipError_t {
        hipLaunchKernelGGL(b2bk::mfma_probe_kernel<DT>, dim3(1), dim3(64), 0, s, a, b, c);
        return hipGetLastError();
    };
    return d;
}
template <int DT>
MfmaProbeDesc describe_mfma32_probe() {
    MfmaProbeDesc d;
    d.dtype = DT;
    d.shape32 = 1;
    d.launch = [](const void* a, const void* b, void* c, hipStream_t s) -> hipError_t {
        hipLaunchKernelGGL(b2bk::mfma32_probe_kernel<DT>, dim3(1), dim3(64), 0, s, a, b, c);
        return hipGetLastError();
    };
    return d;
}

template <int DT, int MODE, bool ORN>
ProbeDesc describe_probe() {
    ProbeDesc d;
    d.dtype = DT;
    d.mode = MODE;
    d.orn = ORN ? 1 : 0;
    d.launch = [](const void* in, void* out, const b2bk::KArgs& a, hipStream_t s) -> hipError_t {
        hipLaunchKernelGGL((b2bk::remap_probe_kernel<DT, MODE, ORN>), dim3(1), dim3(64), 0, s, in, out, a);
        return hipGetLastError();
    };
    return d;
}

}  // namespace b2b

#define B2B_CAT2(a, b) a##b
#define B2B_CAT(a, b) B2B_CAT2(a, b)
// B2B_INSTANCE(dtype, stages, K, N1, N2, N3, mode, orientN, MT, waves, kmap0)
#define B2B_CS_INSTANCE(...)                                                           \
    static ::b2b::Registrar B2B_CAT(b2b_cs_reg_, __LINE__)(                            \
        ::b2b::describe_cs<::b2bk::CsCfg<__VA_ARGS__>>())
// B2B_GEN_INSTANCE(dtype, stages, max width, mode, A tiles ahead)
#define B2B_GEN_INSTANCE(...)                                                          \
    static ::b2b::Registrar B2B_CAT(b2b_gen_reg_, __LINE__)(                           \
        ::b2b::describe_gen<::b2bk::GenCfg<__VA_ARGS__>>())
// B2B_GEN_TYPED(stages, max width, A tiles ahead, type mask[, waves]): relabelled, a type per stage
#define B2B_GEN_TYPED(NST, MAXD, PF, ...)                                               \
    B2B_GEN_INSTANCE(((B2B_FIRST(__VA_ARGS__)) & 1) ? ::b2bk::DT_BF16 : ::b2bk::DT_F16, NST, MAXD, \
                     ::b2bk::MODE_RELABEL, PF, __VA_ARGS__)
#define B2B_FIRST(a, ...) a
// B2B_TF32_INSTANCE(stages, max width, passes[, waves[, fixed widths K, N1, ...]])
#define B2B_TF32_INSTANCE(...)                                                         \
    static ::b2b::Registrar B2B_CAT(b2b_tf32_reg_, __LINE__)(                          \
        ::b2b::describe_tf32<::b2bk::Tf32Cfg<__VA_ARGS__>>())
// B2B_F8_INSTANCE(first GEMM's type, D's type, max width, A tiles ahead)
#define B2B_F8_INSTANCE(...)                                                           \
    static ::b2b::Registrar B2B_CAT(b2b_f8_reg_, __LINE__)(                            \
        ::b2b::describe_f8<::b2bk::F8Cfg<__VA_ARGS__>>())
// B2B_F8A_INSTANCE(D's type, max width)
#define B2B_F8A_INSTANCE(...)                                                          \
    static ::b2b::Registrar B2B_CAT(b2b_f8a_reg_, __LINE__)(                           \
        ::b2b::describe_f8a<::b2bk::F8ACfg<__VA_ARGS__>>())
// B2B_GEN64_INSTANCE(stages, max width, A tiles ahead, tiles per group)
#define B2B_GEN64_INSTANCE(...)                                                        \
    static ::b2b::Registrar B2B_CAT(b2b_gen64_reg_, __LINE__)(                         \
        ::b2b::describe_gen64<::b2bk::Gen64Cfg<__VA_ARGS__>>())
#define B2B_INSTANCE(...)                                                              \
    static ::b2b::Registrar B2B_CAT(b2b_reg_, __LINE__)(                               \
        ::b2b::describe<::b2bk::Cfg<__VA_ARGS__>>())
