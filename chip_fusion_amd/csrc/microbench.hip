// Measurement instruments: the matrix cores alone and an HBM stream alone,
// so that the fused kernels' rates can be read against what the running
// device reaches in practice, not only against its datasheet peaks.
#include <hip/hip_runtime.h>

#include "b2b.h"
#include "b2b_bench.h"
#include "kernels.hpp"

namespace b2bk {

// Independent accumulation chains of the instruction the fused kernels use;
// NACC chains per wave cover the instruction's latency.  The operands are
// small exact values (the sums stay far from overflow for any iters the call
// accepts); the result is written once so the loop stays.
template <int DT>
struct MfmaLoop;
template <>
struct MfmaLoop<DT_F16> {
    static constexpr int NACC = 16;
    static constexpr double FLOP = 2.0 * 16 * 16 * 32;
    __device__ static double run(int64_t iters, unsigned seed) {
        const u4_t a = u4_t{0x2C002C00u ^ (seed & 1), 0x2C002C00u, 0x2C002C00u, 0x2C002C00u};   // 1/16
        f4_t acc[NACC] = {};
        for (int64_t it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < NACC; ++j) acc[j] = Ty<DT_F16>::mma(a, a, acc[j]);
        double s = 0;
#pragma unroll
        for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
        return s;
    }
};
template <>
struct MfmaLoop<DT_BF16> {
    static constexpr int NACC = 16;
    static constexpr double FLOP = 2.0 * 16 * 16 * 32;
    __device__ static double run(int64_t iters, unsigned seed) {
        const u4_t a = u4_t{0x3D803D80u ^ (seed & 1), 0x3D803D80u, 0x3D803D80u, 0x3D803D80u};   // 1/16
        f4_t acc[NACC] = {};
        for (int64_t it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < NACC; ++j) acc[j] = Ty<DT_BF16>::mma(a, a, acc[j]);
        double s = 0;
#pragma unroll
        for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
        return s;
    }
};
template <>
struct MfmaLoop<DT_F64> {
    static constexpr int NACC = 8;
    static constexpr double FLOP = 2.0 * 16 * 16 * 4;
    __device__ static double run(int64_t iters, unsigned seed) {
        const double a = 0.5 + (double)(seed & 1);
        d4_t acc[NACC] = {};
        for (int64_t it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < NACC; ++j) acc[j] = Ty<DT_F64>::mma(a, a, acc[j]);
        double s = 0;
#pragma unroll
        for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
        return s;
    }
};

template <int DT>
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(int64_t iters, unsigned seed, double* sink) {
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = MfmaLoop<DT>::run(iters, seed);
}

// dst = src in 16-byte pieces, four in flight per thread, grid stride;
// stores non-temporal like the fused kernels' D stores
__global__ __launch_bounds__(256) void copy_kernel(const u4_t* __restrict__ src, u4_t* __restrict__ dst,
                                                   int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u4_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = src[i + k * stride];
#pragma unroll
        for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], &dst[i + k * stride]);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(src[i], &dst[i]);
}

// dst[i] = src[i] ^ src[i + n] ^ ... ^ src[i + (R - 1) n]: R read streams of
// n 16-byte pieces for one written stream, two outputs per thread and round
// (2R loads in flight), grid stride, non-temporal stores
template <int R>
__global__ __launch_bounds__(256) void stream_kernel(const u4_t* __restrict__ src, u4_t* __restrict__ dst,
                                                     int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + stride < n16; i += 2 * stride) {
        u4_t v[2][R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            v[0][k] = src[i + k * n16];
            v[1][k] = src[i + stride + k * n16];
        }
        u4_t x = v[0][0], y = v[1][0];
#pragma unroll
        for (int k = 1; k < R; ++k) {
            x ^= v[0][k];
            y ^= v[1][k];
        }
        __builtin_nontemporal_store(x, &dst[i]);
        __builtin_nontemporal_store(y, &dst[i + stride]);
    }
    for (; i < n16; i += stride) {
        u4_t x = src[i];
#pragma unroll
        for (int k = 1; k < R; ++k) x ^= src[i + k * n16];
        __builtin_nontemporal_store(x, &dst[i]);
    }
}

}  // namespace b2bk

extern "C" {

b2b_status_t b2b_bench_mfma(b2b_dtype_t dtype, int32_t workgroups, int64_t iters, void* sink, double* flop,
                            hipStream_t stream) {
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > ((int64_t)1 << 24) || !sink || !flop)
        return B2B_ERROR_INVALID_VALUE;
    double per = 0;
    switch (dtype) {
        case B2B_DTYPE_F16:
            per = b2bk::MfmaLoop<b2bk::DT_F16>::NACC * b2bk::MfmaLoop<b2bk::DT_F16>::FLOP;
            hipLaunchKernelGGL(b2bk::mfma_ceiling_kernel<b2bk::DT_F16>, dim3(workgroups), dim3(256), 0, stream,
                               iters, 0u, (double*)sink);
            break;
        case B2B_DTYPE_BF16:
            per = b2bk::MfmaLoop<b2bk::DT_BF16>::NACC * b2bk::MfmaLoop<b2bk::DT_BF16>::FLOP;
            hipLaunchKernelGGL(b2bk::mfma_ceiling_kernel<b2bk::DT_BF16>, dim3(workgroups), dim3(256), 0, stream,
                               iters, 0u, (double*)sink);
            break;
        case B2B_DTYPE_F64:
            per = b2bk::MfmaLoop<b2bk::DT_F64>::NACC * b2bk::MfmaLoop<b2bk::DT_F64>::FLOP;
            hipLaunchKernelGGL(b2bk::mfma_ceiling_kernel<b2bk::DT_F64>, dim3(workgroups), dim3(256), 0, stream,
                               iters, 0u, (double*)sink);
            break;
        default:
            return B2B_ERROR_NOT_SUPPORTED;
    }
    // four waves a workgroup, one instruction per chain and round
    *flop = (double)workgroups * 4.0 * (double)iters * per;
    return hipGetLastError() == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
}

b2b_status_t b2b_bench_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups, hipStream_t stream) {
    if (!src || !dst || bytes < 64 || bytes % 64 || (uintptr_t)src % 16 || (uintptr_t)dst % 16 ||
        workgroups < 1 || workgroups > 65536)
        return B2B_ERROR_INVALID_VALUE;
    const char *s = (const char*)src, *d = (const char*)dst;
    if (s < d + bytes && d < s + bytes) return B2B_ERROR_INVALID_VALUE;
    hipLaunchKernelGGL(b2bk::copy_kernel, dim3(workgroups), dim3(256), 0, stream, (const b2bk::u4_t*)src,
                       (b2bk::u4_t*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
}

b2b_status_t b2b_bench_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                              int32_t workgroups, hipStream_t stream) {
    if (!src || !dst || write_bytes < 64 || write_bytes % 64 || read_bytes < write_bytes ||
        read_bytes % write_bytes || read_bytes / write_bytes > 4 || (uintptr_t)src % 16 || (uintptr_t)dst % 16 ||
        workgroups < 1 || workgroups > 65536)
        return B2B_ERROR_INVALID_VALUE;
    const char *s = (const char*)src, *d = (const char*)dst;
    if (s < d + write_bytes && d < s + read_bytes) return B2B_ERROR_INVALID_VALUE;
    const int64_t n16 = write_bytes / 16;
    const auto* in = (const b2bk::u4_t*)src;
    auto* out = (b2bk::u4_t*)dst;
    switch (read_bytes / write_bytes) {
        case 1: hipLaunchKernelGGL(b2bk::copy_kernel, dim3(workgroups), dim3(256), 0, stream, in, out, n16); break;
        case 2: hipLaunchKernelGGL(b2bk::stream_kernel<2>, dim3(workgroups), dim3(256), 0, stream, in, out, n16); break;
        case 3: hipLaunchKernelGGL(b2bk::stream_kernel<3>, dim3(workgroups), dim3(256), 0, stream, in, out, n16); break;
        default: hipLaunchKernelGGL(b2bk::stream_kernel<4>, dim3(workgroups), dim3(256), 0, stream, in, out, n16); break;
    }
    return hipGetLastError() == hipSuccess ? B2B_SUCCESS : B2B_ERROR_HIP;
}

}  // extern "C"
